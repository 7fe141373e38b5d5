"""Host-side tests of libmoe.so (no GPU needed: only host entry points are called).

* the library loads and exports every function include/moe_decode.h declares;
* shape/argument validation returns the documented error codes before any
  launch (decode calls with bad arguments never reach the device);
* layout sizes match the closed form, including the flash-moe news page's
  "about 6.75 MB per expert" for the 397B shape at 4 bits ("SSD Expert
  Streaming": 4 active experts of ~6.75 MB each), read as 6.75 MiB;
* the packer agrees with an independent reader of the documented layout.
"""

import numpy as np
import pytest

import quantized_moe_decode_softmax_amd as moe
from quantized_moe_decode_softmax_amd import WORKLOADS
from tests import layout_ref


def shape_of(name, **over):
    kw = WORKLOADS[name].shape_kwargs()
    kw.update(over)
    return moe.make_shape(**kw)


def test_library_exports_every_declared_function():
    L = moe.lib()
    names = moe.header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert moe.moe_version().startswith("moe-decode")


def test_expert_size_closed_form_matches_page():
    # 3 matrices of 4096 x 1024 at 4 bits + a bf16 scale and bias per 64 weights
    kw = dict(hidden=4096, n_experts=512, inter=1024, top_k=10, shared_inter=1024, router_bits=8, expert_bits=4,
              shared_bits=4)
    lay = moe.moe_layer_layout(moe.make_shape(**kw))
    assert lay["expert_stride"] == 3 * 4096 * 1024 * 4 // 8 + 3 * 4096 * 1024 // 64 * 4 == 7077888
    assert lay["expert_stride"] / 2**20 == 6.75


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_layout_matches_independent_reading(name):
    w = WORKLOADS[name]
    lay = moe.moe_layer_layout(moe.make_shape(**w.shape_kwargs()))
    ref = layout_ref.layer_offsets(**w.shape_kwargs())
    assert lay == ref
    for k, v in lay.items():
        assert v % 256 == 0, k


def test_workload_sizes():
    # 35B-A3B shape: 40 layers resident, well under the ~28 GB the model card gives for the whole model
    lay = moe.moe_layer_layout(shape_of("a3b"))
    assert lay["expert_stride"] == 2555904
    total = 40 * lay["total_bytes"]
    assert 26.0e9 < total < 28.0e9
    # 397B shape: 60 layers fit in one 288 GB device
    lay = moe.moe_layer_layout(shape_of("a17b"))
    assert 60 * lay["total_bytes"] < 250e9
    # 3-bit at 10 codes per word: rows of 4096 codes take 410 words
    lay = moe.moe_layer_layout(shape_of("a17b_lowbit"))
    assert lay["expert_stride"] == 2 * (1024 * 1640 + 1024 * 64 * 4) + 4096 * 412 + 4096 * 16 * 4 == 5832704


def test_workspace_bytes():
    s = shape_of("a3b")
    w1 = moe.moe_workspace_bytes(s, 0, 1)
    w8 = moe.moe_workspace_bytes(s, 0, 8)
    assert 0 < w1 < w8 < 64 << 20
    # the descriptor table of an initialised stack: 8 bytes per layer, 256-byte granules
    assert moe.moe_workspace_bytes(s, 40, 1) == w1 + 512
    assert moe.moe_workspace_bytes(s, 1, 1) == w1 + 256
    assert moe.moe_workspace_bytes(s, 4096, 8) == w8 + 4096 * 8
    for nl, T in [(0, 0), (0, 33), (-1, 1), (4097, 1)]:
        with pytest.raises(moe.MoeError) as e:
            moe.moe_workspace_bytes(s, nl, T)
        assert e.value.code == moe.MOE_ERR_INVALID_ARG


def test_validate_and_sizes():
    s = shape_of("a3b")
    for T in (1, 8, 32):
        assert moe.moe_validate(s, T) == 0
    for T in (0, 33):
        with pytest.raises(moe.MoeError) as e:
            moe.moe_validate(s, T)
        assert e.value.code == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as e:
        moe.moe_validate(shape_of("a3b", expert_bits=5), 1)
    assert e.value.code == moe.MOE_ERR_UNSUPPORTED
    lay = moe.moe_layer_layout(s)
    assert moe.moe_expert_bytes(s) == lay["expert_stride"] == 2555904
    assert moe.moe_layer_bytes(s) == lay["total_bytes"]
    # the flash-moe page's ~6.75 MB expert: 4096 x 1024, 4-bit, read as MiB
    a17 = shape_of("a17b")
    assert moe.moe_expert_bytes(a17) == 7077888
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_bytes(shape_of("a3b", group=32))
    assert e.value.code == moe.MOE_ERR_UNSUPPORTED


def test_stack_clear_ranges():
    """The streaming kernel's per-launch clear covers every exchange word, and the
    status word only before a call's first launch (a time-out in an earlier
    launch of the same call stays reported)."""
    for name in WORKLOADS:
        s = shape_of(name)
        for T in (1, 8):
            b0, e0, st_off, total = moe_internal_clear_range(s, T, True)
            b1, e1, st1, _ = moe_internal_clear_range(s, T, False)
            assert (b0, st_off) == (b1, st1)
            assert b0 < st_off < e0 <= total  # first launch: exchange words and status
            assert e1 == st_off               # later launches: everything before the status word
            assert b0 % 256 == 0 and e1 % 256 == 0 and e0 % 256 == 0
            assert total == moe.moe_workspace_bytes(s, 0, T)


def moe_internal_clear_range(s, T, first):
    import ctypes

    L = moe.lib()
    f = L.moe_internal_clear_range
    f.argtypes = [ctypes.POINTER(moe.moe_shape_t), ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)]
    f.restype = ctypes.c_int32
    out = (ctypes.c_int64 * 4)()
    assert f(ctypes.byref(s), T, 1 if first else 0, out) == 0
    return tuple(out)


@pytest.mark.parametrize(
    "field,value,code",
    [
        ("expert_bits", 5, moe.MOE_ERR_UNSUPPORTED),
        ("expert_bits", 7, moe.MOE_ERR_UNSUPPORTED),
        ("shared_bits", 1, moe.MOE_ERR_UNSUPPORTED),
        ("router_bits", 12, moe.MOE_ERR_UNSUPPORTED),
        ("group", 32, moe.MOE_ERR_UNSUPPORTED),
        ("group", 128, moe.MOE_ERR_UNSUPPORTED),
        ("hidden", 100, moe.MOE_ERR_UNSUPPORTED),
        ("hidden", 16384, moe.MOE_ERR_UNSUPPORTED),
        ("inter", 0, moe.MOE_ERR_UNSUPPORTED),
        ("top_k", 0, moe.MOE_ERR_INVALID_ARG),
        ("top_k", 17, moe.MOE_ERR_INVALID_ARG),
        ("n_experts", 0, moe.MOE_ERR_INVALID_ARG),
        ("n_experts", 2000, moe.MOE_ERR_INVALID_ARG),
        ("n_experts", 513, moe.MOE_ERR_INVALID_ARG),
        ("rms_eps", 0.0, moe.MOE_ERR_INVALID_ARG),
    ],
)
def test_shape_validation(field, value, code):
    s = shape_of("tiny", **{field: value})
    with pytest.raises(moe.MoeError) as e:
        moe.moe_validate_shape(s)
    assert e.value.code == code
    assert moe.moe_last_error() != ""


def test_top_k_above_experts_rejected():
    with pytest.raises(moe.MoeError) as e:
        moe.moe_validate_shape(shape_of("tiny", top_k=16, n_experts=8))
    assert e.value.code == moe.MOE_ERR_INVALID_ARG


def test_decode_argument_errors_return_before_launch():
    """Every one of these fails in host validation; no device pointer is touched."""
    s = shape_of("tiny")
    ws = moe.moe_workspace_bytes(s, 0, 2)
    A = 1 << 20  # 256-aligned fake addresses, never dereferenced
    cases = [
        (dict(T=0), moe.MOE_ERR_INVALID_ARG),
        (dict(T=33), moe.MOE_ERR_INVALID_ARG),
        (dict(h_in=0), moe.MOE_ERR_INVALID_ARG),
        (dict(layer=0), moe.MOE_ERR_INVALID_ARG),
        (dict(ws=0), moe.MOE_ERR_INVALID_ARG),
        (dict(layer=A + 8), moe.MOE_ERR_ALIGNMENT),
        (dict(ws=A * 7 + 64), moe.MOE_ERR_ALIGNMENT),
        (dict(h_in=A * 3 + 2), moe.MOE_ERR_ALIGNMENT),
        (dict(ws_bytes=ws - 1), moe.MOE_ERR_WORKSPACE),
        (dict(h_out=A * 2 + 256), moe.MOE_ERR_INVALID_ARG),  # overlaps h_in
    ]
    for over, code in cases:
        a = dict(T=2, layer=A * 16, h_in=A * 2, h_out=A * 4, ws=A * 32, ws_bytes=ws)
        a.update(over)
        with pytest.raises(moe.MoeError) as e:
            moe.moe_decode_layer(s, a["layer"], a["T"], a["h_in"], a["h_out"], None, None, a["ws"], a["ws_bytes"])
        assert e.value.code == code, (over, e.value)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_decode_stack(s, [A * 16, A * 16 + 64], 1, A * 2, A * 4, None, None, None, A * 32, ws)
    assert e.value.code == moe.MOE_ERR_ALIGNMENT
    with pytest.raises(moe.MoeError) as e:
        moe.moe_decode_stack(s, [A * 16, 0], 1, A * 2, A * 4, None, None, None, A * 32, ws)
    assert e.value.code == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as e:
        moe.moe_stack_status(s, 2, 0)
    assert e.value.code == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as e:
        moe.moe_stack_status(s, 33, A * 32)
    assert e.value.code == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as e:
        moe.moe_generate_layer(shape_of("tiny", expert_bits=5), 0, 0, A * 16)
    assert e.value.code == moe.MOE_ERR_UNSUPPORTED
    with pytest.raises(moe.MoeError) as e:
        moe.moe_generate_layer(s, 0, 0, A * 16 + 4)
    assert e.value.code == moe.MOE_ERR_ALIGNMENT


def test_stack_init_argument_errors_return_before_launch():
    """moe_stack_init / moe_stack_decode validate on the host before any launch."""
    s = shape_of("tiny")
    A = 1 << 20
    ws = moe.moe_workspace_bytes(s, 2, 4)
    ok = dict(layers=[A * 16, A * 24], t_max=4, flags=0, ws=A * 32, ws_bytes=ws)
    cases = [
        (dict(layers=[]), moe.MOE_ERR_INVALID_ARG),
        (dict(layers=[A * 16, 0]), moe.MOE_ERR_INVALID_ARG),
        (dict(layers=[A * 16, A * 16 + 128]), moe.MOE_ERR_ALIGNMENT),
        (dict(t_max=0), moe.MOE_ERR_INVALID_ARG),
        (dict(t_max=33), moe.MOE_ERR_INVALID_ARG),
        (dict(flags=4), moe.MOE_ERR_INVALID_ARG),
        (dict(ws=0), moe.MOE_ERR_INVALID_ARG),
        (dict(ws=A * 32 + 16), moe.MOE_ERR_ALIGNMENT),
        (dict(ws_bytes=ws - 1), moe.MOE_ERR_WORKSPACE),  # the table does not fit
    ]
    for over, code in cases:
        a = dict(ok)
        a.update(over)
        with pytest.raises(moe.MoeError) as e:
            moe.moe_stack_init(s, a["layers"], a["t_max"], a["flags"], a["ws"], a["ws_bytes"])
        assert e.value.code == code, (over, e.value)
    # an uninitialised state is refused
    st = moe.moe_stack_t()
    with pytest.raises(moe.MoeError) as e:
        moe.moe_stack_decode(st, 1, A * 2, A * 4, None, None, None)
    assert e.value.code == moe.MOE_ERR_INVALID_ARG


def _gpu_visible() -> bool:
    try:
        import torch

        return torch.cuda.device_count() > 0
    except Exception:  # pragma: no cover
        return False


DEBUG_SYNC_PROBE = r"""
import json, sys
sys.path.insert(0, sys.argv[1])
import quantized_moe_decode_softmax_amd as moe
from quantized_moe_decode_softmax_amd import WORKLOADS
s = moe.make_shape(**WORKLOADS["tiny"].shape_kwargs())
A = 1 << 20
out = {"version": moe.moe_version()}
def code(f):
    try:
        f()
        return 0
    except moe.MoeError as e:
        return e.code
ws = moe.moe_workspace_bytes(s, 1, 2)
out["bad_T"] = code(lambda: moe.moe_decode_layer(s, A * 16, 0, A * 2, A * 4, None, None, A * 32, ws))
out["layer"] = code(lambda: moe.moe_decode_layer(s, A * 16, 2, A * 2, A * 4, None, None, A * 32, ws))
out["stack"] = code(lambda: moe.moe_decode_stack(s, [A * 16], 1, A * 2, A * 4, None, None, None, A * 32, ws))
out["init"] = code(lambda: moe.moe_stack_init(s, [A * 16], 2, 0, A * 32, ws))
out["msg"] = moe.moe_last_error()
print(json.dumps(out))
"""


@pytest.mark.skipif(_gpu_visible(), reason="launches with placeholder pointers; only meaningful with no GPU")
@pytest.mark.parametrize("debug", ["0", "1"])
def test_debug_sync_and_hip_error_mapping_without_device(debug):
    """MOE_DEBUG_SYNC=1 is read once and reported by moe_version; validation still
    comes first, and with no device a launching call maps the HIP failure to
    MOE_ERR_HIP (its launch fails before any synchronisation)."""
    import json
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, MOE_DEBUG_SYNC=debug)
    r = subprocess.run([sys.executable, "-c", DEBUG_SYNC_PROBE, root], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    out = json.loads(r.stdout.strip().splitlines()[-1])
    assert out["version"].endswith("debug-sync") == (debug == "1")
    assert out["bad_T"] == moe.MOE_ERR_INVALID_ARG
    assert out["layer"] == moe.MOE_ERR_HIP
    assert out["stack"] == moe.MOE_ERR_HIP
    assert out["init"] == moe.MOE_ERR_HIP
    assert out["msg"] != ""


@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8])
@pytest.mark.parametrize("rows,cols", [(3, 64), (5, 192), (2, 1024)])
def test_pack_matches_independent_reader(bits, rows, cols):
    rng = np.random.default_rng(bits * 100 + cols)
    codes = rng.integers(0, 2**bits, size=(rows, cols)).astype(np.uint8)
    sc = rng.integers(0, 2**16, size=(rows, cols // 64)).astype(np.uint16)
    bi = rng.integers(0, 2**16, size=(rows, cols // 64)).astype(np.uint16)
    packed = moe.moe_pack_matrix(bits, codes, sc, bi)
    assert packed.size == layout_ref.matrix_bytes(bits, rows, cols)
    c2, s2, b2 = layout_ref.unpack(bits, rows, cols, packed)
    assert np.array_equal(c2, codes) and np.array_equal(s2, sc) and np.array_equal(b2, bi)
    c3, s3, b3 = moe.moe_unpack_matrix(bits, rows, cols, packed)
    assert np.array_equal(c3, codes) and np.array_equal(s3, sc) and np.array_equal(b3, bi)


def test_pack_known_words():
    # 4 bits, LSB first: codes 1..8 in the first dword -> 0x87654321
    codes = np.zeros((1, 64), dtype=np.uint8)
    codes[0, :8] = np.arange(1, 9)
    p = moe.moe_pack_matrix(4, codes, np.zeros((1, 1), np.uint16), np.zeros((1, 1), np.uint16))
    assert p[:4].view(np.uint32)[0] == 0x87654321
    # 3 bits: 10 codes of 7 fill bits 0..14 and 16..30 of the first dword; code 12 (slot 2) -> bit 6 of dword 1
    codes = np.zeros((1, 64), dtype=np.uint8)
    codes[0, :10] = 7
    codes[0, 12] = 5
    p = moe.moe_pack_matrix(3, codes, np.zeros((1, 1), np.uint16), np.zeros((1, 1), np.uint16))
    assert p[:8].view(np.uint32).tolist() == [0x7FFF7FFF, 5 << 6]
    # 6 bits: code 63 at local index 5 -> low nibble at bits 12..15 of dword B, high bits at 14..15 of dword C;
    # at local index 9 (j = 1, upper half) -> bits 16 + 6 .. 16 + 11 of dword A; index 14 (j = 6) -> C bits 16..21
    codes = np.zeros((1, 64), dtype=np.uint8)
    codes[0, 5] = 63
    codes[0, 9] = 0x2A
    codes[0, 14] = 0x15
    p = moe.moe_pack_matrix(6, codes, np.zeros((1, 1), np.uint16), np.zeros((1, 1), np.uint16))
    assert p[:12].view(np.uint32).tolist() == [0x2A << 22, 0xF << 12, (3 << 14) | (0x15 << 16)]
    # scale/bias dword: scale in the low half
    p = moe.moe_pack_matrix(8, np.zeros((1, 64), np.uint8), np.array([[0x3F80]], np.uint16),
                            np.array([[0xBF00]], np.uint16))
    assert p[256:260].view(np.uint32)[0] == 0xBF003F80


def test_pack_rejects_out_of_range_code():
    codes = np.zeros((1, 64), dtype=np.uint8)
    codes[0, 3] = 16
    with pytest.raises(moe.MoeError) as e:
        moe.moe_pack_matrix(4, codes, np.zeros((1, 1), np.uint16), np.zeros((1, 1), np.uint16))
    assert e.value.code == moe.MOE_ERR_INVALID_ARG


def test_gemv_and_matrix_generator_argument_errors():
    """moe_gemv / moe_generate_matrix validate on the host before any launch."""
    A = 1 << 20
    y = A * 64
    for args, code in [((5, 128, 1, A, [(A * 16, 4, y)]), moe.MOE_ERR_UNSUPPORTED),
                       ((8, 100, 1, A, [(A * 16, 4, y)]), moe.MOE_ERR_UNSUPPORTED),
                       ((8, 16384, 1, A, [(A * 16, 4, y)]), moe.MOE_ERR_UNSUPPORTED),
                       ((8, 128, 0, A, [(A * 16, 4, y)]), moe.MOE_ERR_INVALID_ARG),
                       ((8, 128, 33, A, [(A * 16, 4, y)]), moe.MOE_ERR_INVALID_ARG),
                       ((8, 128, 1, A, []), moe.MOE_ERR_INVALID_ARG),
                       ((8, 128, 1, A, [(A * 16, 4, y)] * 5), moe.MOE_ERR_INVALID_ARG),
                       ((8, 128, 1, A, [(A * 16 + 8, 4, y)]), moe.MOE_ERR_ALIGNMENT),
                       ((8, 128, 1, A + 2, [(A * 16, 4, y)]), moe.MOE_ERR_ALIGNMENT),
                       ((8, 128, 1, A, [(A * 16, 4, y + 2)]), moe.MOE_ERR_ALIGNMENT),
                       ((8, 128, 1, A, [(A * 16, 0, y)]), moe.MOE_ERR_INVALID_ARG),
                       ((8, 128, 1, A, [(0, 4, y)]), moe.MOE_ERR_INVALID_ARG),
                       ((8, 128, 2, A, [(A * 16, 4, A + 4)]), moe.MOE_ERR_INVALID_ARG),   # output overlaps x
                       ((8, 128, 1, A, [(A * 16, 8, y), (A * 32, 8, y + 16)]), moe.MOE_ERR_INVALID_ARG)]:
        with pytest.raises(moe.MoeError) as e:
            moe.moe_gemv(*args)
        assert e.value.code == code, (args, e.value)
    for args, code in [((5, 4, 64, 0, 0, 6, A * 16), moe.MOE_ERR_UNSUPPORTED),
                       ((8, 0, 64, 0, 0, 6, A * 16), moe.MOE_ERR_INVALID_ARG),
                       ((8, 4, 100, 0, 0, 6, A * 16), moe.MOE_ERR_INVALID_ARG),
                       ((8, 4, 64, 0, 0, 5, A * 16), moe.MOE_ERR_INVALID_ARG),
                       ((8, 4, 64, 0, -1, 6, A * 16), moe.MOE_ERR_INVALID_ARG),
                       ((8, 4, 64, 0, 0, 6, A * 16 + 4), moe.MOE_ERR_ALIGNMENT)]:
        with pytest.raises(moe.MoeError) as e:
            moe.moe_generate_matrix(*args)
        assert e.value.code == code, (args, e.value)


def test_gqa_argument_errors():
    A = 1 << 20
    ok = moe.moe_attn_shape_t(16, 2, 256, 4096)
    ws = moe.moe_gqa_workspace_bytes(ok, 3)
    # head dim 256: chunks of 64 positions here (4096 / 512 x 2 KV heads < 512
    # chunks for every larger size), one partial (max, sum, pad, acc[d]) each
    assert ws == (4096 // 64) * 3 * 16 * (256 + 4) * 4
    # the card's cache of 131,072 positions: chunks of 512 (256 x 2 KV heads)
    assert moe.moe_gqa_workspace_bytes(moe.moe_attn_shape_t(16, 2, 256, 131072), 1) == 256 * 16 * 260 * 4
    # 40,000 positions: 128 (313 chunks x 2 >= 512; 157 x 2 at 256 is not)
    assert moe.moe_gqa_workspace_bytes(moe.moe_attn_shape_t(16, 2, 256, 40000), 1) == 313 * 16 * 260 * 4
    # head dims 64 and 128 keep 512 (two passes of 256 positions)
    assert moe.moe_gqa_workspace_bytes(moe.moe_attn_shape_t(16, 2, 128, 4096), 2) == 8 * 2 * 16 * 132 * 4
    for sh, code in [(moe.moe_attn_shape_t(16, 2, 96, 4096), moe.MOE_ERR_UNSUPPORTED),
                     (moe.moe_attn_shape_t(15, 2, 256, 4096), moe.MOE_ERR_UNSUPPORTED),
                     (moe.moe_attn_shape_t(32, 2, 256, 4096), moe.MOE_ERR_UNSUPPORTED),  # 16 per KV head at d 256
                     (moe.moe_attn_shape_t(16, 2, 256, 0), moe.MOE_ERR_INVALID_ARG)]:
        with pytest.raises(moe.MoeError) as e:
            moe.moe_gqa_workspace_bytes(sh, 1)
        assert e.value.code == code
    for args, code in [((ok, 0, 0, A, A * 2, A * 4, A * 8, A * 16, ws), moe.MOE_ERR_INVALID_ARG),
                       ((ok, 9, 0, A, A * 2, A * 4, A * 8, A * 16, ws), moe.MOE_ERR_INVALID_ARG),
                       ((ok, 3, 4094, A, A * 2, A * 4, A * 8, A * 16, ws), moe.MOE_ERR_INVALID_ARG),
                       ((ok, 3, -1, A, A * 2, A * 4, A * 8, A * 16, ws), moe.MOE_ERR_INVALID_ARG),
                       ((ok, 3, 0, 0, A * 2, A * 4, A * 8, A * 16, ws), moe.MOE_ERR_INVALID_ARG),
                       ((ok, 3, 0, A + 2, A * 2, A * 4, A * 8, A * 16, ws), moe.MOE_ERR_ALIGNMENT),
                       ((ok, 3, 0, A, A * 2, A * 4, A * 8, A * 16 + 16, ws), moe.MOE_ERR_ALIGNMENT),
                       ((ok, 3, 0, A, A * 2, A * 4, A * 8, A * 16, ws - 1), moe.MOE_ERR_WORKSPACE)]:
        with pytest.raises(moe.MoeError) as e:
            moe.moe_gqa_decode(*args)
        assert e.value.code == code, (args[1:3], e.value)


def test_gdn_argument_errors():
    A = 1 << 20
    ok = moe.moe_gdn_shape_t(16, 32, 128, 128)
    base = (ok, 1, A * 16, A, A * 2, A * 3, A * 4, A * 5, A * 64)
    for over, code in [(dict(shape=moe.moe_gdn_shape_t(16, 32, 96, 128)), moe.MOE_ERR_UNSUPPORTED),
                       (dict(shape=moe.moe_gdn_shape_t(16, 24, 128, 128)), moe.MOE_ERR_INVALID_ARG),
                       (dict(shape=moe.moe_gdn_shape_t(16, 32, 128, 0)), moe.MOE_ERR_INVALID_ARG),
                       (dict(T=0), moe.MOE_ERR_INVALID_ARG), (dict(T=33), moe.MOE_ERR_INVALID_ARG),
                       (dict(state=0), moe.MOE_ERR_INVALID_ARG), (dict(state=A * 16 + 4), moe.MOE_ERR_ALIGNMENT),
                       (dict(o=A * 16 + 1024), moe.MOE_ERR_INVALID_ARG)]:  # o inside the state
        a = list(base)
        for k, v in over.items():
            a[{"shape": 0, "T": 1, "state": 2, "o": 8}[k]] = v
        with pytest.raises(moe.MoeError) as e:
            moe.moe_gdn_step(*a)
        assert e.value.code == code, (over, e.value)
