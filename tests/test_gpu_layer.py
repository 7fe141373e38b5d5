"""GPU parity of single layers and of the generator (run on an MI355X).

Every check calls the HIP path through the C ABI (libmoe.so) and compares with
the fp64 oracle on the same seeded inputs; the oracle never sees a value the
GPU produced except the bytes of the GPU generator, which are checked against
the oracle's own generator (twin test) and are otherwise only read by the GPU.
"""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import gen as ogen  # noqa: E402
from oracle.moe import layer_forward  # noqa: E402
from quantized_moe_decode_softmax_amd import WORKLOADS  # noqa: E402
from quantized_moe_decode_softmax_amd.runtime import DeviceStack, bf16_bits  # noqa: E402
from tests import layout_ref  # noqa: E402
from tests.parity import check_layer, oracle_shape  # noqa: E402

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def small(eb, sb, rb, H=256, E=12, I=128, k=3, Is=192):
    return dict(hidden=H, n_experts=E, inter=I, top_k=k, shared_inter=Is, router_bits=rb, expert_bits=eb,
                shared_bits=sb, rms_eps=1e-6)


SMALL_CASES = [
    small(4, 4, 16),
    small(6, 8, 8),
    small(8, 6, 4),
    small(2, 3, 6),
    small(3, 2, 2),
    small(4, 8, 3, H=384, I=192, Is=64, E=7, k=7),
    small(6, 4, 16, H=1024, I=320, Is=256, E=20, k=5),
]


def _host_bytes(buf: torch.Tensor, off: int, n: int) -> np.ndarray:
    return buf[off:off + n].cpu().numpy()


def _cmp_qmat(got, ref, what):
    c, s, b = got
    rc, rs, rb = ref
    assert np.array_equal(c, rc), f"{what}: codes differ"
    assert np.array_equal(s, ogen.f64_to_bf16_bits(rs)), f"{what}: scales differ"
    assert np.array_equal(b, ogen.f64_to_bf16_bits(rb)), f"{what}: biases differ"


def _check_generator(ds: DeviceStack, layer: int, experts):
    kw, lay = ds.kw, ds.layout
    lw = ogen.GeneratedLayer(oracle_shape(kw), 0, layer)
    buf = ds.layers[layer]
    H, E, I, Is = kw["hidden"], kw["n_experts"], kw["inter"], kw["shared_inter"]
    if kw["router_bits"] == 16:
        got = _host_bytes(buf, lay["router"], E * H * 2).view(np.uint16).reshape(E, H)
        assert np.array_equal(got, ogen.f64_to_bf16_bits(lw.router()[1])), "dense router differs"
    else:
        n = layout_ref.matrix_bytes(kw["router_bits"], E, H)
        _cmp_qmat(layout_ref.unpack(kw["router_bits"], E, H, _host_bytes(buf, lay["router"], n)), lw.router()[1],
                  "router")
    gv = _host_bytes(buf, lay["gatevec"], H * 2).view(np.uint16)
    assert np.array_equal(gv, ogen.f64_to_bf16_bits(lw.gatevec())), "gate vector differs"
    sh = layout_ref.unpack_ffn(_host_bytes(buf, lay["shared"], lay["expert0"] - lay["shared"]), kw["shared_bits"], H,
                               Is)
    for m in ("gate", "up", "down"):
        _cmp_qmat(sh[m], lw.shared()[m], f"shared {m}")
    for e in experts:
        off = lay["expert0"] + e * lay["expert_stride"]
        ex = layout_ref.unpack_ffn(_host_bytes(buf, off, lay["expert_stride"]), kw["expert_bits"], H, I)
        for m in ("gate", "up", "down"):
            _cmp_qmat(ex[m], lw.expert(e)[m], f"expert {e} {m}")


@pytest.mark.parametrize("case", range(len(SMALL_CASES)))
def test_generator_twin_small(case):
    kw = SMALL_CASES[case]
    log(f"[gen twin] case {case} {kw}")
    ds = DeviceStack(kw, n_layers=2)
    torch.cuda.synchronize()
    _check_generator(ds, 1, range(kw["n_experts"]))


def test_generator_twin_tiny_and_rows():
    ds = DeviceStack(WORKLOADS["tiny"].shape_kwargs(), n_layers=1)
    torch.cuda.synchronize()
    _check_generator(ds, 0, range(16))
    for seed in (0, 1000, 2**40 + 3):
        x = ds.rows(seed, 3)
        assert np.array_equal(bf16_bits(x), ogen.f64_to_bf16_bits(ogen.gen_x(seed, 3, 256)))


def _run_layer_check(ds: DeviceStack, layer: int, seeds, T: int):
    osh = oracle_shape(ds.kw)
    lw = ogen.GeneratedLayer(osh, 0, layer)
    worst = 0.0
    for seed in seeds:
        x = ds.rows(seed, T)
        y, ids, w = ds.layer(x, layer)
        torch.cuda.synchronize()
        ref = layer_forward(lw, ogen.bf16_bits_to_f64(bf16_bits(x)))
        r = check_layer(bf16_bits(y), ids.cpu().numpy(), w.cpu().numpy(), ref)
        log(f"  layer {layer} seed {seed} T {T}: {r}")
        assert r.ok, r
        worst = max(worst, r.ratio)
    return worst


def test_tiny_layer_parity():
    log("[parity] tiny T=1")
    ds = DeviceStack(WORKLOADS["tiny"].shape_kwargs(), n_layers=1, t_max=4)
    _run_layer_check(ds, 0, range(1000, 1016), 1)
    _run_layer_check(ds, 0, range(2000, 2004), 4)


@pytest.mark.parametrize("case", range(len(SMALL_CASES)))
def test_small_layer_parity(case):
    kw = SMALL_CASES[case]
    log(f"[parity] case {case} {kw}")
    ds = DeviceStack(kw, n_layers=1, t_max=5)
    _run_layer_check(ds, 0, range(10, 14), 1)
    _run_layer_check(ds, 0, range(20, 22), 5)


@pytest.mark.parametrize("case", [0, 1, 5])
def test_rows_exact_and_deterministic(case):
    kw = SMALL_CASES[case]
    ds = DeviceStack(kw, n_layers=1, t_max=8)
    x = ds.rows(77, 8)
    y8, ids8, w8 = ds.layer(x)
    y8b, ids8b, w8b = ds.layer(x)
    torch.cuda.synchronize()
    assert torch.equal(y8.view(torch.int16), y8b.view(torch.int16))
    assert torch.equal(ids8, ids8b) and torch.equal(w8, w8b)
    for t in range(8):
        y1, ids1, w1 = ds.layer(x[t:t + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16)[0], y8.view(torch.int16)[t]), f"row {t} not exact"
        assert torch.equal(ids1[0], ids8[t]) and torch.equal(w1[0], w8[t])


def test_a3b_layer_parity_full_shape():
    """One 35B-A3B-shaped layer (H 2048, 256 experts, 6-bit) at T = 1 and T = 8."""
    w = WORKLOADS["a3b"]
    log("[parity] a3b layer, generator twin on sampled experts")
    ds = DeviceStack(w.shape_kwargs(), n_layers=1, t_max=8)
    torch.cuda.synchronize()
    _check_generator(ds, 0, [0, 1, 128, 255])
    _run_layer_check(ds, 0, range(1000, 1004), 1)
    _run_layer_check(ds, 0, [5000], 8)
