"""moe_decode_stack_static (the allocation-free variant of moe_decode_stack,
whose workspace is a static device array inside the library) against
moe_decode_stack on a caller-owned workspace, through the C ABI.

Two calls in a row on the same GPU, the second with a smaller input (fewer
rows and layers), each compared bit for bit with moe_decode_stack on the
same inputs: outputs, traces, ids and weights. The first call runs the
per-layer kernels (T = 8), the second the streaming stack kernel (T = 1), so
both kernels' uses of the shared scratch are covered, including the second
call seeing the first call's leftovers. A shape whose workspace does not fit
the static array is refused before any launch.
"""

import sys

import pytest

torch = pytest.importorskip("torch")

import quantized_moe_decode_softmax_amd as moe  # noqa: E402
from quantized_moe_decode_softmax_amd import _lib as L  # noqa: E402
from quantized_moe_decode_softmax_amd.runtime import DeviceStack, _stream  # noqa: E402

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _run(ds, fn, T, n_layers, x):
    out = torch.empty_like(x)
    ids = torch.full((n_layers, T, ds.k), -1, dtype=torch.int32, device=ds.device)
    w = torch.full((n_layers, T, ds.k), -1.0, dtype=torch.float32, device=ds.device)
    tr = torch.empty((n_layers + 1, T, ds.H), dtype=torch.bfloat16, device=ds.device)
    ptrs = [b.data_ptr() for b in ds.layers[:n_layers]]
    if fn == "static":
        L.moe_decode_stack_static(ds.shape, ptrs, T, x.data_ptr(), out.data_ptr(), ids.data_ptr(), w.data_ptr(),
                                  tr.data_ptr(), _stream())
    else:
        L.moe_decode_stack(ds.shape, ptrs, T, x.data_ptr(), out.data_ptr(), ids.data_ptr(), w.data_ptr(),
                           tr.data_ptr(), ds.ws.data_ptr(), ds.ws_bytes, _stream())
    return out, ids, w, tr


def test_static_scratch_matches_workspace_call():
    kw = dict(hidden=2048, n_experts=256, inter=512, top_k=8, shared_inter=512, router_bits=8, expert_bits=6,
              shared_bits=8, rms_eps=1e-6)
    ds = DeviceStack(kw, 6, t_max=8, seed=31)
    for T, n_layers, seed in ((8, 6, 41), (1, 3, 42)):  # the second call is smaller
        x = ds.rows(seed, T)
        got = _run(ds, "static", T, n_layers, x)
        ref = _run(ds, "workspace", T, n_layers, x)
        torch.cuda.synchronize()
        for g, r, what in zip(got, ref, ("out", "ids", "w", "trace")):
            if g.dtype == torch.bfloat16:
                g, r = g.view(torch.int16), r.view(torch.int16)
            assert torch.equal(g, r), (T, n_layers, what)
        log(f"  [static scratch] T={T}, {n_layers} layers: bitwise equal to moe_decode_stack")
    del ds
    torch.cuda.empty_cache()


def test_static_scratch_refuses_oversized_shape():
    # hidden 8192, 512 experts of 8192, top-16 at T = 32: about 28 MiB of workspace
    s = moe.make_shape(hidden=8192, n_experts=512, inter=8192, top_k=16, shared_inter=8192, router_bits=8,
                       expert_bits=4, shared_bits=4)
    assert moe.moe_workspace_bytes(s, 0, 32) > 4 << 20
    A = 1 << 20
    with pytest.raises(moe.MoeError) as e:
        moe.moe_decode_stack_static(s, [A * 16], 32, A * 2, A * 4, None, None, None)
    assert e.value.code == moe.MOE_ERR_WORKSPACE
