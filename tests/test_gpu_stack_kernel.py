"""GPU tests of moe_decode_stack over the compiled variants of its kernels.

One-row stacks run as one streaming kernel per up to 64 layers (one
workgroup per compute unit, cross-workgroup data exchange by polling), with
fixed-shape and generic instantiations; stacks of more rows run layer by
layer, whose variants are chosen by the chunks per lane of the hidden and
intermediate sizes and by the down-projection rows per lane group. One
synthetic shape per variant (with ragged sizes, every code width and the
dense router among them), at T = 1 and T = 2:

* the stack equals chained one-layer calls bit for bit, outputs, ids and
  weights;
* the status word reports that every wait was met;
* layer 0 of the stack agrees with the oracle (same input, pass criteria of
  tests/parity.py);
* a stack longer than 64 layers (two launches of the streaming kernel at
  T = 1) equals its layer calls;
* the initialised stack run with MOE_PATH_PER_LAYER (kernels per layer at
  T = 1) equals the streaming kernel bit for bit.
"""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import gen as ogen  # noqa: E402
from oracle.moe import layer_forward  # noqa: E402
from quantized_moe_decode_softmax_amd.runtime import DeviceStack, bf16_bits  # noqa: E402
from tests.parity import check_layer, oracle_shape  # noqa: E402

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def shp(H, E, I, k, Is, rb, eb, sb):
    return dict(hidden=H, n_experts=E, inter=I, top_k=k, shared_inter=Is, router_bits=rb, expert_bits=eb,
                shared_bits=sb, rms_eps=1e-6)


# (name, shape): the variant each selects on 256 compute units is in the name
# (hidden chunks per lane, intermediate chunks per lane, down rows per lane group)
VARIANTS = [
    ("111", shp(256, 16, 128, 2, 128, 16, 4, 4)),
    ("112", shp(2048, 64, 512, 4, 512, 8, 6, 8)),
    ("114", shp(2048, 32, 1024, 3, 256, 4, 2, 3)),
    ("118_ragged", shp(1536, 48, 2048, 5, 64, 6, 8, 4)),
    ("122", shp(512, 24, 4096, 2, 128, 8, 4, 6)),
    ("211", shp(2560, 20, 128, 4, 64, 3, 4, 2)),
    ("212", shp(4032, 36, 256, 3, 192, 8, 3, 6)),
    ("214", shp(3072, 40, 384, 6, 320, 2, 6, 8)),
    ("218", shp(4096, 40, 1024, 6, 192, 8, 3, 4)),
]


@pytest.mark.parametrize("name,kw", VARIANTS, ids=[v[0] for v in VARIANTS])
@pytest.mark.parametrize("T", [1, 2])
def test_stack_kernel_variant(name, kw, T):
    n_layers = 3
    ds = DeviceStack(kw, n_layers, t_max=32, seed=11)
    ds.check_status = True
    x = ds.rows(500 + T, T)
    out, ids, w, tr = ds.stack(x, trace=True)
    h = x
    for l in range(n_layers):
        h, il, wl = ds.layer(h, l)
        assert torch.equal(il, ids[l]) and torch.equal(wl, w[l]), (name, T, l)
        assert torch.equal(h.view(torch.int16), tr[l + 1].view(torch.int16)), (name, T, l)
    assert torch.equal(out.view(torch.int16), h.view(torch.int16))
    assert ds.status(T) == 0
    ref = layer_forward(ogen.GeneratedLayer(oracle_shape(kw), 11, 0), ogen.bf16_bits_to_f64(bf16_bits(x)))
    r = check_layer(bf16_bits(tr[1]), ids[0].cpu().numpy(), w[0].cpu().numpy(), ref)
    log(f"  [{name} T={T}] layer 0 vs oracle: {r}")
    assert r.ok, r
    del ds
    torch.cuda.empty_cache()


def test_stack_kernel_full_rows_T32():
    """T = 32 (the largest row count): every row's routing and output match the layer calls."""
    kw = shp(2048, 64, 512, 4, 512, 8, 6, 8)
    ds = DeviceStack(kw, 2, t_max=32, seed=5)
    ds.check_status = True
    x = ds.rows(77, 32)
    out, ids, w, _ = ds.stack(x)
    h1, i1, w1 = ds.layer(x, 0)
    h2, i2, w2 = ds.layer(h1, 1)
    assert torch.equal(out.view(torch.int16), h2.view(torch.int16))
    assert torch.equal(ids[0], i1) and torch.equal(ids[1], i2) and torch.equal(w[0], w1) and torch.equal(w[1], w2)
    del ds
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [1, 2])
def test_stack_longer_than_one_launch(T):
    """70 layers: at T = 1 two launches of the streaming kernel (64 + 6) whose
    boundary hands h over in the workspace (with the trace, ids and weights
    offset by the first launch's layers), at T = 2 kernels per layer; both equal
    70 chained one-layer calls bit for bit, and every wait was met."""
    kw = shp(256, 16, 128, 2, 128, 16, 4, 4)
    n = 70
    ds = DeviceStack(kw, n, t_max=2, seed=3)
    ds.check_status = True
    x = ds.rows(9, T)
    out, ids, w, tr = ds.stack(x, trace=True)
    out_nt, ids_nt, w_nt, _ = ds.stack(x)  # no trace: the second launch's output goes to h_out directly
    assert torch.equal(out.view(torch.int16), out_nt.view(torch.int16))
    assert torch.equal(ids, ids_nt) and torch.equal(w, w_nt)
    assert ds.status(T) == 0
    h = x
    for l in range(n):
        h, il, wl = ds.layer(h, l)
        assert torch.equal(il, ids[l]) and torch.equal(wl, w[l]), l
        assert torch.equal(h.view(torch.int16), tr[l + 1].view(torch.int16)), l
    assert torch.equal(out.view(torch.int16), h.view(torch.int16))
    ids_h = ids.cpu().numpy()
    assert np.all((ids_h >= 0) & (ids_h < 16))
    del ds
    torch.cuda.empty_cache()


def test_per_layer_flag_equals_streaming_kernel():
    """The same one-row stack through the persistent streaming kernel and, with
    MOE_PATH_PER_LAYER, through the per-layer kernels: bitwise equal."""
    from quantized_moe_decode_softmax_amd import MOE_PATH_PER_LAYER

    kw = shp(2048, 256, 512, 8, 512, 8, 6, 8)
    ds = DeviceStack(kw, 4, t_max=1, seed=13)
    ds.check_status = True
    for s in range(3):
        x = ds.rows(700 + s, 1)
        out, ids, w, tr = ds.stack(x, trace=True)
        out2, ids2, w2, tr2 = ds.stack(x, trace=True, flags=MOE_PATH_PER_LAYER)
        torch.cuda.synchronize()
        assert torch.equal(tr.view(torch.int16), tr2.view(torch.int16)), s
        assert torch.equal(ids, ids2) and torch.equal(w, w2), s
    del ds
    torch.cuda.empty_cache()
