"""GPU edge cases of the decode path (run on an MI355X), through the C ABI.

* every router logit equal (router rows made identical on the device): the
  top-k is experts 0..k-1 in that order (ties go to the lower id) with
  weights exactly 1/k, on the vector path (T = 1, 5), the matrix-core path
  (T = 16) and the dense bf16 router;
* one expert with top-1: its weight is exactly 1 and the layer agrees with the
  oracle;
* the largest supported sizes (hidden 8192, 512 experts, top-16): the layer
  agrees with the oracle at T = 1, and at T = 32 on sampled rows (each against
  the oracle run on that row alone); a two-layer stack equals chained layer
  calls.
"""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import gen as ogen  # noqa: E402
from oracle.moe import layer_forward  # noqa: E402
from quantized_moe_decode_softmax_amd.runtime import DeviceStack, bf16_bits  # noqa: E402
from tests import layout_ref  # noqa: E402
from tests.parity import check_layer, oracle_shape  # noqa: E402

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def shp(H, E, I, k, Is, rb, eb, sb):
    return dict(hidden=H, n_experts=E, inter=I, top_k=k, shared_inter=Is, router_bits=rb, expert_bits=eb,
                shared_bits=sb, rms_eps=1e-6)


def _tie_router(ds: DeviceStack):
    """Copies router row 0 (codes and scale/bias words) over every other row."""
    kw, lay, buf = ds.kw, ds.layout, ds.layers[0]
    H, E, rb = kw["hidden"], kw["n_experts"], kw["router_bits"]
    r0 = lay["router"]
    if rb == 16:
        rows = buf[r0:r0 + E * H * 2].view(E, H * 2)
        rows[1:] = rows[0]
        return
    nb = layout_ref.row_bytes(rb, H)
    codes = buf[r0:r0 + E * nb].view(E, nb)
    codes[1:] = codes[0]
    s0 = r0 + layout_ref.codes_bytes(rb, E, H)
    sbw = (H // 64) * 4
    sb = buf[s0:s0 + E * sbw].view(E, sbw)
    sb[1:] = sb[0]


@pytest.mark.parametrize("rb", [8, 16])
def test_all_logits_tied(rb):
    kw = shp(256, 12, 128, 3, 192, rb, 6, 8)
    ds = DeviceStack(kw, n_layers=1, t_max=32, seed=31)
    _tie_router(ds)
    k = kw["top_k"]
    for T in (1, 5, 16):
        x = ds.rows(700 + T, T)
        y, ids, w = ds.layer(x)
        out, sids, sw, _ = ds.stack(x)
        torch.cuda.synchronize()
        ih, wh = ids.cpu().numpy(), w.cpu().numpy()
        assert np.array_equal(ih, np.tile(np.arange(k, dtype=np.int32), (T, 1))), (rb, T, ih[:2])
        assert np.all(wh == np.float32(1.0) / np.float32(k)), (rb, T, wh[:2])
        assert torch.equal(out.view(torch.int16), y.view(torch.int16)) and torch.equal(sids[0], ids)
        log(f"  [tied logits, router bits {rb}, T={T}] ids {ih[0].tolist()} weights {wh[0].tolist()}")
    del ds
    torch.cuda.empty_cache()


def test_single_expert_top1():
    kw = shp(256, 1, 128, 1, 128, 8, 4, 8)
    ds = DeviceStack(kw, n_layers=1, t_max=32, seed=41)
    lw = ogen.GeneratedLayer(oracle_shape(kw), 41, 0)
    for T in (1, 3, 12):
        x = ds.rows(800 + T, T)
        y, ids, w = ds.layer(x)
        torch.cuda.synchronize()
        assert np.all(ids.cpu().numpy() == 0) and np.all(w.cpu().numpy() == 1.0)
        ref = layer_forward(lw, ogen.bf16_bits_to_f64(bf16_bits(x)))
        r = check_layer(bf16_bits(y), ids.cpu().numpy(), w.cpu().numpy(), ref)
        log(f"  [one expert, T={T}] {r}")
        assert r.ok, (T, r)
    del ds
    torch.cuda.empty_cache()


def test_largest_sizes():
    kw = shp(8192, 512, 128, 16, 64, 8, 4, 8)
    ds = DeviceStack(kw, n_layers=2, t_max=32, seed=51)
    ds.check_status = True
    osh = oracle_shape(kw)
    lw = ogen.GeneratedLayer(osh, 51, 0)
    x1 = ds.rows(900, 1)
    y1, i1, w1 = ds.layer(x1)
    torch.cuda.synchronize()
    r = check_layer(bf16_bits(y1), i1.cpu().numpy(), w1.cpu().numpy(),
                    layer_forward(lw, ogen.bf16_bits_to_f64(bf16_bits(x1))))
    log(f"  [H 8192, E 512, top-16, T=1] {r}")
    assert r.ok, r
    x = ds.rows(901, 32)
    y, ids, w = ds.layer(x)
    torch.cuda.synchronize()
    yb, ih, wh = bf16_bits(y), ids.cpu().numpy(), w.cpu().numpy()
    xh = ogen.bf16_bits_to_f64(bf16_bits(x))
    for t in (0, 29):
        r = check_layer(yb[t:t + 1], ih[t:t + 1], wh[t:t + 1], layer_forward(lw, xh[t:t + 1]))
        log(f"  [H 8192, E 512, top-16, T=32] row {t} vs oracle on that row: {r}")
        assert r.ok, (t, r)
    for T, xs in ((1, x1), (32, x)):
        out, sids, sw, _ = ds.stack(xs)
        h1, a1, b1 = ds.layer(xs, 0)
        h2, a2, b2 = ds.layer(h1, 1)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), h2.view(torch.int16)), T
        assert torch.equal(sids[0], a1) and torch.equal(sids[1], a2) and torch.equal(sw[1], b2), T
    del ds
    torch.cuda.empty_cache()
