"""GPU parity of the matrix-core path (calls with T > 8 rows, 8-bit router and
shared expert): the router logits, the shared expert's SwiGLU and its down
projection run as grouped dequant-GEMMs on v_mfma_f32_16x16x32_bf16.

* every row of the layer output agrees with the fp64 oracle (tests/parity.py
  pass criteria), for one and two token tiles (T = 9, 16, 17, 32), ragged
  router tiles (E not a multiple of 16), one group per wave and several;
* the 397B-A17B low-bit shape (H 4096, 512 experts, 3-bit routed experts,
  8-bit shared expert and router; all 15 layers resident) at T = 32: all 32
  rows of layer 0 and of the deepest layer (14) against the oracle, the
  two-layer stack equal to chained layer calls, and bitwise-repeatable
  results;
* the same batch with the matrix cores switched off (MOE_PATH_NO_MFMA) agrees
  with the oracle too.
"""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import gen as ogen  # noqa: E402
from oracle.moe import layer_forward  # noqa: E402
from quantized_moe_decode_softmax_amd import WORKLOADS  # noqa: E402
from quantized_moe_decode_softmax_amd.runtime import DeviceStack, bf16_bits  # noqa: E402
from tests.oracle_pool import oracle_rows  # noqa: E402
from tests.parity import check_layer, oracle_shape  # noqa: E402

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def shp(H, E, I, k, Is, eb):
    return dict(hidden=H, n_experts=E, inter=I, top_k=k, shared_inter=Is, router_bits=8, expert_bits=eb,
                shared_bits=8, rms_eps=1e-6)


CASES = [
    ("h256_e12", shp(256, 12, 128, 3, 192, 4)),      # one router tile of 12 rows, 1 group per wave
    ("h384_e20", shp(384, 20, 192, 5, 64, 2)),       # ragged second router tile, waves 6..7 idle
    ("h1024_e40", shp(1024, 40, 320, 4, 320, 3)),    # 2 groups per wave
    ("h2048_e64", shp(2048, 64, 512, 4, 512, 6)),    # 4 groups per wave
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_mfma_layer_parity(name, kw):
    ds = DeviceStack(kw, n_layers=1, t_max=32, seed=21)
    lw = ogen.GeneratedLayer(oracle_shape(kw), 21, 0)
    for T in (9, 16, 17, 32):
        x = ds.rows(300 + T, T)
        y, ids, w = ds.layer(x)
        y2, ids2, w2 = ds.layer(x)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)) and torch.equal(ids, ids2)
        assert torch.equal(w, w2)
        ref = layer_forward(lw, ogen.bf16_bits_to_f64(bf16_bits(x)))
        r = check_layer(bf16_bits(y), ids.cpu().numpy(), w.cpu().numpy(), ref)
        log(f"  [{name} T={T}] {r}")
        assert r.ok, (name, T, r)
    del ds
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def lowbit():
    w = WORKLOADS["a17b_lowbit"]
    ds = DeviceStack(w.shape_kwargs(), n_layers=w.n_layers, t_max=32)
    ds.check_status = True
    torch.cuda.synchronize()
    yield ds
    del ds
    torch.cuda.empty_cache()


def test_mfma_a17b_lowbit_T32(lowbit):
    ds = lowbit
    osh = oracle_shape(ds.kw)
    x = ds.rows(1000, 32)
    y, ids, wt = ds.layer(x, 0)
    y2, ids2, wt2 = ds.layer(x, 0)
    out, sids, swt, tr = ds.stack(x, trace=True, layer_ids=[0, 1])
    h1, i1, w1 = ds.layer(y, 1)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)) and torch.equal(ids, ids2) and torch.equal(wt, wt2)
    assert torch.equal(tr[1].view(torch.int16), y.view(torch.int16))
    assert torch.equal(out.view(torch.int16), h1.view(torch.int16))
    assert torch.equal(sids[0], ids) and torch.equal(sids[1], i1) and torch.equal(swt[1], w1)
    units = len(np.unique(ids.cpu().numpy()))
    log(f"  [a17b_lowbit T=32] unique experts in layer 0: {units}")
    xh = ogen.bf16_bits_to_f64(bf16_bits(x))
    ref = oracle_rows(osh, 0, [0], xh, chain=False)[0]
    r = check_layer(bf16_bits(y), ids.cpu().numpy(), wt.cpu().numpy(), ref)
    log(f"  [a17b_lowbit T=32] layer 0, all 32 rows vs oracle: {r}")
    assert r.ok, r


def test_mfma_a17b_lowbit_deepest_layer(lowbit):
    ds = lowbit
    osh = oracle_shape(ds.kw)
    x = ds.rows(1014, 32)
    y, ids, wt = ds.layer(x, 14)
    torch.cuda.synchronize()
    ref = oracle_rows(osh, 0, [14], ogen.bf16_bits_to_f64(bf16_bits(x)), chain=False)[0]
    r = check_layer(bf16_bits(y), ids.cpu().numpy(), wt.cpu().numpy(), ref)
    log(f"  [a17b_lowbit T=32] layer 14, all 32 rows vs oracle: {r}")
    assert r.ok, r


def test_lowbit_vector_path_matches_oracle(lowbit):
    """MOE_PATH_NO_MFMA keeps the router and shared expert on the vector units:
    the whole 15-layer stack runs; its layer 0 agrees with the oracle and with
    the matrix-core path's routing."""
    from quantized_moe_decode_softmax_amd import MOE_PATH_NO_MFMA

    ds = lowbit
    osh = oracle_shape(ds.kw)
    x = ds.rows(1000, 32)
    out, ids, wt, tr = ds.stack(x, trace=True, flags=MOE_PATH_NO_MFMA)
    out_m, ids_m, wt_m, tr_m = ds.stack(x, trace=True)
    torch.cuda.synchronize()
    assert ds.status(32) == 0
    ref = oracle_rows(osh, 0, [0], ogen.bf16_bits_to_f64(bf16_bits(x)), chain=False)[0]
    r = check_layer(bf16_bits(tr[1]), ids[0].cpu().numpy(), wt[0].cpu().numpy(), ref)
    log(f"  [a17b_lowbit T=32, vector path] layer 0 vs oracle: {r}")
    assert r.ok, r
    agree = float((ids[0] == ids_m[0]).float().mean())
    log(f"  [a17b_lowbit T=32] layer-0 ids equal on both paths: {agree:.3f} of entries")
