"""GPU invariants of the decode path (run on an MI355X), through the C ABI.

* determinism: 100 repeated stack calls give bitwise-identical outputs,
  ids and weights (one-row streaming kernel and multi-row per-layer path);
* no shortcut: changing the weights of an expert a row selected changes that
  row's output, changing an expert no row selected changes nothing (bit for
  bit), on the one-row stack path and on the per-layer path;
* identical experts: when every routed expert holds the same weights, the
  output does not depend on which experts the router picks (the weights of
  the k selected sum to one), up to fp32 rounding.
"""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from quantized_moe_decode_softmax_amd import WORKLOADS  # noqa: E402
from quantized_moe_decode_softmax_amd.runtime import DeviceStack  # noqa: E402

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def shp(H, E, I, k, Is, rb, eb, sb):
    return dict(hidden=H, n_experts=E, inter=I, top_k=k, shared_inter=Is, router_bits=rb, expert_bits=eb,
                shared_bits=sb, rms_eps=1e-6)


def test_determinism_100_calls():
    w = WORKLOADS["a3b"]
    ds = DeviceStack.from_workload(w, n_layers=8, t_max=4)
    ds.check_status = True
    for T in (1, 4):
        x = ds.rows(60 + T, T)
        out0, ids0, w0, _ = ds.stack(x)
        for _ in range(99):
            out, ids, wt, _ = ds.stack(x)
            assert torch.equal(out.view(torch.int16), out0.view(torch.int16))
            assert torch.equal(ids, ids0) and torch.equal(wt, w0)
        torch.cuda.synchronize()
        log(f"  [determinism] 8-layer 35B-A3B stack, T={T}: 100 calls bitwise equal")
    del ds
    torch.cuda.empty_cache()


def _expert_block(ds, e):
    lay = ds.layout
    o = lay["expert0"] + e * lay["expert_stride"]
    return ds.layers[0][o:o + lay["expert_stride"]]


@pytest.mark.parametrize("T", [1, 3])
def test_no_shortcut(T):
    kw = shp(512, 24, 256, 4, 128, 8, 4, 8)
    ds = DeviceStack(kw, n_layers=1, t_max=4, seed=71)
    x = ds.rows(90, T)
    y0, ids0, _, _ = ds.stack(x)
    torch.cuda.synchronize()
    used = set(ids0.cpu().numpy().ravel().tolist())
    unused = [e for e in range(kw["n_experts"]) if e not in used]
    # an expert no row selected: scramble its whole block
    blk = _expert_block(ds, unused[0])
    saved = blk.clone()
    blk.copy_(torch.flip(saved, [0]))
    y1, ids1, _, _ = ds.stack(x)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y0.view(torch.int16)) and torch.equal(ids1, ids0)
    blk.copy_(saved)
    # the expert row 0 selected last (smallest weight): flip the low bit of
    # every code byte of its down projection (the scale and bias are kept)
    e = int(ids0[0, 0, -1])  # layer 0, row 0, last (smallest weight)
    blk = _expert_block(ds, e)
    saved = blk.clone()
    down = ds.layout["expert_down"]
    codes = kw["hidden"] * kw["inter"] * kw["expert_bits"] // 8
    blk[down:down + codes] ^= 1
    y2, ids2, _, _ = ds.stack(x)
    torch.cuda.synchronize()
    assert torch.equal(ids2, ids0)
    assert not torch.equal(y2[0].view(torch.int16), y0[0].view(torch.int16)), "row 0 ignored its expert"
    blk.copy_(saved)
    log(f"  [no shortcut, T={T}] unused expert {unused[0]}: no change; selected expert {e}: row 0 changed")
    del ds
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [1, 5])
def test_identical_experts_make_routing_irrelevant(T):
    kw = shp(256, 12, 128, 3, 64, 16, 4, 4)
    ds = DeviceStack(kw, n_layers=1, t_max=8, seed=81)
    b0 = _expert_block(ds, 0).clone()
    for e in range(1, kw["n_experts"]):
        _expert_block(ds, e).copy_(b0)
    x = ds.rows(95, T)
    y0, ids0, _ = ds.layer(x)
    # reverse the router rows: other experts win, the output must not move
    lay, H, E = ds.layout, kw["hidden"], kw["n_experts"]
    r = ds.layers[0][lay["router"]:lay["router"] + E * H * 2].view(E, H * 2)
    r.copy_(torch.flip(r.clone(), [0]))
    y1, ids1, _ = ds.layer(x)
    torch.cuda.synchronize()
    assert not torch.equal(ids1, ids0)
    a, b = y0.float().cpu().numpy(), y1.float().cpu().numpy()
    rel = float(np.abs(a - b).max() / np.abs(a).max())
    log(f"  [identical experts, T={T}] ids {ids0[0].tolist()} -> {ids1[0].tolist()}, max rel diff {rel:.2e}")
    assert rel <= 8e-3, rel  # two bf16 roundings of the same value at most one unit apart
    del ds
    torch.cuda.empty_cache()
