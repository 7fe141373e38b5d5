"""GPU parity of the Gated DeltaNet decode step (moe_gdn_step), through the C ABI.

Inputs are seeded numpy draws (unit-norm q and k, alpha in (0.5, 1), beta in
(0, 1), normal v and state), uploaded as fp32; the oracle is oracle/gdn.py in
fp64. Checks:
* every key width (64, 128, 256), 1 to 4 value heads per key head, ragged
  d_v, T = 1, 3, 8, 32: the outputs and the final state within 2e-5 of the
  largest oracle value (fp32 arithmetic over at most 32 steps);
* a T-token call equals T one-token calls in order, bit for bit, and calls
  repeat bitwise;
* the delta rule on the GPU: with beta = 1 the new state maps each unit k to
  its v (to fp32 rounding);
* a 35B-A3B-like shape: 16 key heads and 32 value heads of 128 x 128.
"""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import quantized_moe_decode_softmax_amd as moe  # noqa: E402
from oracle.gdn import gdn_rows  # noqa: E402
from quantized_moe_decode_softmax_amd.runtime import _stream  # noqa: E402

pytestmark = pytest.mark.gpu
TOL = 2e-5


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _inputs(seed, T, n_k, n_v, dk, dv):
    rng = np.random.default_rng(seed)
    unit = lambda *s: (lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True))(rng.normal(size=s))  # noqa: E731
    return dict(state=(0.1 * rng.normal(size=(n_v, dv, dk))).astype(np.float32),
                q=unit(T, n_k, dk).astype(np.float32), k=unit(T, n_k, dk).astype(np.float32),
                v=rng.normal(size=(T, n_v, dv)).astype(np.float32),
                alpha=rng.uniform(0.5, 1.0, (T, n_v)).astype(np.float32),
                beta=rng.uniform(0.0, 1.0, (T, n_v)).astype(np.float32))


def _gpu(shape, inp, T):
    d = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in inp.items()}
    o = torch.full(inp["v"].shape, float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_gdn_step(shape, T, d["state"].data_ptr(), d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(),
                     d["alpha"].data_ptr(), d["beta"].data_ptr(), o.data_ptr(), _stream())
    return d["state"], o


CASES = [(2, 2, 64, 64), (2, 4, 128, 128), (1, 3, 256, 96), (4, 8, 128, 70)]


@pytest.mark.parametrize("n_k,n_v,dk,dv", CASES, ids=[f"k{a}_v{b}_dk{c}_dv{d}" for a, b, c, d in CASES])
def test_gdn_parity_and_steps(n_k, n_v, dk, dv):
    shape = moe.moe_gdn_shape_t(n_k, n_v, dk, dv)
    for T in (1, 3, 8, 32):
        inp = _inputs(T * 100 + dk, T, n_k, n_v, dk, dv)
        st, o = _gpu(shape, inp, T)
        st2, o2 = _gpu(shape, inp, T)
        torch.cuda.synchronize()
        assert torch.equal(st, st2) and torch.equal(o, o2)
        s_ref, o_ref = gdn_rows(inp["state"].astype(np.float64), inp["q"], inp["k"], inp["v"], inp["alpha"],
                                inp["beta"])
        eo = float(np.abs(o.cpu().numpy() - o_ref).max() / np.abs(o_ref).max())
        es = float(np.abs(st.cpu().numpy() - s_ref).max() / np.abs(s_ref).max())
        log(f"  [n_k {n_k} n_v {n_v} d_k {dk} d_v {dv} T={T}] output err/max {eo:.2e}, state err/max {es:.2e}")
        assert eo <= TOL and es <= TOL, (T, eo, es)
        if T in (3, 8):  # T tokens == T one-token calls in order
            cur = inp["state"]
            for t in range(T):
                one = {k: (v[t:t + 1] if k != "state" else cur) for k, v in inp.items()}
                st1, o1 = _gpu(shape, one, 1)
                assert torch.equal(o1[0], o[t]), t
                cur = st1.cpu().numpy()
            assert np.array_equal(cur, st.cpu().numpy())


def test_gdn_delta_rule_stores_v():
    n_k, n_v, dk, dv = 2, 4, 128, 128
    inp = _inputs(9, 1, n_k, n_v, dk, dv)
    inp["beta"][:] = 1.0
    st, _ = _gpu(moe.moe_gdn_shape_t(n_k, n_v, dk, dv), inp, 1)
    torch.cuda.synchronize()
    s = st.cpu().numpy().astype(np.float64)
    for h in range(n_v):
        k = inp["k"][0, h // 2].astype(np.float64)
        assert np.allclose(s[h] @ k, inp["v"][0, h], rtol=0, atol=2e-5 * np.abs(inp["v"]).max())


def test_gdn_a3b_like_shape():
    n_k, n_v, dk, dv = 16, 32, 128, 128
    shape = moe.moe_gdn_shape_t(n_k, n_v, dk, dv)
    for T in (1, 3):
        inp = _inputs(300 + T, T, n_k, n_v, dk, dv)
        st, o = _gpu(shape, inp, T)
        torch.cuda.synchronize()
        s_ref, o_ref = gdn_rows(inp["state"].astype(np.float64), inp["q"], inp["k"], inp["v"], inp["alpha"],
                                inp["beta"])
        eo = float(np.abs(o.cpu().numpy() - o_ref).max() / np.abs(o_ref).max())
        es = float(np.abs(st.cpu().numpy() - s_ref).max() / np.abs(s_ref).max())
        log(f"  [16 key / 32 value heads, 128 x 128, T={T}] output err/max {eo:.2e}, state err/max {es:.2e}")
        assert eo <= TOL and es <= TOL
