"""GPU parity of the grouped-query decode attention (moe_gqa_decode), through the C ABI.

* small shapes (head dims 64 / 128 / 256, 1 to 16 query heads per KV head)
  at several positions, among them chunk edges (511, 512, 1023) and the
  first position, T = 1, 3, 8: every output within 2e-5 * max|v| of the fp64
  oracle (bf16 products summed in fp32, fp32 exponentials and sums);
* a T-row call equals the one-row calls at positions p0 + i bit for bit
  (row-exact verify), and repeated calls are bitwise equal;
* cache positions past the last row hold NaN and are never read (the output
  stays finite and equal);
* position 0 alone returns v_0 exactly;
* the card's shape (16 query heads, 2 KV heads, head dim 256) over caches of
  40,000 and 131,072 positions (chunks of 128 and 512 positions; the small
  caches above use 64), T = 1 and 3 near the end, all heads against the
  oracle.
"""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import quantized_moe_decode_softmax_amd as moe  # noqa: E402
from oracle import gen as ogen  # noqa: E402
from oracle.attention import gqa_decode  # noqa: E402
from quantized_moe_decode_softmax_amd.runtime import _stream, bf16_bits  # noqa: E402

pytestmark = pytest.mark.gpu
TOL = 2e-5


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Cache:
    def __init__(self, n_q, n_kv, d, S, seed):
        self.shape = moe.moe_attn_shape_t(n_q, n_kv, d, S)
        self.n_q, self.n_kv, self.d, self.S = n_q, n_kv, d, S
        self.k = torch.empty((n_kv, S, d), dtype=torch.bfloat16, device="cuda")
        self.v = torch.empty((n_kv, S, d), dtype=torch.bfloat16, device="cuda")
        moe.moe_generate_rows(seed, n_kv * S, d, self.k.data_ptr(), _stream())
        moe.moe_generate_rows(seed + 1, n_kv * S, d, self.v.data_ptr(), _stream())
        self.ws_bytes = moe.moe_gqa_workspace_bytes(self.shape, 8)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")

    def q(self, seed, T):
        q = torch.empty((T, self.n_q, self.d), dtype=torch.bfloat16, device="cuda")
        moe.moe_generate_rows(seed, T * self.n_q, self.d, q.data_ptr(), _stream())
        return q

    def run(self, q, p0):
        T = q.shape[0]
        o = torch.full((T, self.n_q, self.d), float("nan"), dtype=torch.float32, device="cuda")
        moe.moe_gqa_decode(self.shape, T, p0, q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), o.data_ptr(),
                           self.ws.data_ptr(), self.ws_bytes, _stream())
        return o

    def host(self, t, n=None):
        x = ogen.bf16_bits_to_f64(bf16_bits(t))
        return x if n is None else x[:, :n]


def _check(c, q, p0, o):
    ref = gqa_decode(c.host(q), c.host(c.k, p0 + q.shape[0]), c.host(c.v, p0 + q.shape[0]), p0)
    scale = float(np.abs(c.host(c.v, p0 + q.shape[0])).max())
    err = float(np.abs(o.cpu().numpy().astype(np.float64) - ref).max() / scale)
    return err


SMALL = [(16, 2, 256, 1300), (8, 8, 64, 1100), (32, 2, 128, 2100), (4, 1, 64, 600), (16, 16, 128, 700)]


@pytest.mark.parametrize("n_q,n_kv,d,S", SMALL, ids=[f"q{a}_kv{b}_d{c}" for a, b, c, _ in SMALL])
def test_attention_small_parity_and_rows(n_q, n_kv, d, S):
    c = Cache(n_q, n_kv, d, S, seed=10 + d)
    for T, p0 in ((1, 0), (1, 511), (1, 512), (3, 509), (8, 1016 % (S - 8)), (3, S - 3), (8, S - 8)):
        q = c.q(500 + p0 + T, T)
        o = c.run(q, p0)
        o2 = c.run(q, p0)
        torch.cuda.synchronize()
        assert torch.equal(o, o2)
        err = _check(c, q, p0, o)
        log(f"  [n_q {n_q} n_kv {n_kv} d {d}] T={T} p0={p0}: err/max|v| = {err:.2e}")
        assert err <= TOL, (T, p0, err)
        if T > 1:
            for i in range(T):
                oi = c.run(q[i:i + 1].contiguous(), p0 + i)
                assert torch.equal(oi[0], o[i]), (T, p0, i)
    del c
    torch.cuda.empty_cache()


def test_attention_unfilled_positions_not_read_and_single_key():
    c = Cache(16, 2, 256, 2000, seed=3)
    q = c.q(77, 3)
    o_ref = c.run(q, 900)
    c.k[:, 903:] = float("nan")
    c.v[:, 903:] = float("nan")
    o = c.run(q, 900)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.equal(o, o_ref)
    # position 0 alone: the output is v_0 (one weight of exactly 1)
    o0 = c.run(q[:1].contiguous(), 0)
    torch.cuda.synchronize()
    v0 = c.v[:, 0].float()
    for h in range(16):
        assert torch.equal(o0[0, h], v0[h // 8])


@pytest.mark.parametrize("S", [40000, 131072], ids=["chunk128", "chunk512"])
def test_attention_card_shape_long_cache(S):
    c = Cache(16, 2, 256, S, seed=5)
    for T, p0 in ((1, S - 2), (3, S - 10)):
        q = c.q(900 + T, T)
        o = c.run(q, p0)
        torch.cuda.synchronize()
        err = _check(c, q, p0, o)
        log(f"  [16 q / 2 kv / d 256, cache {p0 + T} positions] T={T}: err/max|v| = {err:.2e}")
        assert err <= TOL, (T, err)
    del c
    torch.cuda.empty_cache()
