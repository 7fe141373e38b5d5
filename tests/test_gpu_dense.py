"""GPU parity of the dense projections (moe_gemv) and their generator, through the C ABI.

* generator twin: moe_generate_matrix's packed bytes, read back by an
  independent reader of the layout, equal the oracle's dense_matrix codes,
  scales and biases bit for bit, for every code width;
* small shapes over every code width, ragged row counts, 1 to 4 matrices per
  call, 1 to 4 chunks per lane (cols 64 .. 8192) and T = 1, 3, 8, 32: each
  output within 1e-5 * max|y_ref| of the fp64 oracle (fp32 accumulation of
  exact bf16 products over at most 8192 terms);
* a T-row call equals T one-row calls, and a fused call equals separate
  calls, bit for bit;
* the 35B-A3B shapes (fused Q/K/V 4096 + 512 + 512 rows x 2048, attention
  output 2048 x 4096, lm_head 32768 x 2048, 8-bit) at T = 1 and T = 3, checked
  on sampled rows (the oracle run on those rows of the matrices).
"""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import quantized_moe_decode_softmax_amd as moe  # noqa: E402
from oracle import gen as ogen  # noqa: E402
from oracle.dense import gemv  # noqa: E402
from quantized_moe_decode_softmax_amd.runtime import _stream, bf16_bits  # noqa: E402
from tests import layout_ref  # noqa: E402

pytestmark = pytest.mark.gpu
REL = 1e-5


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _matrix(bits, rows, cols, layer, tensor, seed=0):
    buf = torch.empty(moe.moe_matrix_bytes(bits, rows, cols), dtype=torch.uint8, device="cuda")
    moe.moe_generate_matrix(bits, rows, cols, seed, layer, tensor, buf.data_ptr(), _stream())
    return buf


def _x(seed, T, K):
    x = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    moe.moe_generate_rows(seed, T, K, x.data_ptr(), _stream())
    return x


def _run(bits, cols, x, bufs_rows):
    T = x.shape[0]
    ys = [torch.full((T, r), float("nan"), dtype=torch.float32, device="cuda") for _, r in bufs_rows]
    moe.moe_gemv(bits, cols, T, x.data_ptr(), [(b.data_ptr(), r, y.data_ptr()) for (b, r), y in zip(bufs_rows, ys)],
                 _stream())
    return ys


@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8])
def test_generator_twin_dense(bits):
    rows, cols = 37, 320
    buf = _matrix(bits, rows, cols, layer=5, tensor=7)
    torch.cuda.synchronize()
    got = layout_ref.unpack(bits, rows, cols, buf.cpu().numpy())
    c, s, b = ogen.dense_matrix(0, 5, 7, rows, cols, bits)
    assert np.array_equal(got[0], c)
    assert np.array_equal(got[1], ogen.f64_to_bf16_bits(s)) and np.array_equal(got[2], ogen.f64_to_bf16_bits(b))


CASES = [
    (8, 64, (5,)),
    (8, 192, (3, 130)),
    (6, 2048, (129, 7, 64)),
    (4, 4096, (33, 1, 70, 5)),
    (3, 1024, (40,)),
    (2, 8192, (17, 9)),
    (8, 8192, (21,)),
    (8, 4096, (19, 66)),  # two chunks per lane: the decoded-once path at T >= 2
]


@pytest.mark.parametrize("bits,cols,rows", CASES, ids=[f"b{c[0]}_k{c[1]}_n{len(c[2])}" for c in CASES])
def test_gemv_small_parity(bits, cols, rows):
    bufs = [(_matrix(bits, r, cols, layer=1, tensor=6 + i), r) for i, r in enumerate(rows)]
    mats = [ogen.dense_matrix(0, 1, 6 + i, r, cols, bits) for i, r in enumerate(rows)]
    for T in (1, 3, 8, 32):
        x = _x(100 + T, T, cols)
        ys = _run(bits, cols, x, bufs)
        torch.cuda.synchronize()
        refs = gemv(mats, ogen.bf16_bits_to_f64(bf16_bits(x)))
        for m, (y, ref) in enumerate(zip(ys, refs)):
            err = float(np.abs(y.cpu().numpy().astype(np.float64) - ref).max() / np.abs(ref).max())
            log(f"  [bits {bits} cols {cols} T={T} matrix {m} rows {rows[m]}] err/max = {err:.2e}")
            assert err <= REL, (T, m, err)
        if T in (3, 8):  # rows exact; fused equals separate
            for t in range(T):
                y1 = _run(bits, cols, x[t:t + 1].contiguous(), bufs)
                for y, yy in zip(ys, y1):
                    assert torch.equal(y[t:t + 1], yy), (T, t)
            for (b, r), y in zip(bufs, ys):
                (ys1,) = _run(bits, cols, x, [(b, r)])
                assert torch.equal(ys1, y)


def test_gemv_a3b_shapes_sampled():
    H, QD, KD = 2048, 16 * 256, 2 * 256
    specs = [("qkv", 2048, [QD, KD, KD]), ("o_proj", QD, [H]), ("lm_head", H, [32768])]
    rng = np.random.default_rng(0)
    for name, cols, rows in specs:
        bufs = [(_matrix(8, r, cols, layer=3, tensor=6 + i if name == "qkv" else (9 if name == "o_proj" else 10)), r)
                for i, r in enumerate(rows)]
        for T in (1, 3):
            x = _x(7 + T, T, cols)
            ys = _run(8, cols, x, bufs)
            torch.cuda.synchronize()
            xh = ogen.bf16_bits_to_f64(bf16_bits(x))
            for i, ((b, r), y) in enumerate(zip(bufs, ys)):
                tensor = 6 + i if name == "qkv" else (9 if name == "o_proj" else 10)
                c, s, bb = ogen.dense_matrix(0, 3, tensor, r, cols, 8)
                pick = np.unique(np.concatenate([[0, r - 1], rng.integers(0, r, 64)]))
                (ref,) = gemv([(c[pick], s[pick], bb[pick])], xh)
                got = y.cpu().numpy()[:, pick].astype(np.float64)
                err = float(np.abs(got - ref).max() / np.abs(ref).max())
                log(f"  [{name} matrix {i} rows {r} x {cols}, T={T}] {len(pick)} sampled rows: err/max = {err:.2e}")
                assert err <= REL, (name, i, T, err)
                assert torch.isfinite(y).all()
