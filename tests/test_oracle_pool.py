"""The process-pool oracle runner gives exactly the oracle's stack_forward results."""

import numpy as np

from oracle import gen as ogen
from oracle.moe import layer_forward, stack_forward
from tests.oracle_pool import oracle_rows
from tests.parity import oracle_shape

KW = dict(hidden=256, n_experts=16, inter=128, top_k=3, shared_inter=128, router_bits=8, expert_bits=4,
          shared_bits=6, rms_eps=1e-6)


def test_pool_chain_equals_stack_forward():
    osh = oracle_shape(KW)
    x = ogen.gen_x(3, 4, 256)
    a = oracle_rows(osh, 0, [0, 1, 2], x)
    b = stack_forward([ogen.GeneratedLayer(osh, 0, l) for l in range(3)], x)
    for l in range(3):
        for k in ("y", "ids", "w", "gap", "logits", "sgate", "h"):
            assert np.array_equal(np.asarray(a[l][k]), np.asarray(b[l][k])), (l, k)


def test_pool_unchained_equals_layer_forward():
    osh = oracle_shape(KW)
    x = ogen.gen_x(4, 3, 256)
    a = oracle_rows(osh, 0, [2, 5], x, chain=False)
    for i, l in enumerate([2, 5]):
        r = layer_forward(ogen.GeneratedLayer(osh, 0, l), ogen.bf16_round(x))
        for k in ("y", "ids", "w", "gap"):
            assert np.array_equal(np.asarray(a[i][k]), np.asarray(r[k])), (l, k)
