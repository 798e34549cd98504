"""Small helpers shared by the oracle pin tests (no method arithmetic here)."""
import numpy as np

import dsa_synth as S
from oracle import MODE_OFFLOAD, OracleUnit, UnitShape


def unit(max_positions, index_heads=1, index_dim=16, heads=1, top_k=2, hot_slots=4,
         max_query_rows=2, ring_rows=64, mode=MODE_OFFLOAD, softmax_scale=None, replacement=0):
    return OracleUnit(UnitShape(max_positions=max_positions, index_heads=index_heads,
                                index_dim=index_dim, heads=heads, top_k=top_k,
                                hot_slots=hot_slots, max_query_rows=max_query_rows,
                                ring_rows=ring_rows, mode=mode, softmax_scale=softmax_scale,
                                replacement=replacement))


def random_rows(n, seed, row_bytes=656):
    g = np.random.default_rng(seed)
    return g.integers(0, 256, size=(n, row_bytes), dtype=np.uint8)


def zero_queries(R, index_heads, index_dim, heads=1):
    return (np.zeros((R, index_heads, index_dim), np.uint16), np.ones((R, index_heads), np.float32),
            np.zeros((R, heads, 512), np.uint16), np.zeros((R, heads, 64), np.uint16))


def onehot_keys(positions, index_dim):
    k = np.zeros((len(positions), index_dim))
    for i, p in enumerate(positions):
        if p < index_dim:
            k[i, p] = 1.0
    return S.bf16_bits(k)


def select_query(rows_positions, index_dim):
    """Index queries that make row i select exactly rows_positions[i] (one-hot keys)."""
    R = len(rows_positions)
    q = np.zeros((R, 1, index_dim))
    for i, ps in enumerate(rows_positions):
        for p in ps:
            q[i, 0, p] = 2.0
    return S.bf16_bits(q), np.ones((R, 1), np.float32)


def valid_rows(n, seed):
    """n well-formed Q8G64 rows from the workload generator's row recipe."""
    return S.make_rows(np.random.default_rng(seed), n, S.WORKLOADS["tiny"])
