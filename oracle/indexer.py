"""Indexer scores upstream of top-K — TEST INFRASTRUCTURE (see the package
header: only tests, the smoke check and the CPU baseline use this module).

What the pages fix. The indexer picks the top-K tokens of each decode step
and only those enter attention ([P3] "vLLM Hybrid HiSparse：稀疏MLA破解长上下文
显存瓶颈" §"稀疏MLA的核心思想"; [P2] "vLLM GLM 5.3 优化：混合 HiSparse 卸载"
§"解决 KV 缓存内存压力"), and it keeps a per-token key cache of its own, the
indexer KV, which the standard offloading connector moves in whole blocks,
apart from the latent rows ([P2] §"与 vLLM 栈的集成", indexer KV item).

What they leave open, and the reading taken. The pages give no formula for
a token's score. The reading here is the lightning-indexer form of the
sparse attention that these sparse-MLA models descend from: H indexer heads
of dimension 128; per request and step a query q (H x 128) and head weights
w (H); per token t an indexer key k_t (128);

    score_t = sum_j w_j * max(0, <q_j, k_t>).

Queries and keys are bf16 values, weights fp32; here everything is exact
fp64 (bf16 and fp32 values widen exactly).
"""
from __future__ import annotations

import numpy as np

INDEXER_DIM = 128


def indexer_scores(q: np.ndarray, w: np.ndarray, keys: np.ndarray, L: int) -> np.ndarray:
    """Scores of tokens 0..L-1 for one request.

    q [H, 128] and w [H] as float64 values, keys [>= L, 128] float64 values.
    Returns float64 [L]: for every token, the weighted sum over heads of the
    positive part of the head's dot product with the token's key.
    """
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    k = np.asarray(keys[:L], dtype=np.float64)
    dots = k @ q.T                      # [L, H]: <q_j, k_t>
    return np.maximum(dots, 0.0) @ w    # sum_j w_j * max(0, .)
