"""Dense, contiguous single-query attention in float64 (numpy).

TEST INFRASTRUCTURE ONLY. It is the textbook definition the paged oracle must
reduce to when the block table is the identity over a contiguous pool (the
contiguous layout of prior systems described in "Why OS Virtual Memory Paging
Saved LLM Inference" (a8q9.cn), section 1, against which paging only changes
where rows are stored). It pins the C decode oracle; it is never used to
check the GPU library directly.

    out = softmax(scale * K q) V        K, V: [L, D], q: [D]
"""

import numpy as np


def attention(q, K, V, scale):
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    x = float(scale) * (K @ q)
    w = np.exp(x - x.max())
    return (w @ V) / w.sum()


def bf16_bits_to_f64(bits):
    """Exact widening of raw bf16 bits (uint16) to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)
