"""Read side: decode attention over the paged cache (oracle; test infra).

[KV essay] "First, what K and V are": attention is softmax(Q K^T / sqrt(d)) V;
for decoding, the one new query row of each head is scored against every
cached key of its sequence and the softmax weights mix the cached values.
[KV essay] "Paged attention": the kernel reads a sequence's blocks through its
block table, so where the blocks sit does not change the result.
[KV essay] "What the cache costs" and [KV management]: with grouped-query
attention, groups of query heads share one KV head.

Readings taken:

* query head h reads KV head h // G, G = H_q / H_kv (consecutive groups);
* the query of sequence b attends to exactly its ``lens[b]`` cached tokens,
  positions 0 .. lens[b]-1, with no further mask; the query arrives already
  rotated to its own position;
* scale = 1/sqrt(d); everything is evaluated in float64 from the exactly
  widened stored values;
* an fp8 cache holds codes whose values are e4m3(code) times the float32
  scale of their (layer, KV head), or of their (layer, block, KV head) when
  the scales are given per block; the query then comes in a 16-bit format;
* with a sliding window W ([KV essay] "Capping the window": attention
  covers a trailing span of W positions), the query of a sequence of length n
  attends to positions max(0, n - W) .. n-1 only;
* besides ``out`` the log-sum-exp ``lse = m + ln(sum exp(s - m))`` of the
  scaled scores is returned; a sequence of length 0 gives out = 0 and
  lse = -inf;
* (a reading about malformed input, not from the pages) a block-table entry
  outside [0, num_blocks) inside a sequence's length names no block: its
  positions are left out of the softmax, as if absent, and a sequence left
  with no position gives out = 0 and lse = -inf.

The split-K merge (partial softmax states over disjoint token ranges combined
by their log-sum-exp) is stated in ``lse_merge``; the tests check it equals
the direct formula, which is what the oracle reports.
"""

import math

import numpy as np

from .layout import (BLOCK_TOKENS, PoolSpec, block_in_range, gather_sequence,
                     gather_sequence_planes)
from .numerics import to_f64


def softmax_attend(q64: np.ndarray, k64: np.ndarray, v64: np.ndarray, scale: float):
    """One query row against n keys/values (float64): returns (out[d], lse)."""
    n = k64.shape[0]
    if n == 0:
        return np.zeros(v64.shape[-1] if v64.ndim == 2 else q64.shape[-1]), -math.inf
    s = (k64 @ q64) * scale
    m = s.max()
    w = np.exp(s - m)
    l = w.sum()
    return (w @ v64) / l, m + math.log(l)


def decode_contiguous(q, k_seqs, v_seqs, dtype: str, n_q_heads: int, scale=None):
    """Attention with each sequence's K, V given as dense [len][H_kv][d] arrays.

    q: raw [B][H_q][d] in ``dtype``.  Returns out [B][H_q][d], lse [B][H_q].
    """
    q64 = to_f64(q, dtype)
    b_n, hq, d = q64.shape
    assert hq == n_q_heads
    out = np.zeros((b_n, hq, d))
    lse = np.full((b_n, hq), -math.inf)
    for b in range(b_n):
        k64 = to_f64(k_seqs[b], dtype)
        v64 = to_f64(v_seqs[b], dtype)
        h_kv = k64.shape[1] if k64.ndim == 3 else 1
        g = hq // h_kv
        sc = 1.0 / math.sqrt(d) if scale is None else scale
        for h in range(hq):
            if k64.shape[0] == 0:
                continue
            out[b, h], lse[b, h] = softmax_attend(q64[b, h], k64[:, h // g, :],
                                                  v64[:, h // g, :], sc)
    return out, lse


def decode_paged(q, k_pool, v_pool, spec: PoolSpec, layer: int, tables, lens,
                 n_q_heads: int, scale=None, seqs=None, heads=None, by_plane=False,
                 q_dtype=None, k_scale=None, v_scale=None, window=None, num_blocks=None):
    """Decode attention reading K/V through the block tables.

    ``seqs`` / ``heads`` restrict which (sequence, query head) outputs are
    computed (sampling at large sizes); the rest stay 0 / -inf.  ``by_plane``
    gathers a whole plane at a time (same values, faster).  ``window`` (a
    positive int) limits each query to the last ``window`` positions.
    ``num_blocks``, when given, makes positions whose table entry is outside
    [0, num_blocks) drop out of the attention (the tables may then hold such
    entries; without it every entry inside a length must name a block).
    """
    q64 = to_f64(q, spec.dtype if q_dtype is None else q_dtype)
    b_n, hq, d = q64.shape
    g = hq // spec.n_kv_heads
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    seqs = range(b_n) if seqs is None else seqs
    out = np.zeros((b_n, hq, d))
    lse = np.full((b_n, hq), -math.inf)
    for b in seqs:
        qh = range(hq) if heads is None else heads
        kv_heads = sorted({h // g for h in qh})
        gather = gather_sequence_planes if by_plane else gather_sequence
        start = max(0, int(lens[b]) - int(window)) if window else 0
        kept = list(range(start, int(lens[b])))
        if num_blocks is None:
            k_raw, v_raw = gather(k_pool, v_pool, spec, layer, tables[b], int(lens[b]),
                                  heads=kv_heads, start=start)
        else:
            kept = [p for p in kept if block_in_range(tables[b], p, num_blocks)]
            k_raw, v_raw = gather_sequence(k_pool, v_pool, spec, layer, tables[b], int(lens[b]),
                                           heads=kv_heads, positions=kept)
        k64 = to_f64(k_raw, spec.dtype)
        v64 = to_f64(v_raw, spec.dtype)
        if spec.dtype == "fp8":
            # each position's values times the scale of its block and head
            blocks = np.array([int(tables[b][p // BLOCK_TOKENS]) for p in kept], dtype=np.int64)
            for arr, scales in ((k64, k_scale), (v64, v_scale)):
                sa = np.asarray(scales, dtype=np.float64)
                if sa.ndim == 3:
                    per = sa[layer][blocks][:, kv_heads]               # [positions][heads]
                else:
                    per = np.broadcast_to(sa[layer][kv_heads], (len(kept), len(kv_heads)))
                arr *= per[:, :, None]
        for h in qh:
            i = kv_heads.index(h // g)
            if lens[b] == 0 or k64.shape[0] == 0:
                continue
            out[b, h], lse[b, h] = softmax_attend(q64[b, h], k64[:, i, :], v64[:, i, :], sc)
    return out, lse


def partial_state(q64, k64, v64, scale):
    """Softmax state of one token range: (m, l, o) with o unnormalised."""
    s = (k64 @ q64) * scale
    m = s.max()
    w = np.exp(s - m)
    return m, w.sum(), w @ v64


def lse_merge(parts):
    """Merge (m_i, l_i, o_i) states of disjoint ranges: returns (out, lse).

    M = max m_i;  l = sum exp(m_i - M) l_i;  out = sum exp(m_i - M) o_i / l;
    lse = M + ln l.
    """
    big_m = max(p[0] for p in parts)
    l = sum(math.exp(p[0] - big_m) * p[1] for p in parts)
    o = sum(math.exp(p[0] - big_m) * p[2] for p in parts)
    return o / l, big_m + math.log(l)
