"""Write side of the paged cache: inject and append (oracle; test infra).

[InferScale] §3 (connector flow): blocks are first reserved for the memory
tokens without computing them, then the composed K/V is scatter-copied into
those blocks through the slot mapping; §3.3 and §5.1: the stored pre-rotation
key of each token is rotated to the position it lands on.  [InferScale] §2
and [KV essay] "The fix": decoding appends one K/V entry per generated token.

Readings taken where the pages are silent:

* a run is (seq, n, dst_pos, src_token): source tokens src_token ..
  src_token+n-1 land at positions dst_pos .. dst_pos+n-1 of ``seq``;
* every destination must lie inside the sequence's reserved blocks and below
  the rotary table length; two tokens of one call may not share a slot
  (rejected as 'OVERLAP'); positions written by an earlier call may be
  overwritten;
* after the call the sequence's length is max(old length, dst_pos + n);
* the key is rotated to its destination position (rope.rotate_f32) and
  rounded to the cache format; the value is copied bit for bit when the
  source and the cache share a format;
* a quantised (fp8) cache stores code = e4m3(f32(x / scale)) with one
  float32 scale per (layer, KV head) for K and one for V (the key after its
  rotation, the value as given), the division a single float32 division;
* append writes T tokens per sequence at positions len-T .. len-1 of the
  already-extended lengths, rotated the same way (mode "none" stores keys as
  given).

The source store is [layer][token][kv head][d], with element strides
``layer_stride`` and ``token_stride`` and the d elements of a head
contiguous.
"""

import numpy as np

from .layout import (BLOCK_TOKENS, PoolSpec, block_in_range, k_element_offsets, scale_at,
                     v_element_offsets, slot)
from .numerics import from_f32, to_f32, f32_to_e4m3_rne_sat
from .rope import rotate_f32


class InjectError(Exception):
    def __init__(self, code: str, msg: str):
        super().__init__("%s: %s" % (code, msg))
        self.code = code


def validate_runs(tables, lens, runs, max_pos: int):
    """Check every run; return the list of (seq, position, src_token) writes."""
    writes = []
    seen = set()
    for (seq, n, p0, src) in runs:
        if not (0 <= seq < len(tables)):
            raise InjectError("INVALID", "unknown sequence %d" % seq)
        if n < 0 or p0 < 0 or src < 0:
            raise InjectError("INVALID", "negative run field")
        if n == 0:
            continue  # an empty run names no position: nothing to check or write
        row = tables[seq]
        if p0 + n > len(row) * BLOCK_TOKENS:
            raise InjectError("RANGE", "run past reserved capacity")
        if p0 + n > max_pos:
            raise InjectError("RANGE", "run past the rotary table")
        if any(row[p // BLOCK_TOKENS] < 0 for p in range(p0, p0 + n)):
            raise InjectError("RANGE", "run writes positions without a block")
        for t in range(n):
            s = slot(tables[seq], p0 + t)
            if s in seen:
                raise InjectError("OVERLAP", "two tokens target slot %d" % s)
            seen.add(s)
            writes.append((seq, p0 + t, src + t))
    return writes


def _store(x32, dtype, scale):
    """float32 values -> stored codes of the cache format (fp8: x / scale)."""
    if dtype == "fp8":
        return f32_to_e4m3_rne_sat(np.divide(x32, np.float32(scale), dtype=np.float32))
    return from_f32(x32, dtype)


def write_token(k_pool, v_pool, spec: PoolSpec, layer: int, table_row, pos: int,
                k_raw, v_raw, mode: str, cos_t, sin_t, src_dtype=None, k_scale=None,
                v_scale=None):
    """Store one token (all KV heads) of one layer at position ``pos``.

    k_raw, v_raw: [n_kv_heads][d] in ``src_dtype`` (default: the cache's).
    k_scale, v_scale: float32 [n_layers][n_kv_heads], or per block
    [n_layers][num_blocks][n_kv_heads] (fp8 caches only): the code stored is
    e4m3(x / scale) with the scale of the destination's layer, block and head.
    """
    src_dtype = spec.dtype if src_dtype is None else src_dtype
    s = slot(table_row, pos)
    blk, t = divmod(s, BLOCK_TOKENS)
    k32 = to_f32(k_raw, src_dtype)
    k_rot = rotate_f32(k32, np.full(k32.shape[:-1], pos), cos_t, sin_t, mode)
    for h in range(spec.n_kv_heads):
        ks = None if k_scale is None else scale_at(k_scale, layer, blk, h)
        vs = None if v_scale is None else scale_at(v_scale, layer, blk, h)
        k_pool[k_element_offsets(spec, layer, blk, h, t)] = _store(k_rot[h], spec.dtype, ks)
        if src_dtype == spec.dtype:
            v_pool[v_element_offsets(spec, layer, blk, h, t)] = v_raw[h]
        else:
            v_pool[v_element_offsets(spec, layer, blk, h, t)] = _store(
                to_f32(v_raw[h], src_dtype), spec.dtype, vs)


def inject(k_pool, v_pool, spec: PoolSpec, tables, lens, runs, src_k, src_v,
           src_layer_stride: int, src_token_stride: int, layer_begin: int, layer_end: int,
           mode: str, cos_t, sin_t, src_dtype=None, k_scale=None, v_scale=None):
    """Scatter runs of stored, unrotated K/V into the pool; returns new lens."""
    max_pos = cos_t.shape[0]
    if not (0 <= layer_begin <= layer_end <= spec.n_layers):
        raise InjectError("INVALID", "bad layer range")
    writes = validate_runs(tables, lens, runs, max_pos)
    hd = spec.n_kv_heads * spec.head_dim
    for layer in range(layer_begin, layer_end):
        for (seq, pos, src) in writes:
            base = layer * src_layer_stride + src * src_token_stride
            k_raw = src_k[base:base + hd].reshape(spec.n_kv_heads, spec.head_dim)
            v_raw = src_v[base:base + hd].reshape(spec.n_kv_heads, spec.head_dim)
            write_token(k_pool, v_pool, spec, layer, tables[seq], pos, k_raw, v_raw,
                        mode, cos_t, sin_t, src_dtype, k_scale, v_scale)
    new_lens = list(lens)
    for (seq, n, p0, _src) in runs:
        if n > 0:  # the length covers the positions written
            new_lens[seq] = max(new_lens[seq], p0 + n)
    return new_lens


def append(k_pool, v_pool, spec: PoolSpec, layer: int, tables, lens_after, seqs, n_new: int,
           k_new, v_new, mode: str, cos_t, sin_t, src_dtype=None, k_scale=None, v_scale=None,
           num_blocks=None):
    """Write n_new tokens per sequence at its last n_new positions.

    k_new, v_new: raw arrays [len(seqs)][n_new][n_kv_heads][d].  With
    ``num_blocks`` given, the tables and first positions are device data and
    not trusted: a token is not written when its position is negative, past
    the table row, under a rotary pairing at or past the rotary table
    (max_pos = its row count), or when its table entry is outside
    [0, num_blocks).
    """
    max_pos = cos_t.shape[0]
    for i, seq in enumerate(seqs):
        first = lens_after[seq] - n_new
        for t in range(n_new):
            p = first + t
            if num_blocks is not None and (
                    p < 0 or p // BLOCK_TOKENS >= len(tables[seq])
                    or (mode != "none" and p >= max_pos)
                    or not block_in_range(tables[seq], p, num_blocks)):
                continue
            write_token(k_pool, v_pool, spec, layer, tables[seq], first + t,
                        k_new[i, t], v_new[i, t], mode, cos_t, sin_t, src_dtype, k_scale,
                        v_scale)


def copy_blocks(k_pool, v_pool, spec: PoolSpec, pairs, k_scale=None, v_scale=None):
    """Carry out queued copy-on-write copies, one after another in order:
    for each (src, dst) every layer's and KV head's K and V plane of block
    ``src`` is copied into block ``dst`` (a block holds all layers, since one
    table serves every layer).  Per-block fp8 scales (numpy arrays
    [n_layers][num_blocks][n_kv_heads]) travel with their planes; they are
    updated in place."""
    plane = BLOCK_TOKENS * spec.head_dim
    for src, dst in pairs:
        for layer in range(spec.n_layers):
            for h in range(spec.n_kv_heads):
                a = spec.plane_base(layer, int(src), h)
                b = spec.plane_base(layer, int(dst), h)
                k_pool[b:b + plane] = k_pool[a:a + plane].copy()
                v_pool[b:b + plane] = v_pool[a:a + plane].copy()
        for sc in (k_scale, v_scale):
            if sc is not None and np.ndim(sc) == 3:
                sc[:, int(dst), :] = sc[:, int(src), :]
