"""Physical layout of the paged pool (oracle; test infrastructure only).

[KV essay] "Paged attention" and [Inside engines] "PagedAttention: Virtual
Memory for LLM Generation" fix the logical structure: a sequence's positions
are cut into fixed blocks of 16 tokens, and a per-sequence block table maps
logical block i (positions 16i .. 16i+15) to a physical block of a shared
pool.  Position p of a sequence therefore lives in physical block
``table[p // 16]`` at in-block offset ``p % 16``; its "slot" is
``table[p // 16] * 16 + p % 16``.

The pages say nothing of the bytes inside a block.  The reading taken here
(one layout for every writer and reader, so that a pool can be compared byte
for byte):

* every (layer, physical block, KV head) owns one K plane and one V plane of
  16 * d elements each, found through element strides
  ``layer_stride``, ``block_stride``, ``head_stride`` from a K base and a V
  base (so K and V may live in separate arrays or interleaved in one);
* inside a K plane, element (t, j) -- token t of the block, dimension j --
  sits at ``((j // X) * 16 + t) * X + j % X`` with X = 16 bytes / element
  size: the plane is d/X chunks, each chunk holding X consecutive dimensions
  of all 16 tokens;
* inside a V plane, element (t, j) sits at ``j * 16 + t``: dimension-major,
  all 16 tokens of one dimension adjacent.
"""

from dataclasses import dataclass

import numpy as np

from .numerics import ELEM_BYTES

BLOCK_TOKENS = 16


def chunk_elems(dtype: str) -> int:
    """X: how many consecutive dimensions of one token a K-plane chunk holds."""
    return 16 // ELEM_BYTES[dtype]


def slot(table_row, p: int) -> int:
    """Slot of logical position ``p`` through a block-table row."""
    b = table_row[p // BLOCK_TOKENS]
    if b < 0:
        raise IndexError("position %d is past the sequence's blocks" % p)
    return int(b) * BLOCK_TOKENS + p % BLOCK_TOKENS


def k_plane_offset(t, j, dtype: str):
    """In-plane element offset of K(token t, dim j)."""
    x = chunk_elems(dtype)
    return ((np.asarray(j) // x) * BLOCK_TOKENS + np.asarray(t)) * x + np.asarray(j) % x


def v_plane_offset(t, j):
    """In-plane element offset of V(token t, dim j)."""
    return np.asarray(j) * BLOCK_TOKENS + np.asarray(t)


@dataclass(frozen=True)
class PoolSpec:
    """Shape and element strides of a paged pool (K and V share strides)."""
    n_layers: int
    num_blocks: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    layer_stride: int = -1
    block_stride: int = -1
    head_stride: int = -1

    def resolved(self) -> "PoolSpec":
        """Fill unset strides with the dense [layer][block][head][plane] order."""
        plane = BLOCK_TOKENS * self.head_dim
        hs = self.head_stride if self.head_stride >= 0 else plane
        bs = self.block_stride if self.block_stride >= 0 else self.n_kv_heads * hs
        ls = self.layer_stride if self.layer_stride >= 0 else self.num_blocks * bs
        return PoolSpec(self.n_layers, self.num_blocks, self.n_kv_heads, self.head_dim,
                        self.dtype, ls, bs, hs)

    def plane_base(self, layer: int, block: int, head: int) -> int:
        s = self.resolved()
        return layer * s.layer_stride + block * s.block_stride + head * s.head_stride

    def elements(self) -> int:
        """Smallest flat array length that holds every plane."""
        s = self.resolved()
        last = s.plane_base(self.n_layers - 1, self.num_blocks - 1, self.n_kv_heads - 1)
        return last + BLOCK_TOKENS * self.head_dim

    def storage_dtype(self):
        return {"f32": np.float32, "bf16": np.uint16, "f16": np.uint16, "fp8": np.uint8}[self.dtype]


def k_element_offsets(spec: PoolSpec, layer: int, block: int, head: int, t: int) -> np.ndarray:
    """Flat K-array offsets of dimensions 0..d-1 of token t of one plane."""
    j = np.arange(spec.head_dim)
    return spec.plane_base(layer, block, head) + k_plane_offset(t, j, spec.dtype)


def v_element_offsets(spec: PoolSpec, layer: int, block: int, head: int, t: int) -> np.ndarray:
    """Flat V-array offsets of dimensions 0..d-1 of token t of one plane."""
    j = np.arange(spec.head_dim)
    return spec.plane_base(layer, block, head) + v_plane_offset(t, j)


def read_token(k_pool, v_pool, spec: PoolSpec, layer: int, block: int, t: int):
    """Raw K and V of one slot, all heads: two arrays [n_kv_heads][d]."""
    k = np.stack([k_pool[k_element_offsets(spec, layer, block, h, t)]
                  for h in range(spec.n_kv_heads)])
    v = np.stack([v_pool[v_element_offsets(spec, layer, block, h, t)]
                  for h in range(spec.n_kv_heads)])
    return k, v


def scale_at(scales, layer: int, blk: int, h: int) -> float:
    """The float32 scale of an fp8 pool for (layer, block, KV head): scales
    are [n_layers][n_kv_heads] (one per layer and head) or
    [n_layers][num_blocks][n_kv_heads] (one per block as well)."""
    s = np.asarray(scales)
    return float(s[layer, blk, h]) if s.ndim == 3 else float(s[layer, h])


def block_in_range(table_row, p: int, num_blocks: int) -> bool:
    """Whether logical position ``p``'s table entry names a block of the pool
    (0 <= id < num_blocks).  Index data that lives on the device is not
    trusted: a position whose entry is out of range is never read or written
    (its element is skipped)."""
    b = int(table_row[p // BLOCK_TOKENS])
    return 0 <= b < num_blocks


def gather_sequence(k_pool, v_pool, spec: PoolSpec, layer: int, table_row, length: int,
                    heads=None, start: int = 0, positions=None):
    """Raw K, V of positions start..length-1 of one sequence:
    [length - start][H][d] each (or of the listed ``positions``, in order).

    Walks the block table one position at a time (the definition of paged
    reading); ``heads`` restricts the KV heads returned.
    """
    heads = list(range(spec.n_kv_heads)) if heads is None else list(heads)
    sdt = spec.storage_dtype()
    positions = list(range(start, length)) if positions is None else list(positions)
    n = len(positions)
    k = np.empty((n, len(heads), spec.head_dim), dtype=sdt)
    v = np.empty((n, len(heads), spec.head_dim), dtype=sdt)
    for i_p, p in enumerate(positions):
        s = slot(table_row, p)
        blk, t = divmod(s, BLOCK_TOKENS)
        for i, h in enumerate(heads):
            k[i_p, i] = k_pool[k_element_offsets(spec, layer, blk, h, t)]
            v[i_p, i] = v_pool[v_element_offsets(spec, layer, blk, h, t)]
    return k, v


def plane_tokens_k(plane, spec: PoolSpec) -> np.ndarray:
    """A whole K plane (16*d raw elements) as [16 tokens][d].

    The plane is d/X chunks of [16 tokens][X dims]: reshape to
    (d/X, 16, X), bring the token axis first, merge the chunk and dim axes.
    """
    x = chunk_elems(spec.dtype)
    return plane.reshape(spec.head_dim // x, BLOCK_TOKENS, x).transpose(1, 0, 2).reshape(
        BLOCK_TOKENS, spec.head_dim)


def plane_tokens_v(plane, spec: PoolSpec) -> np.ndarray:
    """A whole V plane (16*d raw elements, dimension-major) as [16 tokens][d]."""
    return plane.reshape(spec.head_dim, BLOCK_TOKENS).T


def gather_sequence_planes(k_pool, v_pool, spec: PoolSpec, layer: int, table_row, length: int,
                           heads=None, start: int = 0):
    """Same result as gather_sequence, one whole plane at a time."""
    heads = list(range(spec.n_kv_heads)) if heads is None else list(heads)
    n_blocks = -(-length // BLOCK_TOKENS)
    first = start // BLOCK_TOKENS
    plane = BLOCK_TOKENS * spec.head_dim
    k = np.empty((n_blocks * BLOCK_TOKENS, len(heads), spec.head_dim), spec.storage_dtype())
    v = np.empty_like(k)
    for i in range(first, n_blocks):
        blk = int(table_row[i])
        if blk < 0:
            raise IndexError("logical block %d has no physical block" % i)
        for hi, h in enumerate(heads):
            base = spec.plane_base(layer, blk, h)
            k[i * BLOCK_TOKENS:(i + 1) * BLOCK_TOKENS, hi] = plane_tokens_k(k_pool[base:base + plane], spec)
            v[i * BLOCK_TOKENS:(i + 1) * BLOCK_TOKENS, hi] = plane_tokens_v(v_pool[base:base + plane], spec)
    return k[start:length], v[start:length]
