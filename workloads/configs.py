"""The workload shapes and their seeded input recipes.

Shapes follow the pages' examples: the Llama-3.1-8B grouped-query shape
(32 layers, 8 KV heads of 128, bf16) used for the per-fact storage cost in
"InferScale" and for the grouped-query example in "LLM Inference: KV Caching";
the Llama-3-70B shape (80 layers, 8 KV heads, 128, 16-bit, 8,192 tokens,
batch 32) of "Inside LLM Inference Engines" ("The KV Cache: Mathematical
Formulation"); the 64-head multi-head 70B reading of "Latency Optimization ›
KV Cache Management"; retrieved memories of tens to hundreds of tokens,
several per request, from "InferScale" §6.

Values: every q/K/V element is N(0, 1).  Host-side bfloat16 values are the
top 16 bits of float32 normal samples (truncation: a generator choice, not
the cache's rounding rule); float16 host values are numpy casts.  Large pools
are filled on the device by torch's seeded generator instead (see
``device_normal``), one generator per (seed, layer).
"""

from dataclasses import dataclass, field

import numpy as np

BLOCK = 16


@dataclass(frozen=True)
class Config:
    name: str
    workload: str
    seed: int
    n_layers: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    rope_base: float = 10000.0
    extra: dict = field(default_factory=dict)


TINY = Config(
    "tiny", "tiny fp32 reference: L=1 B=2 Hq=4 Hkv=2 d=64, lens 37/100, 16-block pool, "
    "24-token chunk injected at 40..63 of seq 1",
    1001, 1, 2, 4, 2, 64, "f32",
    extra=dict(lens=(37, 100), num_blocks=16, chunk_len=24, chunk_pos=40))
LLAMA8B_1LAYER = Config(
    "llama3-8b-1layer", "Llama-3-8B-shaped single-layer decode: Hq=32 Hkv=8 d=128 bf16, B=64, "
    "lens U[512,4096], pool 1.2x need",
    1002, 1, 64, 32, 8, 128, "bf16", extra=dict(len_lo=512, len_hi=4096))
LLAMA70B_80LAYER = Config(
    "llama3-70b-80layer", "Llama-3-70B-shaped decode: 80 layers, Hq=64 Hkv=8 d=128 bf16, "
    "B=32 x 8192 tokens, shuffled tables",
    1003, 80, 32, 64, 8, 128, "bf16", extra=dict(length=8192, num_blocks=16384))
INJECT_TOP8 = Config(
    "inject-top8", "KV injection + decode: top-8 of 10k chunks (64..256 tokens) of unrotated "
    "bf16 K/V (32 layers x 8 x 128), B=64, then 32-token suffix and one decode step",
    1004, 32, 64, 32, 8, 128, "bf16",
    extra=dict(n_chunks=10000, chunk_lo=64, chunk_hi=256, top_k=8, prefix_len=32, sep_len=15,
               suffix=32))
RAGGED_MHA = Config(
    "ragged-mha", "ragged MHA decode: Hq=Hkv=64 d=128 fp16, B=256, lens lognormal(median 1024, "
    "sigma 1) clipped to [16,32768], random tables",
    1005, 1, 256, 64, 64, 128, "f16",
    extra=dict(median=1024, sigma=1.0, len_lo=16, len_hi=32768))
MISTRAL_WINDOW = Config(
    "mistral-7b-window", "Mistral-7B-shaped sliding-window decode: 32 layers, Hq=32 Hkv=8 "
    "d=128 bf16, B=32 at position 32768 with a 4096-token window; tables hold the window's "
    "blocks only",
    1006, 32, 32, 32, 8, 128, "bf16", extra=dict(length=32768, window=4096))

MQA_64 = Config(
    "mqa-64-heads", "multi-query decode: 8 layers, Hq=64 Hkv=1 d=128 bf16, B=128 x 8192 tokens, "
    "shuffled tables (64 query heads share each KV head)",
    1007, 8, 128, 64, 1, 128, "bf16", extra=dict(length=8192, num_blocks=65536))

CONFIGS = {c.name: c for c in (TINY, LLAMA8B_1LAYER, LLAMA70B_80LAYER, INJECT_TOP8, RAGGED_MHA,
                                MISTRAL_WINDOW, MQA_64)}


def get_config(name: str) -> Config:
    return CONFIGS[name]


def blocks_for(n: int) -> int:
    return -(-int(n) // BLOCK)


# -- value generators --------------------------------------------------------------
def host_normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0, 1) values in storage form: float32, or uint16 bits for bf16/f16."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    raise ValueError(dtype)


def device_normal(n_elems: int, dtype: str, seed: int, device="cuda"):
    """N(0, 1) values drawn on the device by torch's seeded generator."""
    import torch
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randn(int(n_elems), dtype=tdt, device=device, generator=g)


# -- structure generators ----------------------------------------------------------
def deal_tables(ids: np.ndarray, lens, max_blocks: int) -> np.ndarray:
    """Give each sequence the next ceil(len/16) ids, in order; pad with -1."""
    t = np.full((len(lens), max_blocks), -1, dtype=np.int32)
    at = 0
    for b, ln in enumerate(lens):
        nb = blocks_for(ln)
        t[b, :nb] = ids[at:at + nb]
        at += nb
    return t


def tiny_inputs(cfg: Config = None):
    """Tiny workload: host arrays for a two-run prefill and one injected chunk.

    The source store holds seq 0's 37 tokens, seq 1's 100 tokens and the
    24-token chunk, all unrotated: [L][137 + 24][Hkv][d] fp32.
    """
    cfg = cfg or TINY
    rng = np.random.default_rng(cfg.seed)
    lens = list(cfg.extra["lens"])
    nb = cfg.extra["num_blocks"]
    perm = rng.permutation(nb).astype(np.int32)
    tables = np.full((2, 7), -1, dtype=np.int32)
    tables[0, :3] = perm[0:3]
    tables[1, :7] = perm[3:10]
    n_src = lens[0] + lens[1] + cfg.extra["chunk_len"]
    src_k = host_normal(rng, (cfg.n_layers, n_src, cfg.n_kv_heads, cfg.head_dim), cfg.dtype)
    src_v = host_normal(rng, (cfg.n_layers, n_src, cfg.n_kv_heads, cfg.head_dim), cfg.dtype)
    q = host_normal(rng, (cfg.batch, cfg.n_q_heads, cfg.head_dim), cfg.dtype)
    prefill_runs = [(0, lens[0], 0, 0), (1, lens[1], 0, lens[0])]
    chunk_runs = [(1, cfg.extra["chunk_len"], cfg.extra["chunk_pos"], lens[0] + lens[1])]
    return dict(lens=lens, tables=tables, num_blocks=nb, src_k=src_k, src_v=src_v, q=q,
                prefill_runs=prefill_runs, chunk_runs=chunk_runs, max_blocks=7)


def llama8b_structure(cfg: Config = None, batch=None):
    """Llama-3-8B single layer: lengths, pool size (1.2x need) and dealt random tables."""
    cfg = cfg or LLAMA8B_1LAYER
    rng = np.random.default_rng(cfg.seed)
    b = cfg.batch if batch is None else batch
    lens = rng.integers(cfg.extra["len_lo"], cfg.extra["len_hi"] + 1, size=b).astype(np.int64)
    need = int(sum(blocks_for(x) for x in lens))
    pool = -(-12 * need // 10)
    ids = rng.choice(pool, size=need, replace=False).astype(np.int32)
    max_blocks = blocks_for(cfg.extra["len_hi"])
    return dict(lens=lens, num_blocks=pool, tables=deal_tables(ids, lens, max_blocks),
                max_blocks=max_blocks, rng=rng)


def llama70b_structure(cfg: Config = None, block_tokens: int = BLOCK):
    """Llama-3-70B, 80 layers: all lengths 8192; one shuffled table shared by all layers.
    With 32-token blocks the shuffle is over block pairs of 16-token planes
    (2b, 2b+1), the table listing planes."""
    cfg = cfg or LLAMA70B_80LAYER
    rng = np.random.default_rng(cfg.seed)
    nb = cfg.extra["num_blocks"]
    per = cfg.extra["length"] // BLOCK
    k = block_tokens // BLOCK
    blocks = rng.permutation(nb // k).astype(np.int32)
    planes = (blocks[:, None] * k + np.arange(k, dtype=np.int32)[None, :]).reshape(-1)
    tables = planes.reshape(cfg.batch, per)
    lens = np.full(cfg.batch, cfg.extra["length"], dtype=np.int64)
    return dict(lens=lens, num_blocks=nb, tables=tables, max_blocks=per, rng=rng)


def ragged_mha_structure(cfg: Config = None, batch=None):
    """Ragged MHA: lognormal lengths, pool = exact need, permuted tables."""
    cfg = cfg or RAGGED_MHA
    rng = np.random.default_rng(cfg.seed)
    b = cfg.batch if batch is None else batch
    raw = np.exp(rng.normal(np.log(cfg.extra["median"]), cfg.extra["sigma"], size=b))
    lens = np.clip(np.rint(raw), cfg.extra["len_lo"], cfg.extra["len_hi"]).astype(np.int64)
    need = int(sum(blocks_for(x) for x in lens))
    ids = rng.permutation(need).astype(np.int32)
    max_blocks = int(max(blocks_for(x) for x in lens))
    return dict(lens=lens, num_blocks=need, tables=deal_tables(ids, lens, max_blocks),
                max_blocks=max_blocks, rng=rng)


def inject_structure(cfg: Config = None, n_chunks=None, batch=None):
    """Top-8 injection: chunk store index, per-request composition and run list.

    Store entries: chunk c (64..256 tokens), then a 32-token instruction
    prefix and a 15-token separator.  Each request lays out the prefix at
    positions 0..31, then for each of its 8 distinct chunks a gap of 1..15
    positions (filled from the separator's first tokens) followed by the
    chunk.  Runs are (seq, n, dst_pos, src_token); the whole list is
    shuffled.
    """
    cfg = cfg or INJECT_TOP8
    e = cfg.extra
    rng = np.random.default_rng(cfg.seed)
    nc = e["n_chunks"] if n_chunks is None else n_chunks
    b_n = cfg.batch if batch is None else batch
    chunk_lens = rng.integers(e["chunk_lo"], e["chunk_hi"] + 1, size=nc).astype(np.int64)
    starts = np.zeros(nc + 2, dtype=np.int64)
    starts[1:nc + 1] = np.cumsum(chunk_lens)
    prefix_at = int(starts[nc])
    sep_at = prefix_at + e["prefix_len"]
    n_src = sep_at + e["sep_len"]
    runs = []
    mem_lens = []
    picks = []
    for b in range(b_n):
        ids = rng.choice(nc, size=e["top_k"], replace=False)
        gaps = rng.integers(1, e["sep_len"] + 1, size=e["top_k"])
        picks.append(ids)
        p = 0
        runs.append((b, e["prefix_len"], p, prefix_at))
        p += e["prefix_len"]
        for c, g in zip(ids, gaps):
            runs.append((b, int(g), p, sep_at))
            p += int(g)
            runs.append((b, int(chunk_lens[c]), p, int(starts[c])))
            p += int(chunk_lens[c])
        mem_lens.append(p)
    order = rng.permutation(len(runs))
    runs = [runs[i] for i in order]
    need = int(sum(blocks_for(m + e["suffix"] + 1) for m in mem_lens))
    pool = -(-12 * need // 10)
    max_blocks = int(max(blocks_for(m + e["suffix"] + 1) for m in mem_lens))
    return dict(chunk_lens=chunk_lens, chunk_starts=starts[:nc], n_src=n_src, runs=runs,
                mem_lens=np.array(mem_lens, dtype=np.int64), picks=picks, num_blocks=pool,
                max_blocks=max_blocks, free_list_seed=cfg.seed, rng=rng)


def window_structure(cfg: Config = None):
    """Sliding-window decode: every sequence at the same position, its table
    holding only the blocks of the last ``window`` positions (the rest -1, as
    a window trim leaves them); block ids shuffled."""
    cfg = cfg or MISTRAL_WINDOW
    rng = np.random.default_rng(cfg.seed)
    n, w = cfg.extra["length"], cfg.extra["window"]
    per = blocks_for(n)
    keep_from = max(0, n - w) // BLOCK
    held = per - keep_from
    nb = cfg.batch * held
    tables = np.full((cfg.batch, per), -1, dtype=np.int32)
    tables[:, keep_from:] = rng.permutation(nb).astype(np.int32).reshape(cfg.batch, held)
    lens = np.full(cfg.batch, n, dtype=np.int64)
    return dict(lens=lens, num_blocks=nb, tables=tables, max_blocks=per, window=w, rng=rng)
