// Host runtime of libpkv: block allocator, inject write planner, decode split
// planner, rotary table, argument validation and the C ABI (include/pkv.h).
//
// The allocator follows "LLM Inference: KV Caching" ("Paged attention": free
// list, per-sequence block table, a block handed out when the sequence
// reaches it) and "Inside LLM Inference Engines" ("PagedAttention",
// "Continuous Batching": blocks return to the pool when a sequence ends),
// with a FIFO free list so that the resulting tables are reproducible.
//
// Blocks are shared objects ("LLM Inference: KV Caching", "Paged attention"
// and "Prefix caching"; "Latency Optimization > KV Cache Management" on
// beams and prefix caching): each carries a reference count (the table
// entries naming it) and sits on the free list exactly when the count is 0.
// A sequence about to write into a block other sequences also name first
// takes a private copy (copy-on-write; the copies are queued and carried out
// on the GPU, in order, before any write).  Full blocks can be registered in
// a prefix cache keyed by (the preceding block's entry, the 16 positions'
// 64-bit keys) and compared exactly, so that a new sequence shares the
// longest cached chain from position 0; an entry lasts until its block is
// handed out again or written in place.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pkv_internal.h"

using pkv::DecodeItem;
using pkv::InjectDesc;
using pkv::MergeSeq;
using pkv::kBlock;

namespace {

thread_local std::string g_last_error;

pkv_status fail(pkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pkv_status ok() {
  g_last_error.clear();
  return PKV_OK;
}

pkv_status hip_fail(hipError_t e, const char* what) {
  return fail(PKV_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t blocks_for(int64_t n_tokens) { return (n_tokens + kBlock - 1) / kBlock; }

int elem_bytes(int32_t dtype) {
  switch (dtype) {
    case PKV_F32: return 4;
    case PKV_BF16: return 2;
    case PKV_F16: return 2;
    case PKV_FP8E4M3: return 1;
    default: return 0;
  }
}

// splitmix64 (S. Vigna's published definition): one 64-bit output per call.
struct SplitMix64 {
  uint64_t state;
  uint64_t next() {
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
};

// Pinned host staging for a small H2D upload, reusable once the previous copy
// out of it has landed (tracked with an event on the copying stream).
struct Staging {
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t done = nullptr;
  bool pending = false;

  ~Staging() {
    if (pending && done) (void)hipEventSynchronize(done);
    if (host) (void)hipHostFree(host);
    if (done) (void)hipEventDestroy(done);
  }

  // Returns a host buffer of >= bytes that no in-flight copy reads.
  pkv_status acquire(size_t bytes, void** out) {
    if (!done) {
      hipError_t e = hipEventCreateWithFlags(&done, hipEventDisableTiming);
      if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags");
    }
    if (pending) {
      hipError_t e = hipEventSynchronize(done);
      if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
      pending = false;
    }
    if (bytes > cap) {
      if (host) (void)hipHostFree(host);
      host = nullptr;
      cap = 0;
      size_t want = std::max<size_t>(bytes, 4096);
      hipError_t e = hipHostMalloc(&host, want, hipHostMallocDefault);
      if (e != hipSuccess) return hip_fail(e, "hipHostMalloc");
      cap = want;
    }
    *out = host;
    return PKV_OK;
  }

  pkv_status upload(void* dst, size_t bytes, hipStream_t stream) {
    hipError_t e = hipMemcpyAsync(dst, host, bytes, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
    e = hipEventRecord(done, stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    pending = true;
    return PKV_OK;
  }
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Prefix-cache key of one full block: the block registered for the
// preceding 16 positions (-1 at position 0) and this block's 16 keys.
struct PrefixKey {
  int32_t parent = -1;
  uint64_t keys[32] = {};  // one per position of a block (16 or 32 used)
  bool operator==(const PrefixKey& o) const {
    return parent == o.parent && std::memcmp(keys, o.keys, sizeof(keys)) == 0;
  }
};
struct PrefixKeyHash {
  size_t operator()(const PrefixKey& k) const {
    uint64_t h = 0x9E3779B97F4A7C15ull ^ uint64_t(uint32_t(k.parent));
    for (uint64_t x : k.keys) {
      h = (h ^ x) * 0xBF58476D1CE4E5B9ull;
      h ^= h >> 31;
    }
    return size_t(h);
  }
};

}  // namespace

struct pkv_cache {
  int32_t num_blocks = 0;
  int32_t max_seqs = 0;
  int32_t max_blocks_per_seq = 0;
  int32_t bt = kBlock;   // tokens per allocation block (16 or 32)
  int32_t sub = 1;       // 16-token planes per block
  int64_t blocks_for(int64_t n_tokens) const { return (n_tokens + bt - 1) / bt; }
  // FIFO free list, doubly linked through block ids (head = next handed out),
  // so that a cached block can be taken back from anywhere in O(1).
  std::vector<int32_t> fl_prev, fl_next;
  int32_t fl_head = -1, fl_tail = -1, fl_size = 0;
  std::vector<int32_t> ref;                               // table entries per block
  std::vector<std::pair<int32_t, int32_t>> pending;       // queued copies (src, dst)
  std::unordered_map<PrefixKey, int32_t, PrefixKeyHash> entries;
  std::vector<PrefixKey> entry_key;                       // valid where cached[b]
  std::vector<uint8_t> cached;
  std::vector<std::vector<int32_t>> children;             // entries registered under b
  std::vector<std::vector<int32_t>> tables;
  std::vector<int64_t> lens;
  std::vector<int32_t> desc_of_block;  // inject planner scratch, -1 when idle
  std::vector<uint8_t> touched_flag;   // inject planner scratch per (seq, block index), 0 when idle
  Staging staging;

  void fl_push_back(int32_t b) {
    fl_prev[b] = fl_tail;
    fl_next[b] = -1;
    if (fl_tail >= 0) fl_next[fl_tail] = b; else fl_head = b;
    fl_tail = b;
    ++fl_size;
  }
  void fl_remove(int32_t b) {
    if (fl_prev[b] >= 0) fl_next[fl_prev[b]] = fl_next[b]; else fl_head = fl_next[b];
    if (fl_next[b] >= 0) fl_prev[fl_next[b]] = fl_prev[b]; else fl_tail = fl_prev[b];
    fl_prev[b] = fl_next[b] = -1;
    --fl_size;
  }
  // Drops b's prefix entry and every entry registered under it.
  void forget(int32_t b) {
    std::vector<int32_t> stack{b};
    while (!stack.empty()) {
      const int32_t x = stack.back();
      stack.pop_back();
      if (cached[x]) {
        cached[x] = 0;
        const PrefixKey& key = entry_key[x];
        entries.erase(key);
        if (key.parent >= 0) {
          auto& ch = children[key.parent];
          auto it = std::find(ch.begin(), ch.end(), x);
          if (it != ch.end()) {
            *it = ch.back();
            ch.pop_back();
          }
        }
      }
      for (int32_t y : children[x]) stack.push_back(y);
      children[x].clear();
    }
  }
  // Hands out the free list's head (forgetting what it cached).
  int32_t pop_block() {
    const int32_t b = fl_head;
    fl_remove(b);
    forget(b);
    ref[b] = 1;
    return b;
  }
  // Gives sequence `seq` a private copy of its idx-th block.
  void cow(int32_t seq, int64_t idx) {
    const int32_t old = tables[seq][idx];
    const int32_t fresh = pop_block();
    pending.emplace_back(old, fresh);
    tables[seq][idx] = fresh;
    --ref[old];
  }
  // One past the last table index, among the blocks seq already holds, that
  // its next n_new positions reach (the first is lens[seq] / bt).
  int64_t written_end(int32_t seq, int32_t n_new) const {
    if (n_new <= 0) return 0;
    return std::min<int64_t>(int64_t(tables[seq].size()), blocks_for(lens[seq] + n_new));
  }
  // Drops one reference to each block of a table, in table order.
  void release(const std::vector<int32_t>& t) {
    for (int32_t b : t)
      if (b >= 0 && --ref[b] == 0) fl_push_back(b);  // -1: dropped by a window trim
  }
};

struct pkv_plan {
  int32_t n_seqs = 0, n_q_heads = 0, n_kv_heads = 0, head_dim = 0, part_tokens = 0;
  int32_t n_slots = 0, waves = 1;
  std::vector<DecodeItem> items;
  std::vector<MergeSeq> merges;
  std::vector<int32_t> newest;  // per sequence: lens - 1 (-1: empty)
  size_t off_items = 0, off_merges = 0, off_pos = 0, off_part_o = 0, off_part_ml = 0,
         ws_bytes = 0;
  Staging staging;
};

namespace {

pkv_status check_seq(const pkv_cache* c, int32_t seq) {
  if (!c) return fail(PKV_E_INVALID, "null cache");
  if (seq < 0 || seq >= c->max_seqs)
    return fail(PKV_E_INVALID, "sequence %d out of range [0, %d)", seq, c->max_seqs);
  return PKV_OK;
}

// Validates a pool descriptor: shapes, dtype, alignment.
pkv_status check_pool(const pkv_pool* p) {
  if (!p) return fail(PKV_E_INVALID, "null pool");
  const int eb = elem_bytes(p->dtype);
  if (!eb) return fail(PKV_E_INVALID, "unknown pool dtype %d", p->dtype);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(PKV_E_UNSUPPORTED, "head_dim %d (supported: 64, 128)", p->head_dim);
  if (p->n_layers <= 0 || p->num_blocks <= 0 || p->n_kv_heads <= 0)
    return fail(PKV_E_INVALID, "pool sizes must be positive");
  if (!p->k || !p->v) return fail(PKV_E_INVALID, "null pool pointer");
  if ((reinterpret_cast<uintptr_t>(p->k) | reinterpret_cast<uintptr_t>(p->v)) & 15)
    return fail(PKV_E_INVALID, "pool base pointers must be 16-byte aligned");
  const int64_t plane = int64_t(kBlock) * p->head_dim;
  if (p->layer_stride < 0 || p->block_stride < 0 || p->head_stride < 0)
    return fail(PKV_E_INVALID, "negative pool stride");
  if (((p->layer_stride | p->block_stride | p->head_stride) * eb) % 16)
    return fail(PKV_E_INVALID, "pool strides must be multiples of 16 bytes");
  if (p->n_kv_heads > 1 && p->head_stride < plane)
    return fail(PKV_E_INVALID, "head_stride smaller than a plane");
  if (p->num_blocks > 1 && p->block_stride < plane)
    return fail(PKV_E_INVALID, "block_stride smaller than a plane");
  if (p->dtype == PKV_FP8E4M3 && (!p->k_scale || !p->v_scale))
    return fail(PKV_E_INVALID, "an FP8E4M3 pool needs k_scale and v_scale");
  if (p->scale_mode != 0 && !(p->scale_mode == 1 && p->dtype == PKV_FP8E4M3))
    return fail(PKV_E_INVALID, "scale_mode %d (0, or 1 for an FP8E4M3 pool)", p->scale_mode);
  return PKV_OK;
}

// Format of incoming K/V or q for a pool: the pool's own, or a 16-bit float
// for a quantised (FP8E4M3) pool.
pkv_status check_input_dtype(const pkv_pool* p, int32_t dtype, const char* what) {
  if (p->dtype == PKV_FP8E4M3) {
    if (dtype == PKV_BF16 || dtype == PKV_F16) return PKV_OK;
    return fail(PKV_E_UNSUPPORTED, "%s dtype %d for an FP8E4M3 pool (supported: BF16, F16)",
                what, dtype);
  }
  if (dtype != p->dtype)
    return fail(PKV_E_UNSUPPORTED, "%s dtype %d differs from the pool's %d", what, dtype,
                p->dtype);
  return PKV_OK;
}

pkv_status check_rope(int32_t mode, const float* cos, const float* sin, int32_t max_pos) {
  if (mode != PKV_ROPE_PAIRS && mode != PKV_ROPE_HALVES && mode != PKV_ROPE_NONE)
    return fail(PKV_E_INVALID, "unknown rope mode %d", mode);
  if (mode != PKV_ROPE_NONE && (!cos || !sin))
    return fail(PKV_E_INVALID, "rotary table pointers are null");
  if (max_pos < 0) return fail(PKV_E_INVALID, "negative max_pos");
  return PKV_OK;
}

// Carries out the queued copy-on-write copies on `stream`.  The queue's
// meaning is sequential; copies go out in levels so that no launch holds two
// copies touching a common block as destination, or as the source of one and
// the destination of the other: a copy's level is one above the highest
// level of an earlier copy it depends on.
pkv_status flush_copies(pkv_cache* c, const pkv_pool& pool, hipStream_t stream) {
  for (const auto& pr : c->pending)
    if ((int64_t(pr.first) + 1) * c->sub > pool.num_blocks ||
        (int64_t(pr.second) + 1) * c->sub > pool.num_blocks)
      return fail(PKV_E_RANGE, "copy %d -> %d outside the pool's %d planes", pr.first,
                  pr.second, pool.num_blocks);
  std::unordered_map<int32_t, int32_t> read_at, written_at;  // highest level per block
  std::vector<int32_t> level(c->pending.size());
  int32_t n_levels = 0;
  for (size_t i = 0; i < c->pending.size(); ++i) {
    const int32_t s = c->pending[i].first, d = c->pending[i].second;
    int32_t lv = 0;
    auto bump = [&](const std::unordered_map<int32_t, int32_t>& m, int32_t b) {
      auto it = m.find(b);
      if (it != m.end()) lv = std::max(lv, it->second + 1);
    };
    bump(written_at, s);  // reads what an earlier copy writes
    bump(read_at, d);     // overwrites what an earlier copy reads
    bump(written_at, d);  // overwrites what an earlier copy writes
    level[i] = lv;
    read_at[s] = std::max(read_at.count(s) ? read_at[s] : 0, lv);
    written_at[d] = std::max(written_at.count(d) ? written_at[d] : 0, lv);
    n_levels = std::max(n_levels, lv + 1);
  }
  pkv::CopyBatch batch;
  for (int32_t lv = 0; lv < n_levels; ++lv) {
    batch.n = 0;
    for (size_t i = 0; i <= c->pending.size(); ++i) {
      const bool last = i == c->pending.size();
      if (!last && level[i] == lv) {
        for (int32_t k = 0; k < c->sub; ++k) {  // the block's 16-token planes
          batch.src[batch.n] = c->pending[i].first * c->sub + k;
          batch.dst[batch.n] = c->pending[i].second * c->sub + k;
          ++batch.n;
        }
      }
      if (batch.n + c->sub > pkv::kCopyBatch || (last && batch.n > 0)) {
        hipError_t e = pkv::launch_copy_blocks(pool, batch, stream);
        if (e != hipSuccess) return hip_fail(e, "block copy launch");
        batch.n = 0;
      }
    }
  }
  c->pending.clear();
  return PKV_OK;
}

// Device-visible address of an inject source: device (or managed) memory as
// is; pinned host memory (hipHostMalloc, torch's pin_memory) through the
// address the GPU reads it by over PCIe.  Anything else -- pageable host
// memory in particular, which the GPU cannot read -- is rejected before any
// work is enqueued.
pkv_status resolve_source(const void* p, const char* what, const void** dev, bool* in_host) {
  hipPointerAttribute_t attr;
  std::memset(&attr, 0, sizeof(attr));
  const hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PKV_E_INVALID, "%s %p is neither device memory nor pinned host memory", what, p);
  }
  if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged) {
    *dev = p;
    *in_host = false;
    return PKV_OK;
  }
  if (attr.type == hipMemoryTypeHost && attr.devicePointer) {
    *in_host = true;
    const char* base_h = static_cast<const char*>(attr.hostPointer ? attr.hostPointer : p);
    *dev = static_cast<const char*>(attr.devicePointer) + (static_cast<const char*>(p) - base_h);
    return PKV_OK;
  }
  return fail(PKV_E_INVALID, "%s %p is neither device memory nor pinned host memory", what, p);
}

// Upper bound of destination blocks touched by a list of runs.
int64_t inject_desc_bound(const pkv_run* runs, int32_t n_runs) {
  int64_t n = 0;
  for (int32_t i = 0; i < n_runs; ++i)
    if (runs[i].n_tokens > 0) n += blocks_for(runs[i].n_tokens) + 1;
  return n;
}

}  // namespace

extern "C" {

int32_t pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_last_error(void) { return g_last_error.c_str(); }

uint64_t pkv_kv_bytes(int32_t n_layers, int32_t n_kv_heads, int32_t head_dim, int32_t elem_b,
                      int64_t n_tokens) {
  if (n_layers < 0 || n_kv_heads < 0 || head_dim < 0 || elem_b < 0 || n_tokens < 0) return 0;
  return 2ull * uint64_t(n_layers) * uint64_t(n_kv_heads) * uint64_t(head_dim) *
         uint64_t(elem_b) * uint64_t(n_tokens);
}

// ---------------------------------------------------------------------------
// Allocator
// ---------------------------------------------------------------------------
pkv_status pkv_cache_create(const pkv_cache_config* cfg, pkv_cache** out) {
  if (!cfg || !out) return fail(PKV_E_INVALID, "null argument");
  if (cfg->num_blocks <= 0 || cfg->max_seqs <= 0 || cfg->max_blocks_per_seq <= 0)
    return fail(PKV_E_INVALID, "cache sizes must be positive");
  const int32_t bt = cfg->block_tokens == 0 ? kBlock : cfg->block_tokens;
  if (bt != 16 && bt != 32) return fail(PKV_E_INVALID, "block_tokens must be 16 or 32");
  if (int64_t(cfg->num_blocks) * (bt / kBlock) > INT32_MAX)
    return fail(PKV_E_INVALID, "too many blocks");
  pkv_cache* c = new (std::nothrow) pkv_cache();
  if (!c) return fail(PKV_E_INVALID, "out of host memory");
  c->num_blocks = cfg->num_blocks;
  c->bt = bt;
  c->sub = bt / kBlock;
  c->max_seqs = cfg->max_seqs;
  c->max_blocks_per_seq = cfg->max_blocks_per_seq;
  std::vector<int32_t> order(cfg->num_blocks);
  for (int32_t i = 0; i < cfg->num_blocks; ++i) order[i] = i;
  if (cfg->free_list_seed != 0) {
    SplitMix64 g{cfg->free_list_seed};
    for (int64_t i = int64_t(cfg->num_blocks) - 1; i > 0; --i) {
      uint64_t j = g.next() % uint64_t(i + 1);
      std::swap(order[i], order[j]);
    }
  }
  c->fl_prev.assign(cfg->num_blocks, -1);
  c->fl_next.assign(cfg->num_blocks, -1);
  for (int32_t b : order) c->fl_push_back(b);
  c->ref.assign(cfg->num_blocks, 0);
  c->entry_key.resize(cfg->num_blocks);
  c->cached.assign(cfg->num_blocks, 0);
  c->children.resize(cfg->num_blocks);
  c->tables.resize(cfg->max_seqs);
  c->lens.assign(cfg->max_seqs, 0);
  *out = c;
  return ok();
}

void pkv_cache_destroy(pkv_cache* cache) { delete cache; }

pkv_status pkv_alloc_blocks(pkv_cache* c, int32_t seq, int64_t n_tokens) {
  if (pkv_status st = check_seq(c, seq)) return st;
  if (n_tokens < 0) return fail(PKV_E_INVALID, "negative token count");
  const int64_t want = c->blocks_for(n_tokens);
  if (want > c->max_blocks_per_seq)
    return fail(PKV_E_RANGE, "%lld blocks exceed max_blocks_per_seq %d", (long long)want,
                c->max_blocks_per_seq);
  auto& t = c->tables[seq];
  const int64_t need = std::max<int64_t>(0, want - int64_t(t.size()));
  if (need > c->fl_size)
    return fail(PKV_E_OOM, "need %lld blocks, %d free", (long long)need, c->fl_size);
  for (int64_t i = 0; i < need; ++i) t.push_back(c->pop_block());
  return ok();
}

pkv_status pkv_set_blocks(pkv_cache* c, int32_t seq, const int32_t* ids, int32_t n_ids,
                          int64_t len) {
  if (pkv_status st = check_seq(c, seq)) return st;
  if (n_ids < 0 || (n_ids > 0 && !ids)) return fail(PKV_E_INVALID, "bad id list");
  if (!c->tables[seq].empty()) return fail(PKV_E_INVALID, "sequence %d already owns blocks", seq);
  if (n_ids > c->max_blocks_per_seq)
    return fail(PKV_E_RANGE, "%d blocks exceed max_blocks_per_seq %d", n_ids,
                c->max_blocks_per_seq);
  if (len < 0 || len > int64_t(n_ids) * c->bt)
    return fail(PKV_E_RANGE, "length %lld does not fit %d blocks", (long long)len, n_ids);
  std::vector<uint8_t> taken(c->num_blocks, 0);
  for (int32_t i = 0; i < n_ids; ++i) {
    const int32_t b = ids[i];
    if (b < 0 || b >= c->num_blocks) return fail(PKV_E_INVALID, "block id %d out of range", b);
    if (c->ref[b] != 0) return fail(PKV_E_INVALID, "block id %d is not free", b);
    if (taken[b]) return fail(PKV_E_INVALID, "block id %d repeated", b);
    taken[b] = 1;
  }
  for (int32_t i = 0; i < n_ids; ++i) {
    c->fl_remove(ids[i]);
    c->forget(ids[i]);
    c->ref[ids[i]] = 1;
  }
  c->tables[seq].assign(ids, ids + n_ids);
  c->lens[seq] = len;
  return ok();
}

pkv_status pkv_extend(pkv_cache* c, const int32_t* seqs, int32_t n_seqs, int32_t n_new,
                      int64_t* first_pos_out) {
  if (!c) return fail(PKV_E_INVALID, "null cache");
  if (n_seqs < 0 || (n_seqs > 0 && !seqs) || n_new < 0)
    return fail(PKV_E_INVALID, "bad sequence list or count");
  std::vector<uint8_t> seen(c->max_seqs, 0);
  std::unordered_map<int32_t, int32_t> refs_then;  // counts as they will be when reached
  int64_t total = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    if (pkv_status st = check_seq(c, seqs[i])) return st;
    if (seen[seqs[i]]) return fail(PKV_E_INVALID, "sequence %d repeated", seqs[i]);
    seen[seqs[i]] = 1;
    const int32_t s = seqs[i];
    const int64_t want = c->blocks_for(c->lens[s] + n_new);
    if (want > c->max_blocks_per_seq)
      return fail(PKV_E_RANGE, "sequence %d would need %lld blocks", s, (long long)want);
    total += std::max<int64_t>(0, want - int64_t(c->tables[s].size()));
    const int64_t hi = c->written_end(s, n_new);
    for (int64_t j = c->lens[s] / c->bt; j < hi; ++j) {
      const int32_t b = c->tables[s][j];
      if (b < 0) continue;
      auto it = refs_then.find(b);
      const int32_t r = it == refs_then.end() ? c->ref[b] : it->second;
      if (r > 1) {
        ++total;
        refs_then[b] = r - 1;
      }
    }
  }
  if (total > c->fl_size)
    return fail(PKV_E_OOM, "need %lld blocks, %d free", (long long)total, c->fl_size);
  for (int32_t i = 0; i < n_seqs; ++i) {
    const int32_t s = seqs[i];
    // Blocks already in the table that will receive new positions and that
    // other sequences share (a fork shares reserved blocks past the length
    // too): each is copied before the write.
    const int64_t hi = c->written_end(s, n_new);
    for (int64_t j = c->lens[s] / c->bt; j < hi; ++j) {
      const int32_t b = c->tables[s][j];
      if (b >= 0 && c->ref[b] > 1) c->cow(s, j);
    }
    pkv_alloc_blocks(c, s, c->lens[s] + n_new);
    if (first_pos_out) first_pos_out[i] = c->lens[s];
    c->lens[s] += n_new;
  }
  return ok();
}

pkv_status pkv_free_seq(pkv_cache* c, int32_t seq) {
  if (pkv_status st = check_seq(c, seq)) return st;
  c->release(c->tables[seq]);
  c->tables[seq].clear();
  c->lens[seq] = 0;
  return ok();
}

pkv_status pkv_block_table(const pkv_cache* c, const int32_t* seqs, int32_t n_seqs,
                           int32_t* table_out, int64_t* lens_out) {
  if (!c) return fail(PKV_E_INVALID, "null cache");
  if (n_seqs < 0 || (n_seqs > 0 && (!seqs || !table_out)))
    return fail(PKV_E_INVALID, "bad arguments");
  for (int32_t i = 0; i < n_seqs; ++i)
    if (pkv_status st = check_seq(c, seqs[i])) return st;
  const int64_t width = int64_t(c->max_blocks_per_seq) * c->sub;
  for (int32_t i = 0; i < n_seqs; ++i) {
    const auto& t = c->tables[seqs[i]];
    int32_t* row = table_out + int64_t(i) * width;
    for (int64_t j = 0; j < width; ++j) {
      const int64_t blk = j / c->sub;
      row[j] = blk < int64_t(t.size()) && t[blk] >= 0 ? t[blk] * c->sub + int32_t(j % c->sub) : -1;
    }
    if (lens_out) lens_out[i] = c->lens[seqs[i]];
  }
  return ok();
}

int32_t pkv_table_width(const pkv_cache* c) {
  return c ? c->max_blocks_per_seq * c->sub : -1;
}

int32_t pkv_num_free_blocks(const pkv_cache* c) {
  return c ? c->fl_size : -1;
}

int32_t pkv_free_list(const pkv_cache* c, int32_t* out, int32_t cap) {
  if (!c || (cap > 0 && !out) || cap < 0) return fail(PKV_E_INVALID, "bad arguments");
  int32_t n = 0;
  for (int32_t b = c->fl_head; b >= 0 && n < cap; b = c->fl_next[b]) out[n++] = b;
  ok();
  return n;
}

// ---------------------------------------------------------------------------
// Sharing: fork, copy-on-write copies, prefix cache
// ---------------------------------------------------------------------------
pkv_status pkv_fork(pkv_cache* c, int32_t src_seq, int32_t dst_seq) {
  if (pkv_status st = check_seq(c, src_seq)) return st;
  if (pkv_status st = check_seq(c, dst_seq)) return st;
  if (src_seq == dst_seq || !c->tables[dst_seq].empty() || c->lens[dst_seq] != 0)
    return fail(PKV_E_INVALID, "fork needs a distinct, empty destination sequence");
  for (int32_t b : c->tables[src_seq])
    if (b >= 0) ++c->ref[b];
  c->tables[dst_seq] = c->tables[src_seq];
  c->lens[dst_seq] = c->lens[src_seq];
  return ok();
}

int32_t pkv_block_refcount(const pkv_cache* c, int32_t block) {
  if (!c || block < 0 || block >= c->num_blocks) return fail(PKV_E_INVALID, "bad block id");
  ok();
  return c->ref[block];
}

int32_t pkv_pending_copies(const pkv_cache* c, int32_t* pairs_out, int32_t cap) {
  if (!c || cap < 0 || (cap > 0 && !pairs_out)) return fail(PKV_E_INVALID, "bad arguments");
  const int32_t n = int32_t(c->pending.size());
  for (int32_t i = 0; i < n && i < cap; ++i) {
    pairs_out[2 * i] = c->pending[i].first;
    pairs_out[2 * i + 1] = c->pending[i].second;
  }
  ok();
  return n;
}

pkv_status pkv_copy_blocks(pkv_cache* c, const pkv_pool* pool, void* stream) {
  if (!c) return fail(PKV_E_INVALID, "null cache");
  if (c->pending.empty()) return ok();
  if (pkv_status st = check_pool(pool)) return st;
  return flush_copies(c, *pool, static_cast<hipStream_t>(stream));
}

pkv_status pkv_prefix_match(pkv_cache* c, int32_t seq, const uint64_t* keys, int64_t n_keys,
                            int64_t* matched_out) {
  if (pkv_status st = check_seq(c, seq)) return st;
  if (n_keys < 0 || (n_keys > 0 && !keys)) return fail(PKV_E_INVALID, "bad key list");
  if (!c->tables[seq].empty() || c->lens[seq] != 0)
    return fail(PKV_E_INVALID, "prefix match needs an empty sequence");
  const int64_t full = std::min<int64_t>(n_keys / c->bt, c->max_blocks_per_seq);
  PrefixKey key;
  auto& t = c->tables[seq];
  for (int64_t i = 0; i < full; ++i) {
    std::memcpy(key.keys, keys + i * c->bt, sizeof(uint64_t) * c->bt);
    auto it = c->entries.find(key);
    if (it == c->entries.end()) break;
    const int32_t b = it->second;
    if (c->ref[b] == 0) c->fl_remove(b);
    ++c->ref[b];
    t.push_back(b);
    key.parent = b;
  }
  c->lens[seq] = int64_t(t.size()) * c->bt;
  if (matched_out) *matched_out = c->lens[seq];
  return ok();
}

pkv_status pkv_prefix_commit(pkv_cache* c, int32_t seq, const uint64_t* keys, int64_t n_keys) {
  if (pkv_status st = check_seq(c, seq)) return st;
  if (n_keys < 0 || (n_keys > 0 && !keys)) return fail(PKV_E_INVALID, "bad key list");
  if (n_keys > c->lens[seq])
    return fail(PKV_E_RANGE, "%lld keys for a sequence of %lld tokens", (long long)n_keys,
                (long long)c->lens[seq]);
  const int64_t full = n_keys / c->bt;
  for (int64_t i = 0; i < full; ++i)
    if (c->tables[seq][i] < 0)
      return fail(PKV_E_RANGE, "keys cover positions the sequence no longer holds");
  std::vector<std::pair<PrefixKey, int32_t>> plan;
  PrefixKey key;
  for (int64_t i = 0; i < full; ++i) {
    const int32_t b = c->tables[seq][i];
    std::memcpy(key.keys, keys + i * c->bt, sizeof(uint64_t) * c->bt);
    auto it = c->entries.find(key);
    if (it != c->entries.end()) {
      key.parent = it->second;
      continue;
    }
    if (c->cached[b])
      return fail(PKV_E_INVALID, "block %d already caches other content", b);
    plan.emplace_back(key, b);
    key.parent = b;
  }
  for (const auto& pb : plan) {
    const int32_t b = pb.second;
    c->entries.emplace(pb.first, b);
    c->entry_key[b] = pb.first;
    c->cached[b] = 1;
    if (pb.first.parent >= 0) c->children[pb.first.parent].push_back(b);
  }
  return ok();
}

int32_t pkv_prefix_cached_blocks(const pkv_cache* c) {
  return c ? int32_t(c->entries.size()) : -1;
}

pkv_status pkv_trim_window(pkv_cache* c, const int32_t* seqs, int32_t n_seqs, int32_t window,
                           int64_t* dropped_out) {
  if (!c) return fail(PKV_E_INVALID, "null cache");
  if (n_seqs < 0 || (n_seqs > 0 && !seqs)) return fail(PKV_E_INVALID, "bad sequence list");
  if (window <= 0) return fail(PKV_E_INVALID, "window must be positive");
  for (int32_t i = 0; i < n_seqs; ++i)
    if (pkv_status st = check_seq(c, seqs[i])) return st;
  int64_t dropped = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    auto& t = c->tables[seqs[i]];
    const int64_t keep_from = std::max<int64_t>(0, c->lens[seqs[i]] - window) / c->bt;
    for (int64_t j = 0; j < std::min<int64_t>(keep_from, int64_t(t.size())); ++j) {
      const int32_t b = t[j];
      if (b < 0) continue;
      if (--c->ref[b] == 0) c->fl_push_back(b);
      t[j] = -1;
      ++dropped;
    }
  }
  if (dropped_out) *dropped_out = dropped;
  return ok();
}

// ---------------------------------------------------------------------------
// Rotary table
// ---------------------------------------------------------------------------
pkv_status pkv_rope_table(int32_t head_dim, double base, int32_t max_pos, float* cos_out,
                          float* sin_out) {
  if (head_dim <= 0 || head_dim % 2 || max_pos < 0 || !(base > 0.0))
    return fail(PKV_E_INVALID, "bad rotary table shape or base");
  if (max_pos > 0 && (!cos_out || !sin_out)) return fail(PKV_E_INVALID, "null output");
  const int32_t half = head_dim / 2;
  std::vector<double> theta(half);
  for (int32_t i = 0; i < half; ++i) theta[i] = std::pow(base, -2.0 * double(i) / head_dim);
  for (int64_t p = 0; p < max_pos; ++p) {
    for (int32_t i = 0; i < half; ++i) {
      const double a = double(p) * theta[i];
      cos_out[p * half + i] = float(std::cos(a));
      sin_out[p * half + i] = float(std::sin(a));
    }
  }
  return ok();
}

// ---------------------------------------------------------------------------
// Inject
// ---------------------------------------------------------------------------
size_t pkv_inject_workspace_bytes(const pkv_run* runs, int32_t n_runs) {
  if (n_runs <= 0 || !runs) return 256;
  return align_up(size_t(inject_desc_bound(runs, n_runs)) * sizeof(InjectDesc), 256);
}

pkv_status pkv_host_alloc(size_t n_bytes, void** out) {
  if (!out || n_bytes == 0) return fail(PKV_E_INVALID, "bad arguments");
  *out = nullptr;
  hipError_t e = hipHostMalloc(out, n_bytes, hipHostMallocDefault);
  if (e != hipSuccess) {
    *out = nullptr;
    return hip_fail(e, "pinned host allocation");
  }
  return ok();
}

pkv_status pkv_host_free(void* p) {
  if (!p) return ok();
  hipError_t e = hipHostFree(p);
  if (e != hipSuccess) return hip_fail(e, "pinned host release");
  return ok();
}

pkv_status pkv_inject(pkv_cache* c, const pkv_pool* pool, const pkv_src* src,
                      const pkv_run* runs, int32_t n_runs, int32_t layer_begin,
                      int32_t layer_end, int32_t rope_mode, const float* d_cos,
                      const float* d_sin, int32_t max_pos, void* d_ws, size_t ws_bytes,
                      void* stream) {
  if (!c) return fail(PKV_E_INVALID, "null cache");
  if (pkv_status st = check_pool(pool)) return st;
  if (pkv_status st = check_rope(rope_mode, d_cos, d_sin, max_pos)) return st;
  if (!src || !src->k || !src->v) return fail(PKV_E_INVALID, "null source");
  if (pkv_status st = check_input_dtype(pool, src->dtype, "source")) return st;
  const int eb = elem_bytes(src->dtype);
  if ((reinterpret_cast<uintptr_t>(src->k) | reinterpret_cast<uintptr_t>(src->v)) & 15)
    return fail(PKV_E_INVALID, "source pointers must be 16-byte aligned");
  if (((src->layer_stride | src->token_stride) * eb) % 16 || src->layer_stride < 0 ||
      src->token_stride < int64_t(pool->n_kv_heads) * pool->head_dim)
    return fail(PKV_E_INVALID, "bad source strides");
  if (n_runs < 0 || (n_runs > 0 && !runs)) return fail(PKV_E_INVALID, "bad run list");
  if (layer_begin < 0 || layer_end > pool->n_layers || layer_begin > layer_end)
    return fail(PKV_E_INVALID, "layer range [%d, %d) outside [0, %d)", layer_begin, layer_end,
                pool->n_layers);

  // Resolve every run token to (sequence, logical block, slot); build one
  // write descriptor per destination block, in order of first touch.  A
  // block several sequences share gets one descriptor per writing sequence
  // (copy-on-write below gives all but the last writer a private copy), so
  // descriptors hang off the block's current id in a short chain.
  // Descriptors are per 16-token plane; copy-on-write is per allocation
  // block (a 32-token block is planes 2b, 2b+1).
  std::vector<InjectDesc> descs;
  std::vector<int32_t> dseq, dblk, dnext;  // writer, plane id before copy-on-write, chain
  if (int64_t(c->desc_of_block.size()) < int64_t(c->num_blocks) * c->sub)
    c->desc_of_block.assign(int64_t(c->num_blocks) * c->sub, -1);
  std::vector<int32_t>& desc_of_block = c->desc_of_block;
  auto reset_scratch = [&]() {
    for (int32_t b : dblk) desc_of_block[b] = -1;
  };
  for (int32_t r = 0; r < n_runs; ++r) {
    const pkv_run& run = runs[r];
    pkv_status st = check_seq(c, run.seq);
    if (!st && (run.n_tokens < 0 || run.dst_pos < 0 || run.src_token < 0))
      st = fail(PKV_E_INVALID, "run %d has a negative field", r);
    if (st) {
      reset_scratch();
      return st;
    }
    if (run.n_tokens == 0) continue;
    const auto& table = c->tables[run.seq];
    const int64_t end = int64_t(run.dst_pos) + run.n_tokens;
    if (end > int64_t(table.size()) * c->bt)
      st = fail(PKV_E_RANGE, "run %d ends at %lld past the %lld reserved slots of seq %d", r,
                (long long)end, (long long)(int64_t(table.size()) * c->bt), run.seq);
    else if (end > max_pos)
      st = fail(PKV_E_RANGE, "run %d ends at %lld past the rotary table (%d)", r, (long long)end,
                max_pos);
    else if (run.src_token + run.n_tokens > src->n_tokens ||
             run.src_token + run.n_tokens > INT32_MAX)
      st = fail(PKV_E_RANGE, "run %d reads past the source store", r);
    if (st) {
      reset_scratch();
      return st;
    }
    // One 16-token plane at a time: look its descriptor up once, then fill
    // the run's slots in it.
    for (int32_t t0 = 0; t0 < run.n_tokens;) {
      const int32_t p0 = run.dst_pos + t0;
      const int32_t cb = table[p0 / c->bt];
      if (cb < 0) {
        reset_scratch();
        return fail(PKV_E_RANGE, "seq %d position %d lies in a block a window trim dropped",
                    run.seq, p0);
      }
      const int64_t plane = int64_t(cb) * c->sub + (p0 % c->bt) / kBlock;
      if (plane >= pool->num_blocks) {
        reset_scratch();
        return fail(PKV_E_RANGE, "block %d outside the pool", cb);
      }
      const int32_t blk = int32_t(plane);
      int32_t di = desc_of_block[blk];
      while (di >= 0 && dseq[di] != run.seq) di = dnext[di];
      if (di < 0) {
        di = int32_t(descs.size());
        InjectDesc d;
        d.phys_block = blk;
        d.pos_base = p0 - p0 % kBlock;
        for (int k = 0; k < kBlock; ++k) d.src[k] = -1;
        descs.push_back(d);
        dseq.push_back(run.seq);
        dblk.push_back(blk);
        dnext.push_back(desc_of_block[blk]);
        desc_of_block[blk] = di;
      }
      const int32_t n_here = std::min(run.n_tokens - t0, kBlock - p0 % kBlock);
      int32_t* slots = descs[di].src + p0 % kBlock;
      for (int32_t k = 0; k < n_here; ++k) {
        if (slots[k] >= 0) {
          reset_scratch();
          return fail(PKV_E_OVERLAP, "two tokens of this call target seq %d position %d",
                      run.seq, p0 + k);
        }
        slots[k] = int32_t(run.src_token + t0 + k);
      }
      t0 += n_here;
    }
  }
  reset_scratch();
  const size_t bytes = descs.size() * sizeof(InjectDesc);
  const bool launch = !descs.empty() && layer_end > layer_begin;
  if (launch) {
    if (!d_ws || ws_bytes < bytes)
      return fail(PKV_E_WORKSPACE, "inject workspace %zu bytes, need %zu", ws_bytes, bytes);
    if (reinterpret_cast<uintptr_t>(d_ws) & 15)
      return fail(PKV_E_WORKSPACE, "workspace must be 16-byte aligned");
  }
  pkv_src src_dev = *src;
  bool k_host = false, v_host = false;
  if (launch) {
    if (pkv_status st = resolve_source(src->k, "source K", &src_dev.k, &k_host)) return st;
    if (pkv_status st = resolve_source(src->v, "source V", &src_dev.v, &v_host)) return st;
  }
  // Copy-on-write, all-or-nothing: the written allocation blocks in order of
  // first touch, copies counted with the reference counts as they will be
  // when each block is reached.
  {
    std::vector<std::pair<int32_t, int64_t>> touched;  // (seq, block index)
    {
      const int64_t n_flags = int64_t(c->max_seqs) * c->max_blocks_per_seq;
      if (int64_t(c->touched_flag.size()) < n_flags) c->touched_flag.assign(n_flags, 0);
      for (size_t i = 0; i < descs.size(); ++i) {
        const int64_t idx = descs[i].pos_base / c->bt;
        uint8_t& f = c->touched_flag[int64_t(dseq[i]) * c->max_blocks_per_seq + idx];
        if (!f) {
          f = 1;
          touched.emplace_back(dseq[i], idx);
        }
      }
      for (const auto& si : touched)
        c->touched_flag[int64_t(si.first) * c->max_blocks_per_seq + si.second] = 0;
    }
    // Reference counts as they will be when each touched block is reached
    // (only shared blocks, ref > 1, need a copy or are tracked).
    std::unordered_map<int32_t, int32_t> refs_then;
    int64_t need = 0;
    for (const auto& si : touched) {
      const int32_t b = c->tables[si.first][si.second];
      if (c->ref[b] <= 1) continue;
      auto it = refs_then.find(b);
      const int32_t rc = it == refs_then.end() ? c->ref[b] : it->second;
      if (rc > 1) {
        ++need;
        refs_then[b] = rc - 1;
      }
    }
    if (need > c->fl_size)
      return fail(PKV_E_OOM, "copy-on-write needs %lld blocks, %d free", (long long)need,
                  c->fl_size);
    if ((need > 0 || !c->pending.empty()) &&
        int64_t(c->num_blocks) * c->sub > pool->num_blocks)
      return fail(PKV_E_INVALID, "block copies need every block of the cache (%d) inside the "
                  "pool (%d planes)", c->num_blocks, pool->num_blocks);
    for (const auto& si : touched) {
      const int32_t b = c->tables[si.first][si.second];
      if (c->ref[b] > 1) c->cow(si.first, si.second);
      else c->forget(b);  // written in place: no longer holds what its entry says
    }
    for (size_t i = 0; i < descs.size(); ++i) {
      const int64_t idx = descs[i].pos_base / c->bt;
      descs[i].phys_block = c->tables[dseq[i]][idx] * c->sub + (descs[i].pos_base % c->bt) / kBlock;
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!c->pending.empty())
    if (pkv_status st = flush_copies(c, *pool, s)) return st;
  if (launch) {
    // A few descriptors travel in the kernel arguments; more go through the
    // workspace by one copy.
    const bool inline_descs = descs.size() <= size_t(pkv::kInlineDescs);
    if (!inline_descs) {
      void* host = nullptr;
      if (pkv_status st = c->staging.acquire(bytes, &host)) return st;
      std::memcpy(host, descs.data(), bytes);
      if (pkv_status st = c->staging.upload(d_ws, bytes, s)) return st;
    }
    hipError_t e = pkv::launch_inject(
        *pool, src_dev, k_host || v_host,
        inline_descs ? nullptr : static_cast<const InjectDesc*>(d_ws),
        inline_descs ? descs.data() : nullptr, int(descs.size()), layer_begin, layer_end,
        rope_mode, d_cos, d_sin, s);
    if (e != hipSuccess) return hip_fail(e, "inject launch");
  }
  for (int32_t r = 0; r < n_runs; ++r) {
    const int64_t end = int64_t(runs[r].dst_pos) + runs[r].n_tokens;
    if (runs[r].n_tokens > 0) c->lens[runs[r].seq] = std::max(c->lens[runs[r].seq], end);
  }
  return ok();
}

// ---------------------------------------------------------------------------
// Append
// ---------------------------------------------------------------------------
pkv_status pkv_append_kv(const pkv_pool* pool, int32_t layer, const int32_t* d_tables,
                         int32_t table_stride, const int32_t* d_first_pos, int32_t n_seqs,
                         int32_t n_new, const void* d_k_new, const void* d_v_new,
                         int32_t new_dtype, int32_t rope_mode, const float* d_cos,
                         const float* d_sin, int32_t max_pos, void* stream) {
  if (pkv_status st = check_pool(pool)) return st;
  if (pkv_status st = check_input_dtype(pool, new_dtype, "new K/V")) return st;
  if (pkv_status st = check_rope(rope_mode, d_cos, d_sin, max_pos)) return st;
  if (layer < 0 || layer >= pool->n_layers) return fail(PKV_E_INVALID, "layer %d", layer);
  if (n_seqs < 0 || n_new < 0) return fail(PKV_E_INVALID, "negative count");
  if (n_seqs == 0 || n_new == 0) return ok();
  if (!d_tables || !d_first_pos || !d_k_new || !d_v_new || table_stride <= 0)
    return fail(PKV_E_INVALID, "null device argument or bad table stride");
  if ((reinterpret_cast<uintptr_t>(d_k_new) | reinterpret_cast<uintptr_t>(d_v_new)) & 15)
    return fail(PKV_E_INVALID, "k_new / v_new must be 16-byte aligned");
  hipError_t e = pkv::launch_append(*pool, layer, d_tables, table_stride, d_first_pos, n_seqs,
                                    n_new, d_k_new, d_v_new, new_dtype, rope_mode, d_cos, d_sin,
                                    max_pos, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return ok();
}

// ---------------------------------------------------------------------------
// Decode plan and attention
// ---------------------------------------------------------------------------
pkv_status pkv_decode_plan_create(const int64_t* lens, int32_t n_seqs, int32_t n_q_heads,
                                  int32_t n_kv_heads, int32_t head_dim, int32_t part_tokens,
                                  int32_t window, pkv_plan** out) {
  if (!out || n_seqs < 0 || (n_seqs > 0 && !lens)) return fail(PKV_E_INVALID, "bad arguments");
  if (n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads)
    return fail(PKV_E_INVALID, "n_q_heads must be a positive multiple of n_kv_heads");
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_E_UNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
  if (part_tokens < 0 || part_tokens % kBlock)
    return fail(PKV_E_INVALID, "part_tokens must be a non-negative multiple of 16");
  if (window < 0) return fail(PKV_E_INVALID, "negative window");
  // Each sequence attends to positions [lo, len): lo = len - window under a
  // sliding window, else 0.  Its ranges start at lo rounded down to a block.
  auto first_pos = [&](int64_t len) {
    return window > 0 ? std::max<int64_t>(0, len - window) : 0;
  };
  int64_t total = 0, total_blocks = 0, n_nonempty = 0;
  for (int32_t b = 0; b < n_seqs; ++b) {
    if (lens[b] < 0 || lens[b] > (int64_t(1) << 30))
      return fail(PKV_E_RANGE, "length %lld of sequence %d", (long long)lens[b], b);
    const int64_t span = lens[b] - first_pos(lens[b]) / kBlock * kBlock;
    total += span;
    total_blocks += blocks_for(span);
    n_nonempty += lens[b] > 0;
  }
  // Waves per workgroup: the waves of one workgroup share a token range,
  // taking its blocks in turn, so give each wave at least ~4 blocks.
  int32_t waves = 8;
  const int64_t avg_blocks = n_nonempty ? total_blocks / n_nonempty : 0;
  while (waves > 1 && avg_blocks < 4 * waves) waves /= 2;
  if (const char* env = std::getenv("PKV_DECODE_WAVES")) {
    const int w = std::atoi(env);
    if (w == 1 || w == 2 || w == 4 || w == 8) waves = w;
  }
  int32_t part = part_tokens;
  if (part == 0) {
    if (const char* env = std::getenv("PKV_PART_TOKENS")) part = std::atoi(env);
    if (part <= 0 || part % kBlock) {
      // Spread the work over ~2048 waves (8 per CU of 256): a sequence longer
      // than its share is split into several ranges merged afterwards.
      const int64_t wgs = std::max<int64_t>(1, 2048 / waves);
      const int64_t per = (total * n_kv_heads + wgs - 1) / wgs;
      const int64_t p = (per + kBlock - 1) / kBlock * kBlock;
      part = int32_t(std::min<int64_t>(1 << 30, std::max<int64_t>(int64_t(64) * waves, p)));
    }
  }
  pkv_plan* plan = new (std::nothrow) pkv_plan();
  if (!plan) return fail(PKV_E_INVALID, "out of host memory");
  plan->n_seqs = n_seqs;
  plan->n_q_heads = n_q_heads;
  plan->n_kv_heads = n_kv_heads;
  plan->head_dim = head_dim;
  plan->part_tokens = part;
  plan->waves = waves;
  int32_t slots = 0;
  for (int32_t b = 0; b < n_seqs; ++b) {
    const int64_t lo = first_pos(lens[b]);
    const int64_t start = lo / kBlock * kBlock;
    const int64_t n_items = (lens[b] - start + part - 1) / part;
    if (n_items <= 1) {
      // whole range in one item (an empty one included): final output
      plan->items.push_back(
          DecodeItem{b, int32_t(start), int32_t(lens[b] - start), -1, int32_t(lo), 1});
    } else {
      plan->merges.push_back(MergeSeq{b, slots, int32_t(n_items), 0});
      for (int64_t i = 0; i < n_items; ++i) {
        const int64_t t0 = start + i * part;
        const int64_t n = std::min<int64_t>(part, lens[b] - t0);
        plan->items.push_back(DecodeItem{b, int32_t(t0), int32_t(n), slots++, int32_t(lo),
                                         int32_t(i == n_items - 1)});
      }
    }
  }
  // Longest items first: the dispatcher starts workgroups in grid order, so
  // this approximates longest-processing-time-first scheduling.
  std::stable_sort(plan->items.begin(), plan->items.end(),
                   [](const DecodeItem& x, const DecodeItem& y) { return x.n_tokens > y.n_tokens; });
  plan->n_slots = slots;
  plan->newest.resize(size_t(n_seqs));
  for (int32_t b = 0; b < n_seqs; ++b) plan->newest[b] = int32_t(lens[b] - 1);
  size_t off = 0;
  plan->off_items = off;
  off = align_up(off + plan->items.size() * sizeof(DecodeItem), 256);
  plan->off_merges = off;
  off = align_up(off + plan->merges.size() * sizeof(MergeSeq), 256);
  plan->off_pos = off;
  off = align_up(off + plan->newest.size() * sizeof(int32_t), 256);
  plan->off_part_o = off;
  off = align_up(off + size_t(slots) * n_q_heads * head_dim * sizeof(float), 256);
  plan->off_part_ml = off;
  off = align_up(off + size_t(slots) * n_q_heads * 2 * sizeof(float), 256);
  plan->ws_bytes = std::max<size_t>(off, 256);
  *out = plan;
  return ok();
}

void pkv_decode_plan_destroy(pkv_plan* plan) { delete plan; }

int32_t pkv_decode_plan_items(const pkv_plan* plan) {
  return plan ? int32_t(plan->items.size()) : -1;
}

int32_t pkv_decode_plan_part_tokens(const pkv_plan* plan) {
  return plan ? plan->part_tokens : -1;
}

int32_t pkv_decode_plan_waves(const pkv_plan* plan) { return plan ? plan->waves : -1; }

size_t pkv_decode_workspace_bytes(const pkv_plan* plan) { return plan ? plan->ws_bytes : 0; }

}  // extern "C"

namespace {

// Whether the plan's work list travels in the decode kernel's arguments
// instead of the workspace: at most kInlineItems items, no split sequence
// (the merge reads the workspace), and too few workgroups for the launch
// that appends in a launch of its own (it reads the newest positions from
// the workspace).  Its launches then need no upload.
bool plan_inline(const pkv_plan* plan) {
  return plan->items.size() <= size_t(pkv::kInlineItems) && plan->merges.empty() &&
         int64_t(plan->items.size()) * plan->n_kv_heads < int64_t(16) * pkv::device_cus();
}

}  // namespace

extern "C" {

pkv_status pkv_decode_plan_upload(pkv_plan* plan, void* d_ws, size_t ws_bytes, void* stream) {
  if (!plan) return fail(PKV_E_INVALID, "null plan");
  if (!d_ws || ws_bytes < plan->ws_bytes)
    return fail(PKV_E_WORKSPACE, "decode workspace %zu bytes, need %zu", ws_bytes,
                plan->ws_bytes);
  if (reinterpret_cast<uintptr_t>(d_ws) & 255)
    return fail(PKV_E_WORKSPACE, "workspace must be 256-byte aligned");
  const size_t bytes = plan->off_part_o;
  if (bytes == 0 || plan_inline(plan)) return ok();
  void* host = nullptr;
  if (pkv_status st = plan->staging.acquire(bytes, &host)) return st;
  std::memset(host, 0, bytes);
  std::memcpy(static_cast<char*>(host) + plan->off_items, plan->items.data(),
              plan->items.size() * sizeof(DecodeItem));
  std::memcpy(static_cast<char*>(host) + plan->off_merges, plan->merges.data(),
              plan->merges.size() * sizeof(MergeSeq));
  std::memcpy(static_cast<char*>(host) + plan->off_pos, plan->newest.data(),
              plan->newest.size() * sizeof(int32_t));
  if (pkv_status st = plan->staging.upload(d_ws, bytes, static_cast<hipStream_t>(stream)))
    return st;
  return ok();
}

}  // extern "C"

namespace {

// Fused append of each sequence's newest token (null new_k: none).
struct NewToken {
  const void* k = nullptr;
  const void* v = nullptr;
  int32_t rope_mode = PKV_ROPE_NONE;
  const float* cos = nullptr;
  const float* sin = nullptr;
  int32_t max_pos = 0;
};

// upload_plan: the workspace is the library's static scratch, and the plan's
// work list is copied into it on `stream` before the launch (the
// allocation-free entry point); otherwise the caller uploaded the plan.
pkv_status decode_common(const pkv_plan* plan, const pkv_pool* pool, int32_t layer,
                         const void* d_q, int32_t q_dtype, float scale, const int32_t* d_tables,
                         int32_t table_stride, const NewToken& nt, float* d_out, float* d_lse,
                         void* d_ws, size_t ws_bytes, void* stream, bool upload_plan = false) {
  if (!plan) return fail(PKV_E_INVALID, "null plan");
  if (pkv_status st = check_pool(pool)) return st;
  if (pkv_status st = check_input_dtype(pool, q_dtype, "q")) return st;
  if (layer < 0 || layer >= pool->n_layers) return fail(PKV_E_INVALID, "layer %d", layer);
  if (pool->n_kv_heads != plan->n_kv_heads || pool->head_dim != plan->head_dim)
    return fail(PKV_E_INVALID, "plan and pool disagree on KV heads or head_dim");
  if (pool->dtype == PKV_FP8E4M3 && plan->n_q_heads / plan->n_kv_heads > 64)
    return fail(PKV_E_UNSUPPORTED, "FP8E4M3 decode supports up to 64 query heads per KV head");
  if (nt.k) {
    if (pkv_status st = check_rope(nt.rope_mode, nt.cos, nt.sin, nt.max_pos)) return st;
    if (!nt.v) return fail(PKV_E_INVALID, "null v_new");
    if ((reinterpret_cast<uintptr_t>(nt.k) | reinterpret_cast<uintptr_t>(nt.v)) & 15)
      return fail(PKV_E_INVALID, "k_new / v_new must be 16-byte aligned");
    if (nt.rope_mode != PKV_ROPE_NONE)
      for (const DecodeItem& it : plan->items)
        if (it.last && it.n_tokens > 0 && int64_t(it.t_begin) + it.n_tokens > nt.max_pos)
          return fail(PKV_E_RANGE, "position %lld of sequence %d has no rotary row (max_pos %d)",
                      (long long)(int64_t(it.t_begin) + it.n_tokens - 1), it.seq, nt.max_pos);
  }
  if (plan->n_seqs == 0) return ok();
  if (!d_q || !d_out || !d_tables) return fail(PKV_E_INVALID, "null device argument");
  if (reinterpret_cast<uintptr_t>(d_q) & 15) return fail(PKV_E_INVALID, "q must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(d_out) & 15)
    return fail(PKV_E_INVALID, "out must be 16-byte aligned");
  int64_t max_blocks = 0;
  for (const DecodeItem& it : plan->items)
    max_blocks = std::max<int64_t>(max_blocks, blocks_for(int64_t(it.t_begin) + it.n_tokens));
  if (table_stride <= 0 || max_blocks > table_stride)
    return fail(PKV_E_RANGE, "table_stride %d smaller than %lld blocks", table_stride,
                (long long)max_blocks);
  if (!d_ws || ws_bytes < plan->ws_bytes)
    return fail(PKV_E_WORKSPACE, "decode workspace %zu bytes, need %zu", ws_bytes,
                plan->ws_bytes);
  if (int64_t(plan->items.size()) * pool->n_kv_heads > INT32_MAX)
    return fail(PKV_E_UNSUPPORTED, "%zu work items x %d KV heads exceed one launch",
                plan->items.size(), pool->n_kv_heads);
  char* ws = static_cast<char*>(d_ws);
  pkv::DecodeArgs a{};
  a.q = d_q;
  a.q_dtype = q_dtype;
  a.n_q_heads = plan->n_q_heads;
  a.scale = scale > 0.f ? scale : float(1.0 / std::sqrt(double(plan->head_dim)));
  a.tables = d_tables;
  a.table_stride = table_stride;
  a.items = reinterpret_cast<const DecodeItem*>(ws + plan->off_items);
  const bool inline_items = plan_inline(plan);
  a.h_items = inline_items ? plan->items.data() : nullptr;
  a.n_items = int(plan->items.size());
  a.merges = reinterpret_cast<const MergeSeq*>(ws + plan->off_merges);
  a.n_merges = int(plan->merges.size());
  a.waves = plan->waves;
  a.part_o = reinterpret_cast<float*>(ws + plan->off_part_o);
  a.part_ml = reinterpret_cast<float*>(ws + plan->off_part_ml);
  a.out = d_out;
  a.lse = d_lse;
  a.new_k = nt.k;
  a.new_v = nt.v;
  a.rope_mode = nt.rope_mode;
  a.cos_t = nt.cos;
  a.sin_t = nt.sin;
  a.max_pos = nt.max_pos;
  a.put_pos = reinterpret_cast<const int32_t*>(ws + plan->off_pos);
  a.n_seqs = plan->n_seqs;
  a.timed = !upload_plan;
  int variant = 0;
  if (const char* env = std::getenv("PKV_DECODE_KERNEL")) variant = std::atoi(env);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (upload_plan && !inline_items) {
    // from the plan's own host memory: the runtime stages these small copies
    hipError_t e = hipSuccess;
    if (!plan->items.empty())
      e = hipMemcpyAsync(ws + plan->off_items, plan->items.data(),
                         plan->items.size() * sizeof(DecodeItem), hipMemcpyHostToDevice, hs);
    if (e == hipSuccess && !plan->merges.empty())
      e = hipMemcpyAsync(ws + plan->off_merges, plan->merges.data(),
                         plan->merges.size() * sizeof(MergeSeq), hipMemcpyHostToDevice, hs);
    if (e == hipSuccess && !plan->newest.empty())
      e = hipMemcpyAsync(ws + plan->off_pos, plan->newest.data(),
                         plan->newest.size() * sizeof(int32_t), hipMemcpyHostToDevice, hs);
    if (e != hipSuccess) return hip_fail(e, "work list copy into the static scratch");
  }
  hipError_t e = pkv::launch_decode(*pool, layer, a, variant, hs);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

}  // namespace

extern "C" {

pkv_status pkv_decode_attention(const pkv_plan* plan, const pkv_pool* pool, int32_t layer,
                                const void* d_q, int32_t q_dtype, float scale,
                                const int32_t* d_tables, int32_t table_stride, float* d_out,
                                float* d_lse, void* d_ws, size_t ws_bytes, void* stream) {
  return decode_common(plan, pool, layer, d_q, q_dtype, scale, d_tables, table_stride,
                       NewToken{}, d_out, d_lse, d_ws, ws_bytes, stream);
}

pkv_status pkv_append_decode_attention(const pkv_plan* plan, const pkv_pool* pool, int32_t layer,
                                       const void* d_q, int32_t q_dtype, float scale,
                                       const int32_t* d_tables, int32_t table_stride,
                                       const void* d_k_new, const void* d_v_new,
                                       int32_t rope_mode, const float* d_cos,
                                       const float* d_sin, int32_t max_pos, float* d_out,
                                       float* d_lse, void* d_ws, size_t ws_bytes, void* stream) {
  // (a plan of no sequences has no rows to read: its device arguments may be null)
  if (plan && plan->n_seqs > 0 && (!d_k_new || !d_v_new))
    return fail(PKV_E_INVALID, "null k_new or v_new");
  NewToken nt;
  nt.k = d_k_new;
  nt.v = d_v_new;
  nt.rope_mode = rope_mode;
  nt.cos = d_cos;
  nt.sin = d_sin;
  nt.max_pos = max_pos;
  return decode_common(plan, pool, layer, d_q, q_dtype, scale, d_tables, table_stride, nt, d_out,
                       d_lse, d_ws, ws_bytes, stream);
}

pkv_status pkv_append_decode_attention_noalloc(const pkv_plan* plan, const pkv_pool* pool,
                                               int32_t layer, const void* d_q, int32_t q_dtype,
                                               float scale, const int32_t* d_tables,
                                               int32_t table_stride, const void* d_k_new,
                                               const void* d_v_new, int32_t rope_mode,
                                               const float* d_cos, const float* d_sin,
                                               int32_t max_pos, float* d_out, float* d_lse,
                                               void* stream) {
  if (!plan) return fail(PKV_E_INVALID, "null plan");
  if (plan->ws_bytes > pkv::kScratchBytes)
    return fail(PKV_E_WORKSPACE,
                "the plan needs %zu bytes of workspace, more than the %zu-byte static scratch "
                "of the allocation-free call; use pkv_append_decode_attention with a workspace",
                plan->ws_bytes, pkv::kScratchBytes);
  if (plan->n_seqs > 0 && (!d_k_new || !d_v_new))
    return fail(PKV_E_INVALID, "null k_new or v_new");
  void* ws = nullptr;
  const hipError_t e = pkv::scratch_address(&ws);
  if (e != hipSuccess) return hip_fail(e, "address of the static scratch");
  NewToken nt;
  nt.k = d_k_new;
  nt.v = d_v_new;
  nt.rope_mode = rope_mode;
  nt.cos = d_cos;
  nt.sin = d_sin;
  nt.max_pos = max_pos;
  return decode_common(plan, pool, layer, d_q, q_dtype, scale, d_tables, table_stride, nt, d_out,
                       d_lse, ws, pkv::kScratchBytes, stream, true);
}

pkv_status pkv_kernel_timing(int32_t enable) {
  pkv::set_kernel_timing(enable != 0);
  return ok();
}

int32_t pkv_kernel_times(float* ms_out, int32_t max_n) {
  if (max_n < 0 || (max_n > 0 && !ms_out)) return fail(PKV_E_INVALID, "bad output buffer");
  hipError_t e = hipSuccess;
  const int n = pkv::collect_kernel_times(ms_out, max_n, &e);
  if (e != hipSuccess) return hip_fail(e, "kernel timing events");
  return n;
}

pkv_status pkv_bw_probe(const void* d_src, size_t n_bytes, void* d_sink, void* stream) {
  if (!d_src || !d_sink || n_bytes % 16 || (reinterpret_cast<uintptr_t>(d_src) & 15))
    return fail(PKV_E_INVALID, "bad probe arguments");
  hipError_t e = pkv::launch_bw_probe(d_src, n_bytes, d_sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "probe launch");
  return ok();
}

}  // extern "C"
