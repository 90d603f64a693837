// HIP kernels of libpkv for MI355X (gfx950, CDNA4, wave64).
//
//   inject_rope_kernel     write side: one workgroup per (destination block,
//                          layers); rotates stored pre-RoPE keys to their
//                          destination positions and scatters K/V into the
//                          block's planes ("InferScale" §3 scatter copy through
//                          the slot mapping, §3.3 and §5.1 chunked RoPE).  In
//                          append mode it writes new tokens (the per-step
//                          append of "InferScale" §2 / "LLM Inference: KV
//                          Caching", "The fix"), one workgroup per (sequence,
//                          block touched, group of KV heads).
//   decode_mfma_kernel     read side: one workgroup per (token range, KV head),
//                          its waves taking interleaved blocks; QK^T and PV of
//                          the whole GQA group on MFMA tiles, online softmax
//                          in registers, the waves' states merged in LDS.  It
//                          can also append each sequence's newest token first
//                          (one launch per decode step and layer).
//   decode_valu_kernel     generic read side for any dtype / group size.
//   decode_merge_kernel    log-sum-exp merge of ranges of one sequence that
//                          ran on different workgroups.
//   copy_blocks_kernel     copy-on-write: duplicates whole blocks (every layer,
//                          K and V) before a sequence writes into a block it
//                          shares ("LLM Inference: KV Caching", "Paged
//                          attention"; "Latency Optimization > KV Cache
//                          Management", copy-on-write for beams).
//   bw_probe_kernel        streaming read for the same-run HBM ceiling.
//
// Pool plane layouts (see include/pkv.h): K plane = d/X chunks x 16 tokens x X
// dims (X = 16 bytes / element), V plane = d dims x 16 tokens.
//
// This file is compiled with -ffp-contract=off: the key rotation is two
// float32 products and one float32 add/subtract, never fused, so the stored
// keys are reproducible bit for bit.  Where a fused multiply-add is wanted it
// is written as fmaf().

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

#include "pkv_internal.h"

// Workspace of pkv_append_decode_attention_noalloc (work list, merge list,
// partial softmax states of split sequences).  Each device the library runs
// on holds its own copy until the process ends.  Host code never uses this
// name as an address: pkv::scratch_address() gives the device address.
static __device__ __align__(256) unsigned char scratch[pkv::kScratchBytes];

namespace pkv {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Element formats
// ---------------------------------------------------------------------------
template <int DT> struct Fmt;
template <> struct Fmt<PKV_F32> {
  typedef float T;
  static constexpr int kBytes = 4;
  __device__ static float to_f32(float x) { return x; }
  __device__ static float from_f32(float x) { return x; }
};
template <> struct Fmt<PKV_BF16> {
  typedef uint16_t T;
  static constexpr int kBytes = 2;
  __device__ static float to_f32(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }
  // Round to nearest, ties to even; a NaN becomes the quiet NaN of its sign
  // (0x7FC0 / 0xFFC0), whatever its payload.
  __device__ static uint16_t from_f32(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t(((u >> 16) & 0x8000u) | 0x7FC0u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
  }
};
template <> struct Fmt<PKV_F16> {
  typedef uint16_t T;
  static constexpr int kBytes = 2;
  __device__ static float to_f32(uint16_t x) { return float(__builtin_bit_cast(_Float16, x)); }
  // Hardware conversion under the default round-to-nearest-even mode.
  __device__ static uint16_t from_f32(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
  }
};

// OCP E4M3: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; largest
// finite value 448 (0x7E), 0x7F/0xFF are NaN, no infinities.
template <> struct Fmt<PKV_FP8E4M3> {
  typedef uint8_t T;
  static constexpr int kBytes = 1;
  __device__ static float to_f32(uint8_t b) {
    const uint32_t e = (b >> 3) & 0xF, m = b & 7;
    float v = e == 0 ? float(m) * 0.001953125f  // m * 2^-9
                     : __uint_as_float(((e + 120u) << 23) | (m << 20));
    if ((b & 0x7F) == 0x7F) v = __uint_as_float(0x7fc00000u);
    return (b & 0x80) ? -v : v;
  }
  // Round to nearest, ties to even; magnitudes that would round beyond 448
  // saturate to 448; NaN stays NaN (0x7F with its sign).  CDNA4's packed
  // f32 -> E4M3 conversion rounds to nearest even but turns out-of-range
  // values into the NaN code, so the value is clamped to +-448 first; a check
  // on the GPU over every float32 bit pattern found this equal to the
  // rounding rule above for every non-NaN input.
  __device__ static uint8_t from_f32(float x) {
    if (x != x) return uint8_t(((__float_as_uint(x) >> 24) & 0x80u) | 0x7Fu);
    const float c = fminf(fmaxf(x, -448.0f), 448.0f);
    return uint8_t(__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFF);
  }
};

// 16-byte global access helpers.
__device__ inline uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Streaming (non-temporal) loads for data read exactly once: the cached K/V
// of a decode step.  The hint keeps them from displacing reusable lines.
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
__device__ inline uint4 ld16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline uint2 ld8_stream(const void* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}
// Streaming store for data written once and not read back soon.
__device__ inline void st16_stream(void* p, uint4 v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}
__device__ inline void st8_stream(void* p, uint2 v) {
  const u32x2_t w = {v.x, v.y};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t*>(p));
}
__device__ inline void st4_stream(void* p, uint32_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
}
__device__ inline uint32_t ld4_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// A 16x16 MFMA result holds each column in lanes c, c + 16, c + 32 and
// c + 48.  These combine a value over those four lanes, leaving the result in
// all four, with CDNA4's lane swaps between 16-lane rows and 32-lane halves
// (register to register: no LDS traffic and no wait on it).  Each step adds
// or compares the same two values in every lane of a pair, so all four lanes
// get bit-identical results.
__device__ inline float cols_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float cols_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The X elements of a 16-byte chunk as float32.
template <int DT>
__device__ inline void unpack16(const uint4& c, float* f) {
  typedef typename Fmt<DT>::T T;
  constexpr int X = 16 / Fmt<DT>::kBytes;
  T v[X];
  *reinterpret_cast<uint4*>(v) = c;
#pragma unroll
  for (int e = 0; e < X; ++e) f[e] = Fmt<DT>::to_f32(v[e]);
}

// Rotation of float32 values, two products and one add/subtract each, never
// fused (y0 = x0*c - x1*s, y1 = x0*s + x1*c).  PAIRS: element e pairs with
// e+1 inside the run (pair index (first_dim + e) / 2); HALVES: element e of
// `a` pairs with element e of `b` (pair index first_dim + e).
template <int N>
__device__ inline void rot_pairs_f(float* f, int first_dim, const float* cr, const float* sr) {
#pragma unroll
  for (int e = 0; e < N; e += 2) {
    const int i = (first_dim + e) >> 1;
    const float c = cr[i], s = sr[i];
    const float x0 = f[e], x1 = f[e + 1];
    f[e] = x0 * c - x1 * s;
    f[e + 1] = x0 * s + x1 * c;
  }
}
template <int N>
__device__ inline void rot_halves_f(float* a, float* b, int first_dim, const float* cr,
                                    const float* sr) {
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const int i = first_dim + e;
    const float c = cr[i], s = sr[i];
    const float x0 = a[e], x1 = b[e];
    a[e] = x0 * c - x1 * s;
    b[e] = x0 * s + x1 * c;
  }
}

// N float32 values stored in the pool format PDT; a quantised (fp8) pool
// stores e4m3(x / scale), the division correctly rounded in float32.
template <int PDT, int N>
struct Packed {
  typedef typename Fmt<PDT>::T T;
  T v[N];
  __device__ void set(const float* f, float scale) {
#pragma unroll
    for (int e = 0; e < N; ++e)
      v[e] = Fmt<PDT>::from_f32(PDT == PKV_FP8E4M3 ? f[e] / scale : f[e]);
  }
};
template <int PDT, int N>
__device__ inline void store_packed(void* dst, const Packed<PDT, N>& pk) {
  constexpr int B = N * Fmt<PDT>::kBytes;
  static_assert(B == 16 || B == 8, "16- or 8-byte pieces");
  if constexpr (B == 16) st16_stream(dst, *reinterpret_cast<const uint4*>(pk.v));
  else st8_stream(dst, *reinterpret_cast<const uint2*>(pk.v));
}

// ---------------------------------------------------------------------------
// Inject: one workgroup per (destination block descriptor, layer)
// ---------------------------------------------------------------------------
struct InjectParams {
  char* pool_k;
  char* pool_v;
  int64_t p_layer, p_block, p_head;  // bytes
  int n_kv_heads;
  const float* k_scale;              // quantised pools only: [layers][heads], or
  const float* v_scale;              // [layers][num_blocks][heads] (scale_mode 1)
  int scale_mode;
  const char* src_k;
  const char* src_v;
  int64_t s_layer, s_token;          // bytes
  const InjectDesc* descs;
  int layer_begin;
  int layer_end;
  int layers_per_wg;
  int rope_mode;
  const float* cos_t;
  const float* sin_t;
  // Append mode (app_first non-null): workgroup x = (sequence b, i) makes its
  // own descriptor, block i of the blocks holding positions
  // [first_pos[b], first_pos[b] + app_n_new), whose tokens are source rows
  // b * app_n_new + (position - first_pos[b]); workgroup y takes KV heads
  // y * HG ... of the single layer layer_begin.
  const int32_t* app_first;
  const int32_t* app_tables;
  int app_stride;
  int app_n_new;
  int app_blocks;                    // blocks one sequence's new tokens can touch
  int num_blocks;
  int max_pos;
  // Calls of at most kInlineDescs descriptors carry them here, in the kernel
  // arguments, instead of a device copy (n_inline > 0; descs unused).
  int n_inline;
  InjectDesc inline_descs[kInlineDescs];
};

constexpr int kInjectThreads = 256;

// One workgroup of 4 waves per (destination block, group of layers).  The
// block's 16 rotary rows are staged in LDS once.  Each wave then takes whole
// KV heads (heads wave, wave + 4, ... of every layer of the group): for each
// (layer, head) every lane reads UPH (token, source chunk pair) units -- the
// two 16-byte K and V chunks of a source row (format SDT) -- rotates K in
// float32 and stores it into the K plane in the pool format PDT; V goes
// through the wave's own LDS tile (already in PDT) to be written
// dimension-major.  A wave touches only its own tile, so only the wave's own
// ordering is needed there, no workgroup barrier.  Source chunk pairs are
// (c0, c0 + C/2) so that the halves pairing finds both partners in one unit.
// The lanes walk a head's units chunk fastest: each load instruction takes
// whole 128-byte lines of 8 token rows (bf16 d = 128: the first or second
// half of each row), which measured 1.28x faster than token fastest (64 bytes
// of 16 rows per instruction) on the top-8 injection, and suits PCIe reads
// from a pinned host store as well.  PF: the next (layer, head)'s loads are
// issued before the current one is processed.
template <int SDT, int PDT, int D, int HG, bool PF>
__global__ __launch_bounds__(kInjectThreads) void inject_rope_kernel(InjectParams p) {
  typedef typename Fmt<PDT>::T TP;
  constexpr int ES = Fmt<SDT>::kBytes, EP = Fmt<PDT>::kBytes;
  constexpr int XS = 16 / ES;                 // source elements per 16-byte chunk
  constexpr int XP = 16 / EP;                 // pool elements per 16-byte chunk
  constexpr int CS = D / XS;                  // source chunks per row
  constexpr int UNITS = kBlock * (CS / 2);    // (token, chunk pair) units per head
  constexpr int VPIECES = D * (kBlock / XP);  // 16-byte pieces of a V plane
  constexpr int NWAVE = kInjectThreads / 64;
  constexpr int UPH = UNITS / 64;             // units per lane and head
  constexpr int VPH = VPIECES / 64;           // V pieces per lane and head
  static_assert(XP % XS == 0, "a source chunk lands inside one pool chunk");
  static_assert(UNITS % 64 == 0 && VPIECES % 64 == 0, "whole waves per head");
  __shared__ TP vtile[NWAVE][kBlock][D];
  __shared__ float cs[kBlock][D];
  __shared__ InjectDesc desc;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  int h_begin = 0, h_end = p.n_kv_heads;
  int l0 = p.layer_begin + blockIdx.y * p.layers_per_wg;
  int l1 = min(l0 + p.layers_per_wg, p.layer_end);
  if (p.app_first == nullptr) {
    if (threadIdx.x < sizeof(InjectDesc) / 4)
      reinterpret_cast<int32_t*>(&desc)[threadIdx.x] =
          reinterpret_cast<const int32_t*>(p.n_inline > 0 ? &p.inline_descs[blockIdx.x]
                                                          : &p.descs[blockIdx.x])[threadIdx.x];
  } else {
    const int b = blockIdx.x / p.app_blocks;
    const int first = p.app_first[b];
    const int lo = max(first, 0), hi = first + p.app_n_new;  // positions written
    const int lb = lo / kBlock + (blockIdx.x - b * p.app_blocks);
    if (threadIdx.x < kBlock) {
      const int pos = lb * kBlock + threadIdx.x;
      const bool in = pos >= lo && pos < hi && (p.rope_mode == PKV_ROPE_NONE || pos < p.max_pos);
      desc.src[threadIdx.x] = in ? b * p.app_n_new + (pos - first) : -1;
    } else if (threadIdx.x == kBlock) {
      int blk = -1;
      if (lo < hi && lb * kBlock < hi && lb < p.app_stride)
        blk = p.app_tables[int64_t(b) * p.app_stride + lb];
      desc.phys_block = blk >= 0 && blk < p.num_blocks ? blk : -1;
      desc.pos_base = lb * kBlock;
    }
    h_begin = blockIdx.y * HG;
    h_end = min(h_begin + HG, p.n_kv_heads);
    l0 = p.layer_begin;
    l1 = l0 + 1;
  }
  __syncthreads();
  if (p.app_first != nullptr) {
    bool any = desc.phys_block >= 0;
    bool some = false;
#pragma unroll
    for (int t = 0; t < kBlock; ++t) some |= desc.src[t] >= 0;
    if (!(any && some)) return;  // the same for every thread: nothing to write here
  }
  if (p.rope_mode != PKV_ROPE_NONE) {
    for (int w = threadIdx.x; w < kBlock * (D / 2); w += kInjectThreads) {
      const int t = w / (D / 2), i = w - t * (D / 2);
      if (desc.src[t] < 0) continue;
      const size_t at = size_t(desc.pos_base + t) * (D / 2) + i;
      cs[t][i] = p.cos_t[at];
      cs[t][D / 2 + i] = p.sin_t[at];
    }
  }
  bool full = true;
#pragma unroll
  for (int t = 0; t < kBlock; ++t) full &= desc.src[t] >= 0;
  __syncthreads();

  // this wave's heads h_begin + wave + NWAVE k, for every layer of the group
  const int span = h_end - h_begin;
  const int heads_here = span > wave ? (span - wave + NWAVE - 1) / NWAVE : 0;
  const int n_iter = (l1 - l0) * heads_here;
  auto unit_tc = [&](int u, int& t, int& c0) {
    const int r = lane + 64 * u;
    t = r / (CS / 2);
    c0 = r % (CS / 2);
  };
  // loads of iteration `it`: per unit, K chunks c0 and c0 + C/2, then V's
  auto issue = [&](int it, uint4 (&b)[UPH][4]) {
    const int layer = l0 + it / heads_here;
    const int h = h_begin + wave + NWAVE * (it % heads_here);
    const char* sk = p.src_k + layer * p.s_layer;
    const char* sv = p.src_v + layer * p.s_layer;
#pragma unroll
    for (int u = 0; u < UPH; ++u) {
      int t, c0;
      unit_tc(u, t, c0);
      const int src = desc.src[t];
      if (src >= 0) {
        const int64_t row = int64_t(src) * p.s_token + int64_t(h) * D * ES;
        b[u][0] = ld16_stream(sk + row + c0 * 16);
        b[u][1] = ld16_stream(sk + row + (c0 + CS / 2) * 16);
        b[u][2] = ld16_stream(sv + row + c0 * 16);
        b[u][3] = ld16_stream(sv + row + (c0 + CS / 2) * 16);
      }
    }
  };
  auto process = [&](int it, const uint4 (&b)[UPH][4]) {
    const int layer = l0 + it / heads_here;
    const int h = h_begin + wave + NWAVE * (it % heads_here);
    char* kplane = p.pool_k + layer * p.p_layer + int64_t(desc.phys_block) * p.p_block +
                   int64_t(h) * p.p_head;
    char* vplane = p.pool_v + layer * p.p_layer + int64_t(desc.phys_block) * p.p_block +
                   int64_t(h) * p.p_head;
    // the scales of this (layer, head), or of this (layer, block, head)
    const int64_t si = p.scale_mode == 1
                           ? (int64_t(layer) * p.num_blocks + desc.phys_block) * p.n_kv_heads + h
                           : int64_t(layer) * p.n_kv_heads + h;
#pragma unroll
    for (int u = 0; u < UPH; ++u) {
      int t, c0;
      unit_tc(u, t, c0);
      if (desc.src[t] < 0) continue;
      const int j0 = c0 * XS, j1 = (c0 + CS / 2) * XS;  // first dims of the two chunks
      float kl[XS], kh[XS];
      unpack16<SDT>(b[u][0], kl);
      unpack16<SDT>(b[u][1], kh);
      if (p.rope_mode == PKV_ROPE_PAIRS) {
        rot_pairs_f<XS>(kl, j0, cs[t], cs[t] + D / 2);
        rot_pairs_f<XS>(kh, j1, cs[t], cs[t] + D / 2);
      } else if (p.rope_mode == PKV_ROPE_HALVES) {
        rot_halves_f<XS>(kl, kh, j0, cs[t], cs[t] + D / 2);
      }
      const float ksc = PDT == PKV_FP8E4M3 ? p.k_scale[si] : 1.f;
      Packed<PDT, XS> pk;
      pk.set(kl, ksc);
      store_packed(kplane + (((j0 / XP) * kBlock + t) * XP + j0 % XP) * EP, pk);
      pk.set(kh, ksc);
      store_packed(kplane + (((j1 / XP) * kBlock + t) * XP + j1 % XP) * EP, pk);
      if constexpr (SDT == PDT) {
        *reinterpret_cast<uint4*>(&vtile[wave][t][j0]) = b[u][2];
        *reinterpret_cast<uint4*>(&vtile[wave][t][j1]) = b[u][3];
      } else {
        const float vsc = p.v_scale[si];
        float vf[XS];
        Packed<PDT, XS> pv;
        unpack16<SDT>(b[u][2], vf);
        pv.set(vf, vsc);
        *reinterpret_cast<uint2*>(&vtile[wave][t][j0]) = *reinterpret_cast<const uint2*>(pv.v);
        unpack16<SDT>(b[u][3], vf);
        pv.set(vf, vsc);
        *reinterpret_cast<uint2*>(&vtile[wave][t][j1]) = *reinterpret_cast<const uint2*>(pv.v);
      }
    }
    // the tile is written and read by lanes of this wave only
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // V plane dimension-major, XP tokens per 16-byte piece; a piece with
    // slots this call does not write keeps their old contents.
#pragma unroll
    for (int v = 0; v < VPH; ++v) {
      const int r = lane + 64 * v;
      const int j = r / (kBlock / XP);
      const int t0 = (r % (kBlock / XP)) * XP;
      char* dst = vplane + (int64_t(j) * kBlock + t0) * EP;
      TP out[XP];
      bool need_old = false, any = full;
      if (!full) {
#pragma unroll
        for (int e = 0; e < XP; ++e) {
          need_old |= desc.src[t0 + e] < 0;
          any |= desc.src[t0 + e] >= 0;
        }
      }
      if (!any) continue;  // no slot of this piece is written
      if (need_old) *reinterpret_cast<uint4*>(out) = ld16(dst);
#pragma unroll
      for (int e = 0; e < XP; ++e)
        if (desc.src[t0 + e] >= 0) out[e] = vtile[wave][t0 + e][j];
      st16_stream(dst, *reinterpret_cast<uint4*>(out));
    }
    // the tile's reads are done before the next iteration writes it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  uint4 b0[UPH][4], b1[UPH][4];
  if constexpr (PF) {
    if (n_iter > 0) issue(0, b0);
    for (int it = 0; it < n_iter; it += 2) {
      if (it + 1 < n_iter) issue(it + 1, b1);
      process(it, b0);
      if (it + 1 < n_iter) {
        if (it + 2 < n_iter) issue(it + 2, b0);
        process(it + 1, b1);
      }
    }
  } else {
    for (int it = 0; it < n_iter; ++it) {
      issue(it, b0);
      process(it, b0);
    }
  }
}

// One token's V element j of one head, stored at slot `tin` of the V plane
// (dimension-major: [dim][slot]); a quantised pool stores e4m3(v / vsc).
template <int SDT, int PDT>
__device__ inline void put_v_elem(const char* vin, char* vplane, int tin, int j, float vsc) {
  typedef typename Fmt<SDT>::T TS;
  typedef typename Fmt<PDT>::T TP;
  const TS v = reinterpret_cast<const TS*>(vin)[j];
  TP out;
  if constexpr (SDT == PDT) {
    out = v;
  } else {
    out = Fmt<PDT>::from_f32(Fmt<SDT>::to_f32(v) / vsc);
  }
  reinterpret_cast<TP*>(vplane)[j * kBlock + tin] = out;
}

// ---------------------------------------------------------------------------
// Decode: common parameters
// ---------------------------------------------------------------------------
struct DecodeParams {
  const char* pool_k;
  const char* pool_v;
  int64_t p_layer, p_block, p_head;  // bytes
  int num_blocks;
  int n_kv_heads;
  int n_q_heads;
  int group;                         // n_q_heads / n_kv_heads
  const char* q;
  float scale_log2;                  // scale * log2(e)
  const int32_t* tables;
  int table_stride;
  const DecodeItem* items;
  int n_items;
  int chunk;                         // items per chunk of the launch order
  float* part_o;
  float* part_ml;
  float* out;
  float* lse;
  const float* k_scale;              // quantised pools only: this layer's [heads]
  const float* v_scale;              // scales, or its [num_blocks][heads] (scale_mode 1)
  int scale_mode;
  // Fused append (new_k null: none): rows [seq][n_kv_heads][D] in the
  // query's format; each sequence's token goes to position len - 1.
  const char* new_k;
  const char* new_v;
  int rope_mode;
  const float* cos_t;
  const float* sin_t;
  int max_pos;
  // The work list itself when it travels in the kernel arguments (items
  // null): plans of at most kInlineItems items.
  DecodeItem inline_items[kInlineItems];
};

// Work item i of the launch: from the device work list, or from the kernel
// arguments.  Both are read through the constant address space, so that the
// (wave-uniform) item comes in by scalar loads and its fields stay scalar:
// the work list is not written during the launch, and the kernel's first
// argument, DecodeParams, starts at offset 0 of the kernel-argument segment.
__device__ inline DecodeItem decode_item(const DecodeParams& p, int i) {
  typedef const __attribute__((address_space(4))) char* ConstBytes;
  typedef const __attribute__((address_space(4))) int32_t* ConstWords;
  const ConstBytes list = p.items ? (ConstBytes)p.items
                                  : (ConstBytes)__builtin_amdgcn_kernarg_segment_ptr() +
                                        offsetof(DecodeParams, inline_items);
  const ConstWords w = (ConstWords)(list + int64_t(i) * sizeof(DecodeItem));
  static_assert(sizeof(DecodeItem) == 6 * sizeof(int32_t), "six 32-bit fields");
  return DecodeItem{w[0], w[1], w[2], w[3], w[4], w[5]};
}

// Launch order of the decode kernels: workgroups walk the (longest-first)
// items in chunks of `chunk` items; inside a chunk, head by head, so that
// consecutive workgroups serve consecutive items of the chunk (chunks of 1:
// all heads of an item, then the next item).  All heads of the longest items
// start first either way.  Returns (item, kv head) of workgroup x.
__device__ inline void decode_work(const DecodeParams& p, int x, int& item, int& head) {
  const int per_chunk = p.chunk * p.n_kv_heads;
  const int c0 = (x / per_chunk) * p.chunk;       // first item of this chunk
  const int cc = min(p.chunk, p.n_items - c0);    // items in this chunk
  const int r = x - c0 * p.n_kv_heads;
  head = r / cc;
  item = c0 + r % cc;
}

// Fused append of an item's newest token (the item ends at its sequence's
// last position, pos = t_begin + n_tokens - 1) for KV head g: where its K
// and V rows go and what they are made from.  ok is false (no write) when
// the slot's block id is out of range or the position has no rotary row,
// as in the append kernel.
// A rotary pairing as a type, to instantiate code per pairing.
template <int M>
struct RopeTag {
  static constexpr int value = M;
};

struct NewSlot {
  char* k;          // K head plane of the slot's block
  char* v;          // V head plane
  const char* kin;  // source rows, unrotated
  const char* vin;
  const float* cr;  // rotary rows of the position
  const float* sr;
  float ksc, vsc;   // quantised pools: this head's scales
  int tin;          // slot within the block
  bool ok;
};

template <int SDT, int PDT, int D>
__device__ inline NewSlot new_slot(const DecodeParams& p, const DecodeItem& it, int g) {
  NewSlot ns;
  const int pos = it.t_begin + it.n_tokens - 1;
  ns.tin = pos % kBlock;
  const int64_t row = (int64_t(it.seq) * p.n_kv_heads + g) * D * Fmt<SDT>::kBytes;
  ns.kin = p.new_k + row;
  ns.vin = p.new_v + row;
  // (the host has checked that the position has a rotary row; the clamp
  // only keeps the address in range)
  const int rpos = min(pos, max(p.max_pos - 1, 0));
  const bool rot = p.rope_mode != PKV_ROPE_NONE;  // the tables may be null otherwise
  ns.cr = rot ? p.cos_t + size_t(rpos) * (D / 2) : nullptr;
  ns.sr = rot ? p.sin_t + size_t(rpos) * (D / 2) : nullptr;
  ns.ksc = PDT == PKV_FP8E4M3 ? p.k_scale[g] : 1.f;
  ns.vsc = PDT == PKV_FP8E4M3 ? p.v_scale[g] : 1.f;
  ns.ok = p.rope_mode == PKV_ROPE_NONE || pos < p.max_pos;
  ns.k = ns.v = nullptr;
  return ns;
}

// The slot's K and V head planes once its block id is known; ok drops when
// the id is out of range.
__device__ inline void set_slot_planes(NewSlot& ns, const DecodeParams& p, int blk, int g) {
  ns.ok = ns.ok && blk >= 0 && blk < p.num_blocks;
  const int b = ns.ok ? blk : 0;
  ns.k = const_cast<char*>(p.pool_k) + int64_t(b) * p.p_block + int64_t(g) * p.p_head;
  ns.v = const_cast<char*>(p.pool_v) + int64_t(b) * p.p_block + int64_t(g) * p.p_head;
}

// Pool chunk c (dims c*XP .. c*XP + XP - 1) of the new token's K row: the
// source dims rotated as the inject kernel rotates them (the halves pairing
// reads the partner dims D/2 away as well), stored at the token's slot.  load()
// reads everything the chunk needs and store() computes and writes it, so
// that a caller can issue all its loads before its first store.  The decode
// kernels call them from the lane that later loads this chunk, so the lane's
// own program order makes that load see the store.
template <int SDT, int PDT, int D, int MODE>
struct KChunkPut {
  static constexpr int ES = Fmt<SDT>::kBytes;
  static constexpr int XS = 16 / ES, XP = 16 / Fmt<PDT>::kBytes;
  static constexpr int NS = XP / XS;  // 16-byte source pieces per pool chunk (1 or 2)
  static constexpr int NR = MODE == PKV_ROPE_PAIRS ? XP / 2 : MODE == PKV_ROPE_HALVES ? XP : 0;
  uint4 x[NS], y[NS];                 // the chunk's source dims and (halves) the partner's
  float c[NR > 0 ? NR : 1], s[NR > 0 ? NR : 1];  // rotary rows at the chunk's pair indices

  __device__ void load(const NewSlot& ns, int ch) {
    const int j0 = ch * XP;
#pragma unroll
    for (int i = 0; i < NS; ++i) x[i] = ld16(ns.kin + (j0 + i * XS) * ES);
    if constexpr (MODE == PKV_ROPE_PAIRS) {
#pragma unroll
      for (int e = 0; e < NR; ++e) {
        c[e] = ns.cr[j0 / 2 + e];
        s[e] = ns.sr[j0 / 2 + e];
      }
    } else if constexpr (MODE == PKV_ROPE_HALVES) {
      const int jp = j0 < D / 2 ? j0 + D / 2 : j0 - D / 2;
      const int i0 = j0 < D / 2 ? j0 : jp;  // pair index of the chunk's first dim
#pragma unroll
      for (int i = 0; i < NS; ++i) y[i] = ld16(ns.kin + (jp + i * XS) * ES);
#pragma unroll
      for (int e = 0; e < NR; ++e) {
        c[e] = ns.cr[i0 + e];
        s[e] = ns.sr[i0 + e];
      }
    }
  }

  // The chunk's 16 bytes in the pool format.
  __device__ uint4 pack(const NewSlot& ns, int ch) const {
    float f[XP];
#pragma unroll
    for (int i = 0; i < NS; ++i) unpack16<SDT>(x[i], f + i * XS);
    if constexpr (MODE == PKV_ROPE_PAIRS) {
      rot_pairs_f<XP>(f, 0, c, s);
    } else if constexpr (MODE == PKV_ROPE_HALVES) {
      float g[XP];
#pragma unroll
      for (int i = 0; i < NS; ++i) unpack16<SDT>(y[i], g + i * XS);
      if (ch * XP < D / 2) rot_halves_f<XP>(f, g, 0, c, s);
      else rot_halves_f<XP>(g, f, 0, c, s);
    }
    Packed<PDT, XP> pk;
    pk.set(f, ns.ksc);
    return *reinterpret_cast<const uint4*>(pk.v);
  }

  __device__ void store(const NewSlot& ns, int ch) const {
    st16_stream(ns.k + (ch * kBlock + ns.tin) * 16, pack(ns, ch));
  }
};

// Stores one head's result: final (single-range sequence) or partial state.
// m is in the log2-scaled domain; l is the sum of 2^(s - m).
__device__ inline void store_head_result(const DecodeParams& p, const DecodeItem& it, int hq,
                                         int dim, float o, float m, float l, bool write_ml,
                                         int D) {
  if (it.slot < 0) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    p.out[(int64_t(it.seq) * p.n_q_heads + hq) * D + dim] = o * inv;
    if (write_ml && p.lse)
      p.lse[int64_t(it.seq) * p.n_q_heads + hq] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
  } else {
    p.part_o[(int64_t(it.slot) * p.n_q_heads + hq) * D + dim] = o;
    if (write_ml) {
      p.part_ml[(int64_t(it.slot) * p.n_q_heads + hq) * 2 + 0] = m;
      p.part_ml[(int64_t(it.slot) * p.n_q_heads + hq) * 2 + 1] = l;
    }
  }
}

// ---------------------------------------------------------------------------
// Decode, MFMA: one wave per (work item, KV head), G <= 16 query heads.
//
// Per 16-token block:
//   S^T[t][h] = sum_j K[t][j] q_h[j]   v_mfma_f32_16x16x32 (bf16/f16), D/32 steps
//     A = K plane: lane l loads 16 bytes at (64*s + l)*16 of the plane, i.e.
//         token l%16, chunk 4s + l/16 -- the k-slots of row l%16;
//     B = q: lane l holds head (l%16)'s dims of the same chunk (0 for l%16 >= G).
//   Result: lane l holds scores of tokens 4*(l/16)+r (r<4) for head l%16.
//   Online softmax per head across the 4 lanes sharing l%16 (xor 16, 32).
//   out^T[j][h] += sum_t V^T[j][t] P^T[t][h]   v_mfma_f32_16x16x16, D/16 tiles
//     A = V plane rows 16n + l%16, tokens 4*(l/16)..+3 (8 bytes);
//     B = P^T: exactly the score registers of this lane, converted to
//         16-bit as a hi part plus a lo residual (two MFMAs) so that the
//         probabilities keep ~16 significant bits.
// Accumulators: lane l holds out[head l%16][dims 16n + 4*(l/16) + r].
// ---------------------------------------------------------------------------
template <int DT> struct Mfma;
template <> struct Mfma<PKV_BF16> {
  typedef bf16x8_t V8;
  typedef bf16x4_t V4;
  __device__ static f32x4_t qk(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(V8, a),
                                                    __builtin_bit_cast(V8, b), c, 0, 0, 0);
  }
  __device__ static f32x4_t pv(uint2 a, uint2 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(V4, a),
                                                      __builtin_bit_cast(V4, b), c, 0, 0, 0);
  }
  // Split p into hi + lo 16-bit parts (hi by truncation, lo = rest truncated).
  __device__ static void split(float p, uint16_t& hi, uint16_t& lo) {
    const uint32_t u = __float_as_uint(p) & 0xffff0000u;
    hi = uint16_t(u >> 16);
    lo = uint16_t(__float_as_uint(p - __uint_as_float(u)) >> 16);
  }
};
template <> struct Mfma<PKV_F16> {
  typedef f16x8_t V8;
  typedef f16x4_t V4;
  __device__ static f32x4_t qk(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(V8, a),
                                                   __builtin_bit_cast(V8, b), c, 0, 0, 0);
  }
  __device__ static f32x4_t pv(uint2 a, uint2 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(V4, a),
                                                  __builtin_bit_cast(V4, b), c, 0, 0, 0);
  }
  __device__ static void split(float p, uint16_t& hi, uint16_t& lo) {
    const _Float16 h = static_cast<_Float16>(p);
    const _Float16 l = static_cast<_Float16>(p - float(h));
    hi = __builtin_bit_cast(uint16_t, h);
    lo = __builtin_bit_cast(uint16_t, l);
  }
};

// Four fp8 (OCP E4M3) codes of a dword -> their exact float16 values
// (x: codes 0, 1; y: codes 2, 3).  CDNA4's packed conversion with a unit
// scale is exact for every code (E4M3 values are a subset of float16's),
// NaN included; the per-(layer, head) scales are applied to the scores and
// the output instead.
__device__ inline uint2 e4m3x4_to_f16x4(uint32_t w) {
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  const f16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  const f16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8): wait until at most n vector-memory operations are
// outstanding; wait for every LDS/scalar operation.
constexpr int wait_vm_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int wait_lgkm0_imm() { return 15 | (3 << 14) | (7 << 4); }

// Decode kernel template parameters: KVDT the pool format, QDT the query
// format (equal to KVDT, or BF16/F16 for an fp8 pool whose MFMA operands are
// float16), head dim D, prefetch depth, waves per workgroup NW, NG tiles of
// 16 query heads (a KV head's group of up to 16 NG query heads: every
// block's K and V, loaded once, serve all NG tiles), PUT: whether the
// kernel carries the decode step's append of the newest token (attention
// alone runs an instance without that code, which it would otherwise pay for
// in registers and scheduling even when no token is appended), and BLK: an
// fp8 pool whose scales are per (layer, block, KV head) (its own instance,
// for the same reason).
template <int KVDT, int QDT, int D, int DEPTH, int NW, int NG, bool PUT, bool BLK>
// `tables` is p.tables again as a restrict-qualified argument: the kernel's
// only stores (the fused append) go to the pool, and with the table known
// not to alias them its entries keep coming through scalar loads.
__global__ __launch_bounds__(64 * NW) void decode_mfma_kernel(DecodeParams p,
                                                              const int32_t* __restrict__ tables) {
  constexpr bool FP8 = KVDT == PKV_FP8E4M3;
  constexpr int OT = FP8 ? PKV_F16 : KVDT;  // MFMA operand format
  constexpr int S = D / 32;   // QK MFMA steps of 32 dims
  constexpr int SL = FP8 ? S / 2 : S;  // 16-byte K loads per lane and block
  constexpr int NT = D / 16;  // PV MFMA tiles of 16 dims
  constexpr int VB = FP8 ? 4 : 8;      // V bytes per lane and tile
  const int lane = threadIdx.x & 63;
  // Wave-uniform (scalar register): block-table reads below then become
  // scalar loads, whose waits do not stall on the K/V loads in flight.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & 15;
  const int grp = lane >> 4;
  int item_i, g;
  decode_work(p, blockIdx.x, item_i, g);
  const DecodeItem it = decode_item(p, item_i);
  // Tile t covers query heads g G + 16 t + row (G = p.group).
  auto head_of = [&](int t) { return g * p.group + 16 * t + row; };
  auto head_ok = [&](int t) { return 16 * t + row < p.group; };

  // q operand (B of QK) for head `row` of each tile: the dims whose K this
  // lane loads in the same step (16-bit pools: chunk 4s + grp of 8 dims; fp8
  // pools: half `st % 2` of chunk 4(st/2) + grp of 16 dims).
  uint4 qreg[NG][S];
#pragma unroll
  for (int t = 0; t < NG; ++t) {
    typedef typename Fmt<QDT>::T TQ;
    const TQ* qh = reinterpret_cast<const TQ*>(p.q) +
                   (int64_t(it.seq) * p.n_q_heads + (head_ok(t) ? head_of(t) : g * p.group)) * D;
#pragma unroll
    for (int st = 0; st < S; ++st) {
      const int dim0 = FP8 ? (4 * (st / 2) + grp) * 16 + 8 * (st % 2) : (4 * st + grp) * 8;
      uint4 raw = ld16(qh + dim0);
      if constexpr (FP8 && QDT != PKV_F16) {
        float f[8];
        unpack16<QDT>(raw, f);
        _Float16 hv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[e] = static_cast<_Float16>(f[e]);
        raw = *reinterpret_cast<const uint4*>(hv);
      }
      qreg[t][st] = head_ok(t) ? raw : make_uint4(0, 0, 0, 0);
    }
  }
  // fp8 scales: per (layer, KV head), folded into the score multiplier and
  // the final output; or per (layer, block, KV head) (blockwise), read with
  // each block's id and applied to its scores and to its P·V product.
  constexpr bool blockwise = FP8 && BLK;
  float kmul = 1.f, vmul = 1.f;
  if constexpr (FP8 && !blockwise) {
    kmul = p.k_scale[g];
    vmul = p.v_scale[g];
  }
  const float score_mul = p.scale_log2 * kmul;

  const int32_t* tab = tables + int64_t(it.seq) * p.table_stride + it.t_begin / kBlock;
  const char* kbase = p.pool_k + int64_t(g) * p.p_head;
  const char* vbase = p.pool_v + int64_t(g) * p.p_head;
  const int nblk = (it.n_tokens + kBlock - 1) / kBlock;
  // This wave takes blocks wave, wave + NW, wave + 2 NW, ...
  const int nj = nblk > wave ? (nblk - wave + NW - 1) / NW : 0;
  // Fused append: the wave that takes the newest token's block (its j-th,
  // put_j) makes the token's K chunks and V elements in the pool format
  // before its loop, each lane those it holds when it loads that block (K
  // chunks 4s + grp and V dims 16n + row of the slot); when it takes that
  // block it puts them into its registers in place of the loaded ones and
  // writes the block's planes back.  Other waves: put_j = -1.
  int put_j = -1;
  if constexpr (PUT) {
    if (p.new_k != nullptr && it.last && it.n_tokens > 0) {
      const int lb = (it.n_tokens - 1) / kBlock;
      if (lb % NW == wave) put_j = lb / NW;
    }
  }

  f32x4_t acc[NG][NT];
  float m[NG];  // running max (log2 domain), uniform over the head's lanes
  float l[NG];  // this lane's share of the running sum
#pragma unroll
  for (int t = 0; t < NG; ++t) {
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[t][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m[t] = -INFINITY;
    l[t] = 0.f;
  }

  uint4 kbuf[DEPTH][SL];
  uint2 vbuf[DEPTH][NT];   // fp8: only .x holds the 4 codes
  bool okbuf[DEPTH];
  float kscb[DEPTH], vscb[DEPTH];  // blockwise fp8 scales of the blocks in flight
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) kscb[d] = vscb[d] = 1.f;

  int put_blk = -1;  // block id read for the newest token's block
  // Block ids are read one issue ahead (issues come in order j = 0, 1, ...),
  // so the scalar load's latency does not sit between a block's arrival and
  // the next block's loads.
  // Staged instance (attention alone, one tile, 8 waves, 16-bit pools, two
  // blocks in flight per wave: kernel variant 12): each block's K and V
  // planes go to the wave's LDS buffer d by direct loads (global_load_lds,
  // 1 KiB per instruction, no VGPRs while in flight) and are read from there
  // when the block is taken.  The compiler does not track direct loads
  // against LDS reads, so the waits are explicit: before block j the wave
  // waits until only block j + 1's loads are outstanding (loads complete in
  // order), and before refilling buffer d it waits for its LDS reads.  Same
  // values and order as the register path, so the results are bit-identical.
  constexpr bool STAGE = !PUT && NG == 1 && NW == 8 && !FP8 && DEPTH == 2;
  constexpr int PLANE = kBlock * D * 2;           // bytes of a K or a V plane
  constexpr int NDL = 2 * PLANE / 1024;           // direct loads per block
  __shared__ __align__(16) char stage[STAGE ? NW : 1][2][STAGE ? 2 * PLANE : 16];
  int blk_next = nj > 0 ? tab[wave] : 0;
  auto issue = [&](int j, int d) {
    int blk = blk_next;
    if (j + 1 < nj) blk_next = tab[wave + (j + 1) * NW];
    if (j == put_j) put_blk = blk;
    const bool ok = unsigned(blk) < unsigned(p.num_blocks);
    okbuf[d] = ok;
    blk = ok ? blk : 0;
    if constexpr (blockwise) {
      kscb[d] = p.k_scale[int64_t(blk) * p.n_kv_heads + g];
      vscb[d] = p.v_scale[int64_t(blk) * p.n_kv_heads + g];
    }
    const char* kp = kbase + int64_t(blk) * p.p_block;
    const char* vp = vbase + int64_t(blk) * p.p_block;
    if constexpr (STAGE) {
      typedef __attribute__((address_space(3))) void* lds_ptr;
      asm volatile("" ::: "memory");
#pragma unroll
      for (int c = 0; c < PLANE / 1024; ++c)  // aux 2: non-temporal, as ld16_stream
        __builtin_amdgcn_global_load_lds(kp + c * 1024 + lane * 16,
                                         (lds_ptr)&stage[wave][d][c * 1024], 16, 0, 2);
#pragma unroll
      for (int c = 0; c < PLANE / 1024; ++c)
        __builtin_amdgcn_global_load_lds(vp + c * 1024 + lane * 16,
                                         (lds_ptr)&stage[wave][d][PLANE + c * 1024], 16, 0, 2);
      asm volatile("" ::: "memory");
      return;
    }
#pragma unroll
    for (int s = 0; s < SL; ++s) kbuf[d][s] = ld16_stream(kp + (64 * s + lane) * 16);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      if constexpr (FP8) vbuf[d][n].x = ld4_stream(vp + (16 * n + row) * 16 + grp * 4);
      else vbuf[d][n] = ld8_stream(vp + (16 * n + row) * 32 + grp * 8);
    }
  };

  NewSlot ns{};
  // The token's K and V rows in the pool format, made by the whole wave
  // (lane i < D/2 rotates pair i; lanes take V dims lane, lane + 64) and
  // read back, when the wave takes the token's block, by the lanes that hold
  // the slot (K chunks 4s + grp in lanes with row == slot, V dims 16n + row
  // in lanes with grp == slot / 4): kept in LDS meanwhile, not in registers.
  // The source values are all read before the wave's first block is issued:
  // loads complete in order, so waiting for them does not wait for that
  // block, and no load waits behind the arithmetic of another.
  typedef typename Fmt<KVDT>::T TP;
  typedef typename Fmt<QDT>::T TQ;
  __shared__ __align__(16) TP new_row[2][D];
  TQ nk[2], nv[D / 64];
  float nrc = 1.f, nrs = 0.f;  // rotary row at the lane's pair
  const bool halves = p.rope_mode == PKV_ROPE_HALVES;
  const int nj0 = halves ? lane : 2 * lane;           // the lane's pair (lane < D/2)
  const int nj1 = halves ? lane + D / 2 : 2 * lane + 1;
  auto load_new = [&]() {
    const TQ* kin = reinterpret_cast<const TQ*>(ns.kin);
    const TQ* vin = reinterpret_cast<const TQ*>(ns.vin);
    if (lane < D / 2) {
      nk[0] = kin[nj0];
      nk[1] = kin[nj1];
      if (p.rope_mode != PKV_ROPE_NONE) {
        nrc = ns.cr[lane];
        nrs = ns.sr[lane];
      }
    }
#pragma unroll
    for (int e = 0; e < D / 64; ++e) nv[e] = vin[lane + 64 * e];
  };
  auto make_new = [&]() {
    if (lane < D / 2) {
      float x0 = Fmt<QDT>::to_f32(nk[0]), x1 = Fmt<QDT>::to_f32(nk[1]);
      if (p.rope_mode != PKV_ROPE_NONE) {
        const float y0 = x0 * nrc - x1 * nrs;
        const float y1 = x0 * nrs + x1 * nrc;
        x0 = y0;
        x1 = y1;
      }
      new_row[0][nj0] = Fmt<KVDT>::from_f32(FP8 ? x0 / ns.ksc : x0);
      new_row[0][nj1] = Fmt<KVDT>::from_f32(FP8 ? x1 / ns.ksc : x1);
    }
#pragma unroll
    for (int e = 0; e < D / 64; ++e) {
      if constexpr (QDT == KVDT) new_row[1][lane + 64 * e] = nv[e];
      else new_row[1][lane + 64 * e] = Fmt<KVDT>::from_f32(Fmt<QDT>::to_f32(nv[e]) / ns.vsc);
    }
    // the row is written and read by lanes of this one wave
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  if constexpr (PUT) {
    static_assert(DEPTH == 1, "the fused append runs with one block in flight");
    if (put_j >= 0) {
      // The token's loads, then the wave's first block (it has one: put_j
      // is among its blocks), then the row: all in one path, so that the row
      // waits for the token's loads only.
      ns = new_slot<QDT, KVDT, D>(p, it, g);
      if constexpr (blockwise) {  // the scales of the block the token goes to
        const int pb = tab[wave + put_j * NW];
        const int64_t pi = int64_t(unsigned(pb) < unsigned(p.num_blocks) ? pb : 0) * p.n_kv_heads + g;
        ns.ksc = p.k_scale[pi];
        ns.vsc = p.v_scale[pi];
      }
      load_new();
      issue(0, 0);
      make_new();
      if (!ns.ok) put_j = -1;  // no write, and the block is read as stored
    } else if (nj > 0) {
      issue(0, 0);
    }
  } else {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
      if (d < nj) issue(d, d);
  }

  // One block of the wave's range (j its index among the wave's blocks, d
  // its prefetch buffer; AT_PUT: the newest token's block, put_j).  A macro,
  // not a lambda: the lambda form measured ~1 % slower on the 16-bit decode
  // steps (its code differs in register allocation and waits).
#define PKV_DECODE_BLOCK(j, d, AT_PUT) \
  do {                                 \
          if (AT_PUT) {                                                                          \
            /* the newest token's slot: the values made above, not the pool's */                 \
            if (row == ns.tin) {                                                                 \
  _Pragma("unroll")                                                                              \
              for (int s = 0; s < SL; ++s)                                                       \
                kbuf[d][s] = *reinterpret_cast<const uint4*>(                                    \
                    &new_row[0][(4 * s + grp) * (16 / sizeof(TP))]);                             \
            }                                                                                    \
            if (grp == ns.tin / 4) {                                                             \
              const int e = ns.tin & 3;  /* token 4 grp + e of the lane's V registers */         \
  _Pragma("unroll")                                                                              \
              for (int n = 0; n < NT; ++n) {                                                     \
                const uint32_t vnew = uint32_t(new_row[1][16 * n + row]);                        \
                if constexpr (FP8) {                                                             \
                  const uint32_t mask = 0xFFu << (8 * e);                                        \
                  vbuf[d][n].x = (vbuf[d][n].x & ~mask) | (vnew << (8 * e));                     \
                } else {                                                                         \
                  const uint32_t mask = 0xFFFFu << (16 * (e & 1));                               \
                  const uint32_t bits = vnew << (16 * (e & 1));                                  \
                  uint32_t x = vbuf[d][n].x, y = vbuf[d][n].y;                                   \
                  if (e < 2) x = (x & ~mask) | bits;                                             \
                  else y = (y & ~mask) | bits;                                                   \
                  vbuf[d][n] = make_uint2(x, y);                                                 \
                }                                                                                \
              }                                                                                  \
            }                                                                                    \
            /* The block's K and V planes go back to the pool whole, with the */                 \
            /* token in place: full lines, where the token's own elements would */               \
            /* be partial writes to every line of the V plane.  (The slot's */                   \
            /* block id was read when this block was issued.) */                                 \
            if (unsigned(put_blk) < unsigned(p.num_blocks)) {                                    \
              char* kp = const_cast<char*>(kbase) + int64_t(put_blk) * p.p_block;                \
              char* vp = const_cast<char*>(vbase) + int64_t(put_blk) * p.p_block;                \
  _Pragma("unroll")                                                                              \
              for (int s = 0; s < SL; ++s) st16_stream(kp + (64 * s + lane) * 16, kbuf[d][s]);   \
  _Pragma("unroll")                                                                              \
              for (int n = 0; n < NT; ++n) {                                                     \
                if constexpr (FP8) st4_stream(vp + (16 * n + row) * 16 + grp * 4, vbuf[d][n].x); \
                else st8_stream(vp + (16 * n + row) * 32 + grp * 8, vbuf[d][n]);                 \
              }                                                                                  \
            }                                                                                    \
          }                                                                                      \
          if constexpr (STAGE) {                                                                 \
            asm volatile("" ::: "memory");                                                       \
            if (j + 1 < nj) __builtin_amdgcn_s_waitcnt(wait_vm_imm(NDL));                        \
            else __builtin_amdgcn_s_waitcnt(wait_vm_imm(0));                                     \
            asm volatile("" ::: "memory");                                                       \
            _Pragma("unroll")                                                                    \
            for (int s2 = 0; s2 < SL; ++s2)                                                      \
              kbuf[d][s2] = *(const uint4*)&stage[wave][d][(64 * s2 + lane) * 16];              \
            _Pragma("unroll")                                                                    \
            for (int n = 0; n < NT; ++n)                                                         \
              vbuf[d][n] = *(const uint2*)&stage[wave][d][PLANE + (16 * n + row) * 32 + grp * 8]; \
          }                                                                                      \
          /* every tile's scores before the next block's loads reuse kbuf[d] */                  \
          f32x4_t sc[NG];                                                                        \
  _Pragma("unroll")                                                                              \
          for (int t = 0; t < NG; ++t) sc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};                      \
          if constexpr (FP8) {                                                                   \
  _Pragma("unroll")                                                                              \
            for (int s = 0; s < SL; ++s) {                                                       \
              const uint4 w = kbuf[d][s];                                                        \
              const uint2 a0 = e4m3x4_to_f16x4(w.x), a1 = e4m3x4_to_f16x4(w.y);                  \
              const uint2 a2 = e4m3x4_to_f16x4(w.z), a3 = e4m3x4_to_f16x4(w.w);                  \
              const uint4 k0 = make_uint4(a0.x, a0.y, a1.x, a1.y);                               \
              const uint4 k1 = make_uint4(a2.x, a2.y, a3.x, a3.y);                               \
  _Pragma("unroll")                                                                              \
              for (int t = 0; t < NG; ++t) {                                                     \
                sc[t] = Mfma<OT>::qk(k0, qreg[t][2 * s], sc[t]);                                 \
                sc[t] = Mfma<OT>::qk(k1, qreg[t][2 * s + 1], sc[t]);                             \
              }                                                                                  \
            }                                                                                    \
          } else {                                                                               \
  _Pragma("unroll")                                                                              \
            for (int s = 0; s < S; ++s)                                                          \
  _Pragma("unroll")                                                                              \
              for (int t = 0; t < NG; ++t) sc[t] = Mfma<OT>::qk(kbuf[d][s], qreg[t][s], sc[t]);  \
          }                                                                                      \
          uint2 vcur[NT];                                                                        \
  _Pragma("unroll")                                                                              \
          for (int n = 0; n < NT; ++n)                                                           \
            vcur[n] = FP8 ? e4m3x4_to_f16x4(vbuf[d][n].x) : vbuf[d][n];                          \
          const bool blk_ok = okbuf[d];                                                          \
          /* this block's scales, before the next issue reuses the slot */                       \
          const float ksb = kscb[d], vsb = vscb[d];                                              \
          if constexpr (STAGE) {  /* this block's LDS reads are done before buffer d refills */ \
            asm volatile("" ::: "memory");                                                       \
            __builtin_amdgcn_s_waitcnt(wait_lgkm0_imm());                                        \
            asm volatile("" ::: "memory");                                                       \
          }                                                                                      \
          if (j + DEPTH < nj) issue(j + DEPTH, d);                                               \
                                                                                                 \
          const int valid = it.n_tokens - (wave + j * NW) * kBlock;  /* tokens in range */       \
          /* Slots of this block before a sliding window's start (positive only */               \
          /* in the window's first block). */                                                    \
          const int skip = it.lo - (it.t_begin + (wave + j * NW) * kBlock);                      \
          /* Scaled scores; slots outside [lo, end) or of a rejected block id */                 \
          /* get -inf.  A whole block (the common case; wave-uniform) needs no */                \
          /* masks, and the masked case rewrites the values in place. */                         \
          float s4[NG][4];                                                                       \
          float smul = score_mul;                                                                \
          if constexpr (blockwise) smul = p.scale_log2 * ksb;                                    \
  _Pragma("unroll")                                                                              \
          for (int t = 0; t < NG; ++t)                                                           \
  _Pragma("unroll")                                                                              \
            for (int r = 0; r < 4; ++r) s4[t][r] = sc[t][r] * smul;                              \
          if (!(blk_ok && valid >= kBlock && skip <= 0)) {                                       \
            /* The masked slots may hold anything, NaN included: zero their V */                 \
            /* so that 0-weight * V stays 0.  Lane holds tokens 4*grp + e, */                    \
            /* e = 0..3, as 16-bit halves of x, y. */                                            \
            const int lim = blk_ok ? valid : 0;                                                  \
            auto in = [&](int e) { return e < lim && e >= skip; };                               \
            const uint32_t mx0 = (in(4 * grp + 0) ? 0x0000ffffu : 0u) |                          \
                                 (in(4 * grp + 1) ? 0xffff0000u : 0u);                           \
            const uint32_t mx1 = (in(4 * grp + 2) ? 0x0000ffffu : 0u) |                          \
                                 (in(4 * grp + 3) ? 0xffff0000u : 0u);                           \
  _Pragma("unroll")                                                                              \
            for (int n = 0; n < NT; ++n) {                                                       \
              vcur[n].x &= mx0;                                                                  \
              vcur[n].y &= mx1;                                                                  \
            }                                                                                    \
  _Pragma("unroll")                                                                              \
            for (int t = 0; t < NG; ++t)                                                         \
  _Pragma("unroll")                                                                              \
              for (int r = 0; r < 4; ++r)                                                        \
                if (!in(4 * grp + r)) s4[t][r] = -INFINITY;                                      \
          }                                                                                      \
  _Pragma("unroll")                                                                              \
          for (int t = 0; t < NG; ++t) {                                                         \
            float mx = -INFINITY;                                                                \
  _Pragma("unroll")                                                                              \
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s4[t][r]);                                \
            mx = cols_max(mx);                                                                   \
            /* Rescale the running state only when some head's maximum grows (a */               \
            /* wave-uniform test): otherwise the factor would be exactly 1, and */               \
            /* after the first blocks of a long range it rarely grows. */                        \
            const bool grow = mx > m[t];  /* false while both are -inf */                        \
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {                                        \
              /* 0 when m was -inf */                                                            \
              const float alpha = grow ? __builtin_amdgcn_exp2f(m[t] - mx) : 1.f;                \
              l[t] *= alpha;                                                                     \
  _Pragma("unroll")                                                                              \
              for (int n = 0; n < NT; ++n) acc[t][n] *= alpha;                                   \
              m[t] = fmaxf(m[t], mx);                                                            \
            }                                                                                    \
            /* m is -inf only while every score seen so far is masked; then every */             \
            /* s4 is -inf too and its weight must be 0. */                                       \
            const float m_ref = m[t] == -INFINITY ? 0.f : m[t];                                  \
            /* The hardware 2^x (about one ulp over the normal range): the */                    \
            /* arguments are <= 0, and weights below 2^-126, which it may flush */               \
            /* to 0, are far below one ulp of the sum (at least 1). */                           \
            float pr[4];                                                                         \
  _Pragma("unroll")                                                                              \
            for (int r = 0; r < 4; ++r) {                                                        \
              pr[r] = __builtin_amdgcn_exp2f(s4[t][r] - m_ref);                                  \
              l[t] += pr[r];                                                                     \
            }                                                                                    \
            /* 16-bit pools: P as a 16-bit high part plus a 16-bit residual, */                  \
            /* two MFMAs (a single bf16 P could exceed the tolerance).  fp8 */                   \
            /* pools: P rounded once to float16 (relative error at most 2^-12, */                \
            /* far inside the tolerance), one MFMA. */                                           \
            constexpr bool LO = !FP8;                                                            \
            uint16_t ph[4], pl[4];                                                               \
  _Pragma("unroll")                                                                              \
            for (int r = 0; r < 4; ++r) {                                                        \
              if constexpr (LO) Mfma<OT>::split(pr[r], ph[r], pl[r]);                            \
              else ph[r] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(pr[r]));           \
            }                                                                                    \
            const uint2 bh = make_uint2(uint32_t(ph[0]) | (uint32_t(ph[1]) << 16),               \
                                        uint32_t(ph[2]) | (uint32_t(ph[3]) << 16));              \
            uint2 bl = make_uint2(0, 0);                                                         \
            if constexpr (LO)                                                                    \
              bl = make_uint2(uint32_t(pl[0]) | (uint32_t(pl[1]) << 16),                         \
                              uint32_t(pl[2]) | (uint32_t(pl[3]) << 16));                        \
            if constexpr (blockwise) {                                                           \
              /* this block's P·V on its own, then scaled by its V scale */                      \
  _Pragma("unroll")                                                                              \
              for (int n = 0; n < NT; ++n) {                                                     \
                f32x4_t b = Mfma<OT>::pv(vcur[n], bh, f32x4_t{0.f, 0.f, 0.f, 0.f});              \
                if constexpr (LO) b = Mfma<OT>::pv(vcur[n], bl, b);                              \
  _Pragma("unroll")                                                                              \
                for (int r = 0; r < 4; ++r) acc[t][n][r] = fmaf(vsb, b[r], acc[t][n][r]);        \
              }                                                                                  \
            } else {                                                                             \
  _Pragma("unroll")                                                                              \
              for (int n = 0; n < NT; ++n) {                                                     \
                acc[t][n] = Mfma<OT>::pv(vcur[n], bh, acc[t][n]);                                \
                if constexpr (LO) acc[t][n] = Mfma<OT>::pv(vcur[n], bl, acc[t][n]);              \
              }                                                                                  \
            }                                                                                    \
          } \
  } while (0)
  // fp8 pools run the newest token's block, the wave's last (put_j ==
  // nj - 1), after the loop, so the loop carries none of the append's values
  // and tests (their decode step measured 2-3 % faster that way); 16-bit pools
  // test for it in the loop (the separate block measured ~1 % slower there).
  if constexpr (FP8) {
    const int nmain = put_j >= 0 ? put_j : nj;
    for (int j0 = 0; j0 < nmain; j0 += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        const int j = j0 + d;
        if (j < nmain) PKV_DECODE_BLOCK(j, d, false);
      }
    }
    if constexpr (PUT) {
      if (put_j >= 0) {
        const int j = put_j, d = put_j % DEPTH;
        PKV_DECODE_BLOCK(j, d, true);
      }
    }
  } else {
    for (int j0 = 0; j0 < nj; j0 += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        const int j = j0 + d;
        if (j < nj) PKV_DECODE_BLOCK(j, d, PUT && j == put_j);
      }
    }
  }
#undef PKV_DECODE_BLOCK

#pragma unroll
  for (int t = 0; t < NG; ++t) {
    l[t] = cols_sum(l[t]);
  }

  if constexpr (NW > 1) {
    // Merge the waves' softmax states, one tile of heads at a time.  Every
    // wave scales its partial output to the common maximum and parks it in
    // LDS; wave w then sums output tiles w, w + NW, ... over all waves in
    // fixed order (wave 0, 1, ...).
    __shared__ float sm_m[NW][16], sm_l[NW][16];
    // (the staged instance parks the partial outputs in its staging buffers,
    // which every wave has finished with by the first barrier below)
    typedef float SmO[16][D + 4];
    SmO* sm_o;
    if constexpr (STAGE) {
      static_assert(sizeof(SmO) * NW <= sizeof(stage), "merge buffers fit the staging area");
      sm_o = reinterpret_cast<SmO*>(&stage[0][0][0]);
    } else {
      __shared__ float sm_o_arr[NW][16][D + 4];
      sm_o = sm_o_arr;
    }
#pragma unroll
    for (int t = 0; t < NG; ++t) {
      if (t > 0) __syncthreads();  // the previous tile's reads of LDS are done
      if (grp == 0) {
        sm_m[wave][row] = m[t];
        sm_l[wave][row] = l[t];
      }
      __syncthreads();
      float big_m = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) big_m = fmaxf(big_m, sm_m[w][row]);
      float big_l = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = sm_m[w][row];
        big_l += (mw == -INFINITY ? 0.f : exp2f(mw - big_m)) * sm_l[w][row];
      }
      const float own = m[t] == -INFINITY ? 0.f : exp2f(m[t] - big_m);
#pragma unroll
      for (int n = 0; n < NT; ++n)
        *reinterpret_cast<f32x4_t*>(&sm_o[wave][row][16 * n + 4 * grp]) = acc[t][n] * own;
      __syncthreads();
      if (head_ok(t)) {
        for (int n = wave; n < NT; n += NW) {
          f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int w = 0; w < NW; ++w)
            a += *reinterpret_cast<const f32x4_t*>(&sm_o[w][row][16 * n + 4 * grp]);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            store_head_result(p, it, head_of(t), 16 * n + 4 * grp + r, a[r] * vmul, big_m,
                              big_l, n == 0 && r == 0 && grp == 0, D);
        }
      }
    }
    return;
  }

#pragma unroll
  for (int t = 0; t < NG; ++t) {
    if (!head_ok(t)) continue;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        store_head_result(p, it, head_of(t), 16 * n + 4 * grp + r, acc[t][n][r] * vmul, m[t],
                          l[t], n == 0 && r == 0 && grp == 0, D);
    }
  }
}

// ---------------------------------------------------------------------------
// Decode, packed dot products on the VALU (bf16/f16 pools, G <= 4 query heads
// per KV head, attention alone): the workgroup shape, block order, loads and
// online softmax of decode_mfma_kernel, with the two contractions done by
// v_dot2_f32_{bf16,f16} instead of matrix instructions.  Kept as a measured
// alternative for small query groups.
//
// Per 16-token block, lane (row, grp) = (lane % 16, lane / 16):
//   scores:  the lane holds K chunks 4s + grp of token `row` (the MFMA
//            kernel's loads) and the same dims of each query head; its
//            partial dot products are summed over the four lanes of a token
//            (lane swaps), so every lane of row t holds s[t][h];
//   softmax: maximum and weights per head over the 16 tokens of a row (DPP
//            row operations); the running sum is kept per token row;
//   PV:      the lane holds V dims 16n + row for tokens 4 grp .. 4 grp + 3
//            (the MFMA kernel's loads) and fetches those tokens' weights
//            from the lanes of their rows (ds_bpermute); the weights go to
//            16-bit as a hi part plus a lo residual, as in the MFMA kernel,
//            and each (dim, head) takes four dot2 steps.  The partial outputs
//            are summed over the four token groups at the end.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ inline float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Maximum / sum over the 16 lanes of each row, result in every lane of the
// row (quad swaps, then half-row and row mirrors); each step combines the
// same two values in both lanes of a pair, so the row's lanes agree bit for
// bit.
__device__ inline float row_max16(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));   // quad_perm 1,0,3,2
  x = fmaxf(x, dpp_f<0x4E>(x));   // quad_perm 2,3,0,1
  x = fmaxf(x, dpp_f<0x141>(x));  // row_half_mirror
  return fmaxf(x, dpp_f<0x140>(x));  // row_mirror
}
__device__ inline float row_sum16(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0x141>(x);
  return x + dpp_f<0x140>(x);
}

template <int DT> struct Dot2;
template <> struct Dot2<PKV_BF16> {
  typedef __attribute__((ext_vector_type(2))) __bf16 V2;
  __device__ static float dot(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(V2, a), __builtin_bit_cast(V2, b),
                                           c, false);
  }
};
template <> struct Dot2<PKV_F16> {
  typedef __attribute__((ext_vector_type(2))) _Float16 V2;
  __device__ static float dot(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(V2, a), __builtin_bit_cast(V2, b), c, false);
  }
};

template <int KVDT, int D, int NW, int GM>
__global__ __launch_bounds__(64 * NW) void decode_dot2_kernel(DecodeParams p,
                                                              const int32_t* __restrict__ tables) {
  constexpr int S = D / 32;   // 16-byte K loads per lane and block (chunks 4s + grp)
  constexpr int NT = D / 16;  // 8-byte V loads per lane and block (dims 16n + row)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = lane & 15;
  const int grp = lane >> 4;
  int item_i, g;
  decode_work(p, blockIdx.x, item_i, g);
  const DecodeItem it = decode_item(p, item_i);
  const int group = p.group;

  // query dims matching this lane's K chunks, every head of the group
  uint4 qreg[GM][S];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    const int hh = h < group ? h : 0;
    const uint16_t* qh = reinterpret_cast<const uint16_t*>(p.q) +
                         (int64_t(it.seq) * p.n_q_heads + g * group + hh) * D;
#pragma unroll
    for (int st = 0; st < S; ++st) qreg[h][st] = ld16(qh + (4 * st + grp) * 8);
  }
  const int32_t* tab = tables + int64_t(it.seq) * p.table_stride + it.t_begin / kBlock;
  const char* kbase = p.pool_k + int64_t(g) * p.p_head;
  const char* vbase = p.pool_v + int64_t(g) * p.p_head;
  const int nblk = (it.n_tokens + kBlock - 1) / kBlock;
  const int nj = nblk > wave ? (nblk - wave + NW - 1) / NW : 0;

  float acc[GM][NT];
  float m[GM], l[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[h][n] = 0.f;
    m[h] = -INFINITY;
    l[h] = 0.f;
  }
  uint4 kbuf[S];
  uint2 vbuf[NT];
  bool okb = false;
  int blk_next = nj > 0 ? tab[wave] : 0;
  auto issue = [&](int j) {
    int blk = blk_next;
    if (j + 1 < nj) blk_next = tab[wave + (j + 1) * NW];
    okb = unsigned(blk) < unsigned(p.num_blocks);
    blk = okb ? blk : 0;
    const char* kp = kbase + int64_t(blk) * p.p_block;
    const char* vp = vbase + int64_t(blk) * p.p_block;
#pragma unroll
    for (int st = 0; st < S; ++st) kbuf[st] = ld16_stream(kp + (64 * st + lane) * 16);
#pragma unroll
    for (int n = 0; n < NT; ++n) vbuf[n] = ld8_stream(vp + (16 * n + row) * 32 + grp * 8);
  };
  if (nj > 0) issue(0);
  for (int j = 0; j < nj; ++j) {
    float part[GM];
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      float a = 0.f;
#pragma unroll
      for (int st = 0; st < S; ++st) {
        a = Dot2<KVDT>::dot(kbuf[st].x, qreg[h][st].x, a);
        a = Dot2<KVDT>::dot(kbuf[st].y, qreg[h][st].y, a);
        a = Dot2<KVDT>::dot(kbuf[st].z, qreg[h][st].z, a);
        a = Dot2<KVDT>::dot(kbuf[st].w, qreg[h][st].w, a);
      }
      part[h] = a;
    }
    uint2 vcur[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) vcur[n] = vbuf[n];
    const bool blk_ok = okb;
    if (j + 1 < nj) issue(j + 1);

    const int valid = it.n_tokens - (wave + j * NW) * kBlock;
    const int skip = it.lo - (it.t_begin + (wave + j * NW) * kBlock);
    const int lim = blk_ok ? valid : 0;
    const bool masked = !(blk_ok && valid >= kBlock && skip <= 0);
    const bool row_in = row < lim && row >= skip;
    if (masked) {
      auto in = [&](int e) { return e < lim && e >= skip; };
      const uint32_t mx0 = (in(4 * grp + 0) ? 0x0000ffffu : 0u) | (in(4 * grp + 1) ? 0xffff0000u : 0u);
      const uint32_t mx1 = (in(4 * grp + 2) ? 0x0000ffffu : 0u) | (in(4 * grp + 3) ? 0xffff0000u : 0u);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        vcur[n].x &= mx0;
        vcur[n].y &= mx1;
      }
    }
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      float sc = cols_sum(part[h]) * p.scale_log2;   // s[row][h], same in the row's 4 lanes
      if (masked && !row_in) sc = -INFINITY;
      const float mx = row_max16(sc);                // wave-uniform
      if (mx > m[h]) {
        const float alpha = __builtin_amdgcn_exp2f(m[h] - mx);  // 0 when m was -inf
        l[h] *= alpha;
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[h][n] *= alpha;
        m[h] = mx;
      }
      const float m_ref = m[h] == -INFINITY ? 0.f : m[h];
      const float pr = __builtin_amdgcn_exp2f(sc - m_ref);
      l[h] += pr;
      // weights of tokens 4 grp + r from the lanes of those rows (same grp)
      uint16_t ph[4], pl[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int src = (grp * 16 + 4 * grp + r) * 4;
        const float w = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(pr)));
        Mfma<KVDT>::split(w, ph[r], pl[r]);
      }
      const uint32_t h01 = uint32_t(ph[0]) | (uint32_t(ph[1]) << 16);
      const uint32_t h23 = uint32_t(ph[2]) | (uint32_t(ph[3]) << 16);
      const uint32_t l01 = uint32_t(pl[0]) | (uint32_t(pl[1]) << 16);
      const uint32_t l23 = uint32_t(pl[2]) | (uint32_t(pl[3]) << 16);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        float a = acc[h][n];
        a = Dot2<KVDT>::dot(vcur[n].x, h01, a);
        a = Dot2<KVDT>::dot(vcur[n].y, h23, a);
        a = Dot2<KVDT>::dot(vcur[n].x, l01, a);
        a = Dot2<KVDT>::dot(vcur[n].y, l23, a);
        acc[h][n] = a;
      }
    }
  }
  // full sums: tokens over the row, outputs over the four token groups
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    l[h] = row_sum16(l[h]);
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[h][n] = cols_sum(acc[h][n]);
  }
  __shared__ float sm_m[NW][GM], sm_l[NW][GM];
  __shared__ float sm_o[NW][GM][D];
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      sm_m[wave][h] = m[h];
      sm_l[wave][h] = l[h];
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    float big_m = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) big_m = fmaxf(big_m, sm_m[w][h]);
    const float own = m[h] == -INFINITY ? 0.f : exp2f(m[h] - big_m);
    if (grp == 0) {
#pragma unroll
      for (int n = 0; n < NT; ++n) sm_o[wave][h][16 * n + row] = acc[h][n] * own;
    }
  }
  __syncthreads();
  for (int o = threadIdx.x; o < GM * D; o += 64 * NW) {
    const int h = o / D, dim = o - h * D;
    if (h >= group) continue;
    float big_m = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) big_m = fmaxf(big_m, sm_m[w][h]);
    float big_l = 0.f, a = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = sm_m[w][h];
      big_l += (mw == -INFINITY ? 0.f : exp2f(mw - big_m)) * sm_l[w][h];
      a += sm_o[w][h][dim];
    }
    store_head_result(p, it, g * group + h, dim, a, big_m, big_l, dim == 0, D);
  }
}

// ---------------------------------------------------------------------------
// Decode, generic VALU: one wave per (work item, KV head); any dtype, any
// group size (query heads in passes of up to 4).
//   scores: lane l takes token l%16 and a quarter l/16 of the dimensions;
//           quarters are summed with xor-16/32 shuffles;
//   PV:     lane l owns dims l (+64); probabilities go through LDS.
// ---------------------------------------------------------------------------
constexpr int kValuHeads = 4;

template <int DT, int D>
__global__ __launch_bounds__(64) void decode_valu_kernel(DecodeParams p,
                                                         const int32_t* __restrict__ tables) {
  typedef typename Fmt<DT>::T T;
  constexpr int E = Fmt<DT>::kBytes;
  constexpr int X = 16 / E;
  constexpr int C = D / X;
  constexpr int QC = C / 4;     // chunks per dimension quarter
  constexpr int DL = D / 64;    // dims per lane in PV
  __shared__ float ps[kValuHeads][kBlock];
  const int lane = threadIdx.x;
  const int tok = lane & 15;
  const int quarter = lane >> 4;
  int item_i, g;
  decode_work(p, blockIdx.x, item_i, g);
  const DecodeItem it = decode_item(p, item_i);
  const int32_t* tab = tables + int64_t(it.seq) * p.table_stride + it.t_begin / kBlock;
  const char* kbase = p.pool_k + int64_t(g) * p.p_head;
  const char* vbase = p.pool_v + int64_t(g) * p.p_head;
  const int nblk = (it.n_tokens + kBlock - 1) / kBlock;
  // Fused append: the newest token is written first, each lane storing the
  // K chunks (quarter * QC + c of the slot) and V dims (lane + 64k) that it
  // loads itself below.
  if (p.new_k != nullptr && it.last && it.n_tokens > 0) {
    NewSlot ns = new_slot<DT, DT, D>(p, it, g);
    set_slot_planes(ns, p, tab[(it.n_tokens - 1) / kBlock], g);
    if (ns.ok) {
      if (tok == ns.tin) {
        auto put_k = [&](auto mode_tag) {
          for (int c = 0; c < QC; ++c) {
            KChunkPut<DT, DT, D, decltype(mode_tag)::value> kc;
            kc.load(ns, quarter * QC + c);
            kc.store(ns, quarter * QC + c);
          }
        };
        if (p.rope_mode == PKV_ROPE_PAIRS) put_k(RopeTag<PKV_ROPE_PAIRS>{});
        else if (p.rope_mode == PKV_ROPE_HALVES) put_k(RopeTag<PKV_ROPE_HALVES>{});
        else put_k(RopeTag<PKV_ROPE_NONE>{});
      }
      for (int k = 0; k < DL; ++k) put_v_elem<DT, DT>(ns.vin, ns.v, ns.tin, lane + 64 * k, ns.vsc);
    }
  }

  for (int h0 = 0; h0 < p.group; h0 += kValuHeads) {
    const int nh = min(kValuHeads, p.group - h0);
    // (head loops run to kValuHeads, unrolled, with a uniform i < nh test, so
    // the per-head arrays stay in registers)
    float qv[kValuHeads][QC * X];
#pragma unroll
    for (int i = 0; i < kValuHeads; ++i) {
      const int hq = g * p.group + h0 + min(i, nh - 1);
      const T* qh = reinterpret_cast<const T*>(p.q + (int64_t(it.seq) * p.n_q_heads + hq) * D * E);
#pragma unroll
      for (int c = 0; c < QC; ++c)
#pragma unroll
        for (int e = 0; e < X; ++e) qv[i][c * X + e] = Fmt<DT>::to_f32(qh[(quarter * QC + c) * X + e]);
    }
    float m[kValuHeads], l[kValuHeads], acc[kValuHeads][DL];
#pragma unroll
    for (int i = 0; i < kValuHeads; ++i) {
      m[i] = -INFINITY;
      l[i] = 0.f;
#pragma unroll
      for (int k = 0; k < DL; ++k) acc[i][k] = 0.f;
    }
    // Each block's K chunk elements and V row elements are loaded one block
    // ahead (with its table entry), so their latency overlaps the previous
    // block's arithmetic; rows of more than 256 bytes load in turn.
    constexpr bool PF = D * E <= 256;
    T kraw[QC * X];
    T vraw[DL][kBlock];
    auto load_block = [&](int blk) {
      const bool okb = unsigned(blk) < unsigned(p.num_blocks);
      const char* kp = kbase + int64_t(okb ? blk : 0) * p.p_block;
      const char* vp = vbase + int64_t(okb ? blk : 0) * p.p_block;
#pragma unroll
      for (int c = 0; c < QC; ++c) {
        const T* chunk = reinterpret_cast<const T*>(kp + ((quarter * QC + c) * kBlock + tok) * 16);
#pragma unroll
        for (int e = 0; e < X; ++e) kraw[c * X + e] = chunk[e];
      }
#pragma unroll
      for (int k = 0; k < DL; ++k) {
        const T* vrow = reinterpret_cast<const T*>(vp + int64_t(lane + 64 * k) * kBlock * E);
#pragma unroll
        for (int t = 0; t < kBlock; ++t) vraw[k][t] = vrow[t];
      }
    };
    int blk_next = nblk > 0 ? tab[0] : 0;
    if (PF && nblk > 0) load_block(blk_next);
    for (int bi = 0; bi < nblk; ++bi) {
      const int blk = blk_next;
      if (!PF) load_block(blk);
      const bool ok = unsigned(blk) < unsigned(p.num_blocks);
      const bool live = ok && (bi * kBlock + tok) < it.n_tokens &&
                        it.t_begin + bi * kBlock + tok >= it.lo;
      float kv[QC * X];
#pragma unroll
      for (int e = 0; e < QC * X; ++e) kv[e] = Fmt<DT>::to_f32(kraw[e]);
      float vv[DL][kBlock];
      const int lim = ok ? it.n_tokens - bi * kBlock : 0;  // live tokens of the block
      const int skip = it.lo - (it.t_begin + bi * kBlock);  // before a window's start
#pragma unroll
      for (int k = 0; k < DL; ++k)
#pragma unroll
        for (int t = 0; t < kBlock; ++t)
          vv[k][t] = t < lim && t >= skip ? Fmt<DT>::to_f32(vraw[k][t]) : 0.f;
      if (bi + 1 < nblk) {
        blk_next = tab[bi + 1];
        if (PF) load_block(blk_next);
      }
#pragma unroll
      for (int i = 0; i < kValuHeads; ++i) {
        if (i >= nh) continue;
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < QC * X; ++e) s = fmaf(qv[i][e], kv[e], s);
        s += __shfl_xor(s, 16);
        s += __shfl_xor(s, 32);
        s = live ? s * p.scale_log2 : -INFINITY;
        float mx = s;
        mx = fmaxf(mx, __shfl_xor(mx, 1));
        mx = fmaxf(mx, __shfl_xor(mx, 2));
        mx = fmaxf(mx, __shfl_xor(mx, 4));
        mx = fmaxf(mx, __shfl_xor(mx, 8));
        const float m_new = fmaxf(m[i], mx);
        float pr = 0.f;
        if (m_new != -INFINITY) {
          const float alpha = exp2f(m[i] - m_new);
          pr = exp2f(s - m_new);
          float bsum = pr;
          bsum += __shfl_xor(bsum, 1);
          bsum += __shfl_xor(bsum, 2);
          bsum += __shfl_xor(bsum, 4);
          bsum += __shfl_xor(bsum, 8);
          l[i] = l[i] * alpha + bsum;
#pragma unroll
          for (int k = 0; k < DL; ++k) acc[i][k] *= alpha;
          m[i] = m_new;
        }
        if (lane < kBlock) ps[i][lane] = pr;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < DL; ++k) {
#pragma unroll
        for (int i = 0; i < kValuHeads; ++i) {
          if (i >= nh) continue;
          float a = acc[i][k];
#pragma unroll
          for (int t = 0; t < kBlock; ++t) a = fmaf(ps[i][t], vv[k][t], a);
          acc[i][k] = a;
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < kValuHeads; ++i) {
      if (i >= nh) continue;
      const int hq = g * p.group + h0 + i;
#pragma unroll
      for (int k = 0; k < DL; ++k)
        store_head_result(p, it, hq, lane + 64 * k, acc[i][k], m[i], l[i], lane == 0 && k == 0, D);
    }
  }
}

// ---------------------------------------------------------------------------
// Merge: one wave per (sequence split over several workgroups, query head);
// partial states combined in ascending range order:
//   M = max m_i, L = sum 2^(m_i - M) l_i, out = sum 2^(m_i - M) o_i / L,
//   lse = (M + log2 L) * ln 2.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(const MergeSeq* merges,
                                                          const float* part_o,
                                                          const float* part_ml, float* out,
                                                          float* lse, int n_q_heads) {
  constexpr int DL = D / 64;
  const MergeSeq ms = merges[blockIdx.x];
  const int hq = blockIdx.y;
  const int lane = threadIdx.x;
  float big_m = -INFINITY;
  for (int i = 0; i < ms.count; ++i)
    big_m = fmaxf(big_m, part_ml[(int64_t(ms.first + i) * n_q_heads + hq) * 2]);
  float L = 0.f, o[DL];
#pragma unroll
  for (int k = 0; k < DL; ++k) o[k] = 0.f;
  for (int i = 0; i < ms.count; ++i) {
    const int64_t slot = int64_t(ms.first + i) * n_q_heads + hq;
    const float mi = part_ml[slot * 2];
    const float w = mi == -INFINITY ? 0.f : exp2f(mi - big_m);
    L = fmaf(w, part_ml[slot * 2 + 1], L);
#pragma unroll
    for (int k = 0; k < DL; ++k) o[k] = fmaf(w, part_o[slot * D + lane + 64 * k], o[k]);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int k = 0; k < DL; ++k)
    out[(int64_t(ms.seq) * n_q_heads + hq) * D + lane + 64 * k] = o[k] * inv;
  if (lane == 0 && lse)
    lse[int64_t(ms.seq) * n_q_heads + hq] = L > 0.f ? (big_m + __log2f(L)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// Bandwidth probe
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bw_probe_kernel(const u32x4_t* src, size_t n16,
                                                       u32x4_t* sink) {
  u32x4_t a = {0u, 0u, 0u, 0u};
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; i < n16; i += stride) a ^= __builtin_nontemporal_load(src + i);
  if (a.x == 0x12345678u && a.y == 0x9abcdef0u) sink[0] = a;
}

// ---------------------------------------------------------------------------
// Block copy (copy-on-write).  One workgroup per (pair, layer, K or V): the
// n_kv_heads planes of one layer of the source block, 16 bytes per lane and
// step, streaming loads and stores (each byte is read once and written once).
// ---------------------------------------------------------------------------
struct CopyParams {
  const char* k;      // K base (bytes)
  const char* v;      // V base (bytes)
  int64_t p_layer, p_block, p_head;  // byte strides
  int n_kv_heads;
  int plane_units;    // 16-byte units per plane
  // Per-(layer, block, head) scales of a quantised pool (null otherwise):
  // the copy carries a block's scales with its planes.
  float* k_scale;
  float* v_scale;
  int num_blocks;
};

__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyParams p, CopyBatch b) {
  const int pair = blockIdx.x;
  const int64_t layer_off = int64_t(blockIdx.y) * p.p_layer;
  const char* base = (blockIdx.z == 0 ? p.k : p.v) + layer_off;
  const char* src = base + int64_t(b.src[pair]) * p.p_block;
  char* dst = const_cast<char*>(base) + int64_t(b.dst[pair]) * p.p_block;
  const int units = p.n_kv_heads * p.plane_units;
  for (int u = threadIdx.x; u < units; u += blockDim.x) {
    const int h = u / p.plane_units;
    const int64_t off = int64_t(h) * p.p_head + int64_t(u - h * p.plane_units) * 16;
    st16_stream(dst + off, ld16_stream(src + off));
  }
  float* sc = blockIdx.z == 0 ? p.k_scale : p.v_scale;
  if (sc != nullptr && threadIdx.x < p.n_kv_heads) {
    const int64_t l = int64_t(blockIdx.y) * p.num_blocks;
    sc[(l + b.dst[pair]) * p.n_kv_heads + threadIdx.x] =
        sc[(l + b.src[pair]) * p.n_kv_heads + threadIdx.x];
  }
}

int elem_size(int dtype) {
  return dtype == PKV_F32 ? 4 : dtype == PKV_FP8E4M3 ? 1 : 2;
}

template <typename K, typename P>
hipError_t launch(K kernel, dim3 grid, dim3 block, hipStream_t stream, const P& params) {
  hipLaunchKernelGGL(kernel, grid, block, 0, stream, params);
  return hipGetLastError();
}

// Kernel timing for measurement (this thread's decode launches): when on,
// each launch carries a start/stop event pair attached to its own dispatch,
// so the pair spans the dispatch and the kernel's execution (a few
// microseconds more than a profiler's kernel timestamps).
struct KernelTiming {
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pairs;
};
thread_local KernelTiming g_timing;

template <typename K, typename... A>
hipError_t launch_decode_kernel(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                                bool timed, A... args) {
  if (!g_timing.on || !timed) {
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
    return hipGetLastError();
  }
  hipEvent_t a = nullptr, b = nullptr;
  hipError_t e = hipEventCreate(&a);
  if (e == hipSuccess) e = hipEventCreate(&b);
  if (e != hipSuccess) {
    if (a) (void)hipEventDestroy(a);
    return e;
  }
  hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, a, b, 0, args...);
  e = hipGetLastError();
  g_timing.pairs.emplace_back(a, b);
  return e;
}

// Dynamic LDS that keeps kernel F at one workgroup per CU: enough that two
// workgroups' LDS do not fit in one CU (160 KiB on gfx950).  The one-tile,
// 8-wave decode kernel without the append code fits in 128 VGPRs, so two of
// its workgroups could share a CU; when a launch has only a few workgroups
// per CU, that pins pairs of workgroups together from the start instead of
// handing each CU the next workgroup as it frees (the 8B-shaped layer, 512
// workgroups, measured 8 % slower that way).  Computed once per kernel.
template <auto F>
size_t one_per_cu_lds() {
  static const size_t pad = [] {
    int dev = 0, per_cu = 0;
    hipFuncAttributes fa{};
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                              dev) != hipSuccess ||
        hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(F)) != hipSuccess) {
      (void)hipGetLastError();
      return size_t(0);
    }
    const size_t half = size_t(per_cu) / 2 + 1;
    return fa.sharedSizeBytes < half ? half - fa.sharedSizeBytes : size_t(0);
  }();
  return pad;
}

}  // namespace

// CUs of the current device (cached per device).
int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0) {
      (void)hipGetLastError();
      v = 256;
    }
    cus[dev] = v;
  }
  return cus[dev];
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_inject(const pkv_pool& pool, const pkv_src& src, bool src_in_host_memory,
                         const InjectDesc* d_desc, const InjectDesc* h_desc, int n_desc,
                         int layer_begin, int layer_end, int rope_mode, const float* d_cos,
                         const float* d_sin, hipStream_t stream) {
  const int eb = elem_size(pool.dtype);
  const int sb = elem_size(src.dtype);
  InjectParams p{};
  p.pool_k = static_cast<char*>(pool.k);
  p.pool_v = static_cast<char*>(pool.v);
  p.p_layer = pool.layer_stride * eb;
  p.p_block = pool.block_stride * eb;
  p.p_head = pool.head_stride * eb;
  p.n_kv_heads = pool.n_kv_heads;
  p.k_scale = pool.k_scale;
  p.v_scale = pool.v_scale;
  p.scale_mode = pool.scale_mode;
  p.num_blocks = pool.num_blocks;
  p.src_k = static_cast<const char*>(src.k);
  p.src_v = static_cast<const char*>(src.v);
  p.s_layer = src.layer_stride * sb;
  p.s_token = src.token_stride * sb;
  p.descs = d_desc;
  if (h_desc != nullptr) {
    if (n_desc > kInlineDescs) return hipErrorInvalidValue;
    p.n_inline = n_desc;
    for (int i = 0; i < n_desc; ++i) p.inline_descs[i] = h_desc[i];
  } else if (d_desc == nullptr) {
    return hipErrorInvalidValue;
  }
  p.layer_begin = layer_begin;
  p.layer_end = layer_end;
  p.rope_mode = rope_mode;
  p.cos_t = d_cos;
  p.sin_t = d_sin;
  // Each workgroup walks a few layers of one block, reusing its staged
  // rotary rows; ~50k workgroups measured best on the top-8 injection.
  const int n_layers = layer_end - layer_begin;
  int lpw = int(std::min<int64_t>(n_layers, std::max<int64_t>(1, int64_t(n_layers) * n_desc / 49152)));
  if (const char* env = std::getenv("PKV_INJECT_LAYERS_PER_WG")) {
    const int v = std::atoi(env);
    if (v > 0) lpw = std::min(v, n_layers);
  }
  p.layers_per_wg = lpw;
  dim3 grid(n_desc, (n_layers + lpw - 1) / lpw);
  dim3 block(kInjectThreads);
  (void)src_in_host_memory;  // one walk serves device and pinned host stores
  // The next (layer, head)'s loads issued before the current one is processed
  // (PKV_INJECT_PREFETCH=0: not).
  bool pf = true;
  if (const char* env = std::getenv("PKV_INJECT_PREFETCH")) pf = std::atoi(env) != 0;
#define PKV_INJ(SDT, PDT, DD, F) \
  if (src.dtype == SDT && pool.dtype == PDT && pool.head_dim == DD && pf == F) \
    return launch(inject_rope_kernel<SDT, PDT, DD, 4, F>, grid, block, stream, p);
#define PKV_INJ_H(SDT, PDT, DD) PKV_INJ(SDT, PDT, DD, false) PKV_INJ(SDT, PDT, DD, true)
#define PKV_INJ_D(SDT, PDT) PKV_INJ_H(SDT, PDT, 64) PKV_INJ_H(SDT, PDT, 128)
  PKV_INJ_D(PKV_F32, PKV_F32) PKV_INJ_D(PKV_BF16, PKV_BF16) PKV_INJ_D(PKV_F16, PKV_F16)
  PKV_INJ_D(PKV_BF16, PKV_FP8E4M3) PKV_INJ_D(PKV_F16, PKV_FP8E4M3)
#undef PKV_INJ
#undef PKV_INJ_H
#undef PKV_INJ_D
  return hipErrorInvalidValue;
}

hipError_t launch_append(const pkv_pool& pool, int layer, const int32_t* d_tables,
                         int table_stride, const int32_t* d_first_pos, int n_seqs, int n_new,
                         const void* d_k, const void* d_v, int new_dtype, int rope_mode,
                         const float* d_cos, const float* d_sin, int max_pos,
                         hipStream_t stream) {
  // The inject kernel in append mode: one workgroup per (sequence, block the
  // new tokens can touch, group of 4 KV heads), its descriptor made on the
  // device from the sequence's first position and table row.
  const int eb = elem_size(pool.dtype);
  const int sb = elem_size(new_dtype);
  constexpr int HG = 4;
  InjectParams p{};
  p.pool_k = static_cast<char*>(pool.k);
  p.pool_v = static_cast<char*>(pool.v);
  p.p_layer = pool.layer_stride * eb;
  p.p_block = pool.block_stride * eb;
  p.p_head = pool.head_stride * eb;
  p.n_kv_heads = pool.n_kv_heads;
  p.k_scale = pool.k_scale;
  p.v_scale = pool.v_scale;
  p.scale_mode = pool.scale_mode;
  p.src_k = static_cast<const char*>(d_k);
  p.src_v = static_cast<const char*>(d_v);
  p.s_layer = 0;
  p.s_token = int64_t(pool.n_kv_heads) * pool.head_dim * sb;
  p.layer_begin = layer;
  p.layer_end = layer + 1;
  p.layers_per_wg = 1;
  p.rope_mode = rope_mode;
  p.cos_t = d_cos;
  p.sin_t = d_sin;
  p.app_first = d_first_pos;
  p.app_tables = d_tables;
  p.app_stride = table_stride;
  p.app_n_new = n_new;
  p.app_blocks = (n_new + 2 * kBlock - 2) / kBlock;  // ceil((n_new + 15) / 16)
  p.num_blocks = pool.num_blocks;
  p.max_pos = max_pos;
  if (int64_t(n_seqs) * p.app_blocks > INT32_MAX) return hipErrorInvalidValue;
  dim3 grid(unsigned(n_seqs * p.app_blocks), unsigned((pool.n_kv_heads + HG - 1) / HG));
  dim3 block(kInjectThreads);
#define PKV_APP(SDT, PDT, DD) \
  if (new_dtype == SDT && pool.dtype == PDT && pool.head_dim == DD) \
    return launch(inject_rope_kernel<SDT, PDT, DD, HG, false>, grid, block, stream, p);
#define PKV_APP_D(SDT, PDT) PKV_APP(SDT, PDT, 64) PKV_APP(SDT, PDT, 128)
  PKV_APP_D(PKV_F32, PKV_F32) PKV_APP_D(PKV_BF16, PKV_BF16) PKV_APP_D(PKV_F16, PKV_F16)
  PKV_APP_D(PKV_BF16, PKV_FP8E4M3) PKV_APP_D(PKV_F16, PKV_FP8E4M3)
#undef PKV_APP
#undef PKV_APP_D
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const pkv_pool& pool, int layer, const DecodeArgs& a,
                         int kernel_variant, hipStream_t stream) {
  const int eb = elem_size(pool.dtype);
  DecodeParams p;
  p.pool_k = static_cast<const char*>(pool.k) + int64_t(layer) * pool.layer_stride * eb;
  p.pool_v = static_cast<const char*>(pool.v) + int64_t(layer) * pool.layer_stride * eb;
  p.p_layer = pool.layer_stride * eb;
  p.p_block = pool.block_stride * eb;
  p.p_head = pool.head_stride * eb;
  p.num_blocks = pool.num_blocks;
  p.n_kv_heads = pool.n_kv_heads;
  p.n_q_heads = a.n_q_heads;
  p.group = a.n_q_heads / pool.n_kv_heads;
  p.q = static_cast<const char*>(a.q);
  p.scale_log2 = a.scale * kLog2e;
  p.tables = a.tables;
  p.table_stride = a.table_stride;
  p.items = a.items;
  p.n_items = a.n_items;
  if (a.h_items) {
    if (a.n_items > kInlineItems || a.n_merges > 0) return hipErrorInvalidValue;
    p.items = nullptr;
    for (int i = 0; i < a.n_items; ++i) p.inline_items[i] = a.h_items[i];
  }
  // Items per chunk of the launch order: the longest-first item order is
  // kept from chunk to chunk, and inside a chunk consecutive workgroups take
  // one KV head of consecutive items.  The dispatcher hands consecutive
  // workgroups to the 8 XCDs in turn.  In item-major order (chunks of 1: all
  // heads of an item, then the next item), with a KV-head count that is a
  // multiple of 8, each XCD takes the same heads of every item; in chunks of
  // 8 items each XCD takes all heads of its own items.  Launches of many
  // rounds of workgroups per CU (ragged batches) measured faster in chunks
  // of 8: ragged MHA (64 KV heads, 64 workgroups per CU) 2.13-2.19 against
  // 2.20-2.25 ms per step, chunks of 4 in between, 16 and more slower (32:
  // 2.39).  Launches of one or two rounds keep item-major order, which gives
  // every XCD one head of every item: in chunks of 8 the XCD that takes the
  // first item of each chunk gets the longest items, and the 8B-shaped layer
  // (two rounds) measured 92.4-92.7 against 90.7-91.6 us.  Fully head-major
  // order was the slowest (8B-shaped 5.4 against 6.2 TB/s).
  const bool many_rounds =
      int64_t(a.n_items) * pool.n_kv_heads >= int64_t(16) * device_cus();
  p.chunk = many_rounds ? 8 : 1;
  if (const char* env = std::getenv("PKV_DECODE_CHUNK")) {
    const int v = std::atoi(env);
    if (v > 0) p.chunk = v;
  }
  p.chunk = std::max(1, std::min(p.chunk, std::max(1, a.n_items)));
  p.part_o = a.part_o;
  p.part_ml = a.part_ml;
  p.out = a.out;
  p.lse = a.lse;
  // this layer's scales: [heads], or [num_blocks][heads] per block
  const int64_t per_layer = int64_t(pool.scale_mode == 1 ? pool.num_blocks : 1) * pool.n_kv_heads;
  p.k_scale = pool.k_scale ? pool.k_scale + int64_t(layer) * per_layer : nullptr;
  p.v_scale = pool.v_scale ? pool.v_scale + int64_t(layer) * per_layer : nullptr;
  p.scale_mode = pool.scale_mode;
  p.new_k = static_cast<const char*>(a.new_k);
  p.new_v = static_cast<const char*>(a.new_v);
  p.rope_mode = a.rope_mode;
  p.cos_t = a.cos_t;
  p.sin_t = a.sin_t;
  p.max_pos = a.max_pos;
  hipError_t e = hipSuccess;
  if (a.n_items > 0) {
    dim3 grid(unsigned(a.n_items) * unsigned(pool.n_kv_heads));
    // variant: 0 automatic, 1 generic VALU kernel (not for fp8 pools), 2 packed
    // dot products on the VALU where they apply (decode_dot2_kernel), 10 + k
    // MFMA kernel with a prefetch depth of k blocks (k = 1, 2; for attention
    // alone with one tile, 8 waves and a 16-bit pool, depth 2 stages K and V
    // through LDS by direct loads).
    // Tiles of 16 query heads per KV head: groups up to 64 run on MFMA.
    const int ng = p.group <= 16 ? 1 : p.group <= 32 ? 2 : p.group <= 64 ? 4 : 0;
    const bool mfma = (kernel_variant != 1 || pool.dtype == PKV_FP8E4M3) &&
                      pool.dtype != PKV_F32 && ng > 0;
    // More tiles hold more accumulators: 2 tiles fit 8 waves per workgroup
    // (two per SIMD), 4 tiles one wave per SIMD.
    int nw = a.waves;
    if (ng == 2) nw = nw >= 8 ? 8 : 4;
    if (ng == 4) nw = 4;
    // The decode step's append (new token rows given) runs the PUT instance,
    // an fp8 pool with per-block scales the BLK one.  Exception: a 16-bit
    // pool's one-tile, 8-wave launch of at least 16 workgroups per CU (ragged
    // batches of short sequences) appends in a launch of its own first and
    // then runs attention alone, which gives the same bytes and outputs.
    // That PUT instance needs more than 128 VGPRs, so one of its workgroups
    // fits per CU, where attention alone runs two and hides each one's
    // start-up behind the other's loads; on ragged MHA (16,384 workgroups)
    // the two launches measured 2.14 ms against 2.22 ms for one (on the
    // 8B-shaped layer, 512 workgroups, one launch is the faster: 100 against
    // 106 us).
    bool put = a.new_k != nullptr;
    if (put && mfma && ng == 1 && nw == 8 && pool.dtype != PKV_FP8E4M3 && a.put_pos &&
        grid.x >= 16u * unsigned(device_cus())) {
      e = launch_append(pool, layer, a.tables, a.table_stride, a.put_pos, a.n_seqs, 1, a.new_k,
                        a.new_v, a.q_dtype, a.rope_mode, a.cos_t, a.sin_t, a.max_pos, stream);
      if (e != hipSuccess) return e;
      put = false;
      p.new_k = p.new_v = nullptr;
    }
    const bool blk = pool.dtype == PKV_FP8E4M3 && pool.scale_mode == 1;
    // One block in flight per wave measured fastest with 8 waves per workgroup
    // (depth 2 is instantiated for attention alone only).
    const int depth = kernel_variant == 12 && !put ? 2 : 1;
    // 8-wave launches with fewer than 16 workgroups per CU run one workgroup
    // per CU (see one_per_cu_lds); many-workgroup launches (ragged batches)
    // may run two, which hides each workgroup's start-up behind another's
    // loads.  Launches of fewer waves per workgroup are left alone: they need
    // several workgroups per CU to fill it.
    const bool one_per_cu = nw == 8 && grid.x < 16u * unsigned(device_cus());
    bool launched = false;
#define PKV_DEC_MFMA(KV, Q, DD, DEP, W, G)                                                   \
    if (!launched && mfma && pool.dtype == KV && a.q_dtype == Q && pool.head_dim == DD &&    \
        depth == DEP && nw == W && ng == G) {                                                \
      constexpr bool B8 = KV == PKV_FP8E4M3; /* per-block scales exist for fp8 only */       \
      if (put && blk) {                                                                      \
        constexpr auto k = decode_mfma_kernel<KV, Q, DD, DEP, W, G, DEP == 1, B8>;           \
        e = launch_decode_kernel(k, grid, dim3(64 * W), one_per_cu ? one_per_cu_lds<k>() : 0, \
                                 stream, a.timed, p, p.tables);                              \
      } else if (put) {                                                                      \
        constexpr auto k = decode_mfma_kernel<KV, Q, DD, DEP, W, G, DEP == 1, false>;        \
        e = launch_decode_kernel(k, grid, dim3(64 * W), one_per_cu ? one_per_cu_lds<k>() : 0, \
                                 stream, a.timed, p, p.tables);                              \
      } else if (blk) {                                                                      \
        constexpr auto k = decode_mfma_kernel<KV, Q, DD, DEP, W, G, false, B8>;              \
        e = launch_decode_kernel(k, grid, dim3(64 * W), one_per_cu ? one_per_cu_lds<k>() : 0, \
                                 stream, a.timed, p, p.tables);                              \
      } else {                                                                               \
        constexpr auto k = decode_mfma_kernel<KV, Q, DD, DEP, W, G, false, false>;           \
        e = launch_decode_kernel(k, grid, dim3(64 * W), one_per_cu ? one_per_cu_lds<k>() : 0, \
                                 stream, a.timed, p, p.tables);                              \
      }                                                                                      \
      launched = true;                                                                       \
    }
#define PKV_DEC_MFMA_W(KV, Q, DD, DEP) \
    PKV_DEC_MFMA(KV, Q, DD, DEP, 1, 1) PKV_DEC_MFMA(KV, Q, DD, DEP, 2, 1) \
    PKV_DEC_MFMA(KV, Q, DD, DEP, 4, 1) PKV_DEC_MFMA(KV, Q, DD, DEP, 8, 1)
#define PKV_DEC_MFMA_G(KV, Q, DD) \
    PKV_DEC_MFMA(KV, Q, DD, 1, 4, 2) PKV_DEC_MFMA(KV, Q, DD, 1, 8, 2) \
    PKV_DEC_MFMA(KV, Q, DD, 1, 4, 4)
#define PKV_DEC_MFMA_ALL(KV, Q) \
    PKV_DEC_MFMA_W(KV, Q, 64, 1) PKV_DEC_MFMA_W(KV, Q, 64, 2) \
    PKV_DEC_MFMA_W(KV, Q, 128, 1) PKV_DEC_MFMA_W(KV, Q, 128, 2) \
    PKV_DEC_MFMA_G(KV, Q, 64) PKV_DEC_MFMA_G(KV, Q, 128)
#define PKV_DEC_VALU(DT, DD)                                                                 \
    if (!launched && pool.dtype == DT && pool.head_dim == DD) {                              \
      e = launch_decode_kernel(decode_valu_kernel<DT, DD>, grid, dim3(64), 0, stream,        \
                               a.timed, p, p.tables);                                        \
      launched = true;                                                                       \
    }
    // variant 2: packed dot products on the VALU for small query groups
    // (attention alone, 8-wave workgroups)
    const bool dot2 = kernel_variant == 2 && !put && p.group <= 4 && nw == 8 &&
                      (pool.dtype == PKV_BF16 || pool.dtype == PKV_F16) && a.q_dtype == pool.dtype;
#define PKV_DEC_DOT2(KV, DD, GG)                                                             \
    if (!launched && dot2 && pool.dtype == KV && pool.head_dim == DD &&                      \
        (GG == 4 ? p.group > 2 : GG == 2 ? p.group == 2 : p.group == 1)) {                   \
      constexpr auto k = decode_dot2_kernel<KV, DD, 8, GG>;                                  \
      e = launch_decode_kernel(k, grid, dim3(512), one_per_cu ? one_per_cu_lds<k>() : 0,      \
                               stream, a.timed, p, p.tables);                                \
      launched = true;                                                                       \
    }
#define PKV_DEC_DOT2_G(KV, DD) PKV_DEC_DOT2(KV, DD, 1) PKV_DEC_DOT2(KV, DD, 2) PKV_DEC_DOT2(KV, DD, 4)
    PKV_DEC_DOT2_G(PKV_BF16, 64) PKV_DEC_DOT2_G(PKV_BF16, 128)
    PKV_DEC_DOT2_G(PKV_F16, 64) PKV_DEC_DOT2_G(PKV_F16, 128)
#undef PKV_DEC_DOT2
#undef PKV_DEC_DOT2_G
    PKV_DEC_MFMA_ALL(PKV_BF16, PKV_BF16) PKV_DEC_MFMA_ALL(PKV_F16, PKV_F16)
    PKV_DEC_MFMA_ALL(PKV_FP8E4M3, PKV_BF16) PKV_DEC_MFMA_ALL(PKV_FP8E4M3, PKV_F16)
    PKV_DEC_VALU(PKV_F32, 64) PKV_DEC_VALU(PKV_F32, 128) PKV_DEC_VALU(PKV_BF16, 64)
    PKV_DEC_VALU(PKV_BF16, 128) PKV_DEC_VALU(PKV_F16, 64) PKV_DEC_VALU(PKV_F16, 128)
#undef PKV_DEC_MFMA
#undef PKV_DEC_MFMA_W
#undef PKV_DEC_MFMA_G
#undef PKV_DEC_MFMA_ALL
#undef PKV_DEC_VALU
    if (!launched) return hipErrorInvalidValue;
    if (e != hipSuccess) return e;
  }
  if (a.n_merges > 0) {
    dim3 grid(a.n_merges, a.n_q_heads);
    if (pool.head_dim == 64)
      hipLaunchKernelGGL(decode_merge_kernel<64>, grid, dim3(64), 0, stream, a.merges, a.part_o,
                         a.part_ml, a.out, a.lse, a.n_q_heads);
    else
      hipLaunchKernelGGL(decode_merge_kernel<128>, grid, dim3(64), 0, stream, a.merges,
                         a.part_o, a.part_ml, a.out, a.lse, a.n_q_heads);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_copy_blocks(const pkv_pool& pool, const CopyBatch& batch, hipStream_t stream) {
  if (batch.n <= 0) return hipSuccess;
  const int eb = elem_size(pool.dtype);
  CopyParams p;
  p.k = static_cast<const char*>(pool.k);
  p.v = static_cast<const char*>(pool.v);
  p.p_layer = pool.layer_stride * eb;
  p.p_block = pool.block_stride * eb;
  p.p_head = pool.head_stride * eb;
  p.n_kv_heads = pool.n_kv_heads;
  p.plane_units = kBlock * pool.head_dim * eb / 16;
  const bool blockwise = pool.dtype == PKV_FP8E4M3 && pool.scale_mode == 1;
  p.k_scale = blockwise ? const_cast<float*>(pool.k_scale) : nullptr;
  p.v_scale = blockwise ? const_cast<float*>(pool.v_scale) : nullptr;
  p.num_blocks = pool.num_blocks;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(batch.n, pool.n_layers, 2), dim3(256), 0, stream,
                     p, batch);
  return hipGetLastError();
}

void set_kernel_timing(bool on) { g_timing.on = on; }

int collect_kernel_times(float* ms_out, int max_n, hipError_t* err) {
  int n = 0;
  *err = hipSuccess;
  for (auto& pr : g_timing.pairs) {
    float ms = -1.f;
    hipError_t e = hipEventSynchronize(pr.second);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, pr.first, pr.second);
    if (e != hipSuccess && *err == hipSuccess) *err = e;
    if (ms_out && n < max_n) ms_out[n] = ms;
    ++n;
    (void)hipEventDestroy(pr.first);
    (void)hipEventDestroy(pr.second);
  }
  g_timing.pairs.clear();
  return n;
}

hipError_t scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));  // with this device current
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_bw_probe(const void* src, size_t n_bytes, void* sink, hipStream_t stream) {
  const size_t n16 = n_bytes / 16;
  const int blocks = 2048;  // measured best for a streaming read on 256 CUs
  hipLaunchKernelGGL(bw_probe_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const u32x4_t*>(src), n16, static_cast<u32x4_t*>(sink));
  return hipGetLastError();
}

}  // namespace pkv
