// Internal interface between the host runtime (pkv_host.cpp) and the HIP
// kernels (pkv_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pkv.h"

namespace pkv {

constexpr int kBlock = PKV_BLOCK_TOKENS;

// Write plan of one destination block for an inject call: the physical block,
// the logical position of its first slot, and for each of its 16 slots the
// source token to write there (-1: leave the slot as it is).
struct InjectDesc {
  int32_t phys_block;
  int32_t pos_base;
  int32_t src[kBlock];
};
static_assert(sizeof(InjectDesc) == 72, "descriptor layout");

// One decode work item: tokens [t_begin, t_begin + n_tokens) of sequence seq
// (t_begin a multiple of 16).  slot < 0: the item covers the whole sequence
// (an empty one included) and writes the final output; otherwise it stores
// its partial softmax state in partial slot `slot`, merged afterwards.
struct DecodeItem {
  int32_t seq;
  int32_t t_begin;   // first position of the range (a multiple of 16)
  int32_t n_tokens;  // positions t_begin .. t_begin + n_tokens - 1
  int32_t slot;      // partial-result slot, or -1 for a final result
  int32_t lo;        // first position attended (a sliding window's start)
  int32_t last;      // 1 if the range ends at the sequence's last position
};

// Plans of at most kInlineItems work items with no split sequence (and not
// run as an append launch plus attention) travel in the decode kernel's
// arguments: no device copy of the work list is made for them.
constexpr int kInlineItems = 128;

// Merge work: sequence seq owns partial slots [first, first + count).
struct MergeSeq {
  int32_t seq;
  int32_t first;
  int32_t count;
  int32_t _pad;
};

// Calls of at most kInlineDescs descriptors pass them in the kernel
// arguments (h_desc: host memory, read at the launch) instead of a device copy
// (d_desc); exactly one of the two is used.
constexpr int kInlineDescs = 4;
hipError_t launch_inject(const pkv_pool& pool, const pkv_src& src, bool src_in_host_memory,
                         const InjectDesc* d_desc, const InjectDesc* h_desc, int n_desc,
                         int layer_begin, int layer_end, int rope_mode, const float* d_cos,
                         const float* d_sin, hipStream_t stream);

hipError_t launch_append(const pkv_pool& pool, int layer, const int32_t* d_tables,
                         int table_stride, const int32_t* d_first_pos, int n_seqs, int n_new,
                         const void* d_k, const void* d_v, int new_dtype, int rope_mode,
                         const float* d_cos, const float* d_sin, int max_pos,
                         hipStream_t stream);

struct DecodeArgs {
  const void* q;
  int q_dtype;
  int n_q_heads;
  float scale;
  const int32_t* tables;
  int table_stride;
  const DecodeItem* items;
  // Host copy of the work list when the plan travels in the kernel
  // arguments (then items is unused); null otherwise.
  const DecodeItem* h_items;
  int n_items;
  const MergeSeq* merges;
  int n_merges;
  int waves;       // waves per workgroup sharing one item (1, 2, 4 or 8)
  float* part_o;   // [n_slots][n_q_heads][head_dim]
  float* part_ml;  // [n_slots][n_q_heads][2]
  float* out;
  float* lse;      // may be null
  // Fused append of each sequence's newest token (position len - 1) before
  // it is attended: rows [n_seqs][n_kv_heads][head_dim] in the query's
  // format, unrotated; null when no token is appended.
  const void* new_k;
  const void* new_v;
  int rope_mode;
  const float* cos_t;
  const float* sin_t;
  int max_pos;
  // Each sequence's newest position (lens - 1, -1 for an empty sequence),
  // device int32[n_seqs] in the workspace: for launches that append in a
  // launch of their own before attention alone.
  const int32_t* put_pos;
  int n_seqs;
  // false: never attach timing events (the allocation-free entry point)
  bool timed;
};

// kernel_variant: 0 = automatic, 1 = force the generic VALU kernel.
hipError_t launch_decode(const pkv_pool& pool, int layer, const DecodeArgs& a,
                         int kernel_variant, hipStream_t stream);

// Compute units of the current device (cached per device; 256 when no device
// answers).
int device_cus();

hipError_t launch_bw_probe(const void* src, size_t n_bytes, void* sink, hipStream_t stream);

// Workspace of the allocation-free decode step: a file-scope device array of
// kScratchBytes in pkv_kernels.hip, one copy per device.
constexpr size_t kScratchBytes = size_t(PKV_NOALLOC_SCRATCH_BYTES);
static_assert(kScratchBytes % 256 == 0, "scratch size");
// Device address of the current device's copy, looked up (hipGetSymbolAddress)
// on the first call per device and kept; never the array's host-side name.
hipError_t scratch_address(void** out);

// Measurement: dispatch-attached timing of this thread's decode launches.
void set_kernel_timing(bool on);
// Waits for the recorded launches, writes up to max_n durations (ms) in launch
// order, drops them all and returns how many there were; *err holds the
// first HIP error met.
int collect_kernel_times(float* ms_out, int max_n, hipError_t* err);

// Copy-on-write copies handed to one launch (a kernel argument, no device
// staging): pairs i < n copy every layer's K and V planes of block src[i]
// into block dst[i].  No two pairs of a batch may touch a common block as
// destination, or as source of one and destination of another.
constexpr int kCopyBatch = 256;
struct CopyBatch {
  int32_t n;
  int32_t src[kCopyBatch];
  int32_t dst[kCopyBatch];
};
hipError_t launch_copy_blocks(const pkv_pool& pool, const CopyBatch& batch, hipStream_t stream);

}  // namespace pkv
