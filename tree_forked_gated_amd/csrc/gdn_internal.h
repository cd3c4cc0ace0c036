// Internal declarations shared by the HIP sources of the gdn_tree library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_tree.h"

namespace gdn {

constexpr int kChunk = GDN_TREE_CHUNK;  // rows of one tree-WY chunk
constexpr int kThreads = 256;           // workgroup of the walk: four wave64s
constexpr unsigned long long kNoError = ~0ull;
constexpr int kUnmapped = 0x7fffffff;  // out_map / state_map entry of a token nobody asked for

// Error word: the smallest (code << 32 | index) any kernel raised.
__device__ inline void raise_error(unsigned long long* err, int code, long long index) {
  atomicMin(err, ((unsigned long long)(unsigned)code << 32) | (unsigned long long)(uint32_t)index);
}

// Device pointers into a forward workspace (see gdn_tree_layout for the public part).
struct Meta {
  unsigned long long* err;
  int* n_seg;
  int* n_fork;
  int* tok_seq;
  int* depth;
  int* fork_slot;
  int* seg_start;
  int* seg_len;
  int* seg_seq;
  int* seg_mode;
  int* seg_entry;
  int* seg_slot;
  int* seg_level;
  int* level_count;
  int* level_ptr;
  int* level_items;
  unsigned long long* tree_mask;
  float* fork_states;
  // internal tables
  int* is_start;
  int* is_fork;
  int* out_map;
  int* state_map;
  int* seg_depth0;
  int* level_fill;  // [max_levels][kLenBuckets] entries placed so far
  int* level_bkt;   // [max_levels][kLenBuckets] segments per length bucket
  int* walk_ctr;    // [max_levels][kSchedInts]: the walk's work counters, then fewest and most chunks of a segment
  int* scan_sums;  // [2 * n_scan_blocks] block totals, then their exclusive offsets
  unsigned long long* plan_tag;  // fingerprint of the sizes the metadata was built for
  int4* unit_info;  // per level entry (level_items order): {start, len, mode | seq << 1, fork slot}
};

constexpr int kScanTile = 1024;  // tokens per block of the metadata scans (four per thread)
constexpr int kWalkQueues = 8;  // work counters per level: one per XCD of the walk's grid
constexpr int kSchedInts = kWalkQueues + 2;  // per level: the counters, the fewest and the most chunks of a segment
// Each level lists its segments longest first, by chunk count (bucket 0: 63 or
// more chunks, bucket 63 - c: c chunks), so that the walk's queues start the
// longest items first.
constexpr int kLenBuckets = 64;
__host__ __device__ inline int len_bucket(int nchunks) { return kLenBuckets - 1 - (nchunks < kLenBuckets - 1 ? nchunks : kLenBuckets - 1); }

struct LayoutFull {
  gdn_tree_layout pub;
  size_t is_start, is_fork, out_map, state_map, seg_depth0, level_fill, level_bkt, walk_ctr, scan_sums, plan_tag, unit_info;
  int n_scan_blocks;
};

// Host: byte offsets of every table for these sizes (256-byte aligned).
bool compute_layout(const gdn_tree_dims& d, LayoutFull* L);
Meta meta_from(void* workspace, const LayoutFull& L);

// Per-process caches of device queries (host): the compute-unit count of the
// current device, and the dynamic-LDS attribute of a kernel, set once per
// (kernel, device), with its occupancy at `threads` threads when asked for
// (occupancy may be NULL). Thread safe; a race only repeats idempotent calls.
hipError_t current_device_cus(int* cus);
hipError_t ensure_dynamic_lds(const void* kernel, int bytes, int threads, int* occupancy);

// Host launchers (enqueue only). Return hipSuccess or the launch error.
hipError_t launch_plan(const gdn_tree_fwd_args& a, const Meta& m, const LayoutFull& L, unsigned long long tag,
                       hipStream_t s);
// Before a walk over an already planned workspace: checks the fingerprint and
// clears the walk's work counters.
hipError_t launch_replan_check(const Meta& m, int max_levels, unsigned long long tag, hipStream_t s);
// Fingerprint of the sizes a plan depends on (never 0).
unsigned long long plan_fingerprint(const gdn_tree_fwd_args& a);
hipError_t launch_walk(const gdn_tree_fwd_args& a, const Meta& m, int bv, hipStream_t s);
hipError_t launch_commit(const gdn_tree_commit_args& a, unsigned long long* err, hipStream_t s);
bool walk_supported(int dtype, int dk, int bv);
// Pipelined MFMA walk for bf16 inputs with d_k = 128 (d_v tiles of 16, 32 or 64
// columns): state waves plus helper waves
bool walk_pipe_supported(int dtype, int dk, int bv);
hipError_t launch_walk_pipe(const gdn_tree_fwd_args& a, const Meta& m, int bv, hipStream_t s);
int walk_lds_bytes(int dtype, int dk, int bv);

// ForkAttention (attention.hip): the workspace is the planner's layout for the
// stream (without fork-state slots), then the attention's item and span tables.
struct AttnLayout {
  LayoutFull plan;
  gdn_tree_dims pd;  // the sizes the planner runs with
  size_t item_info, spans, item_off, n_items, claim, total;
};
bool attn_layout(const gdn_attn_dims& d, AttnLayout* A);
hipError_t launch_attention(const gdn_attn_args& a, const AttnLayout& A, hipStream_t s);
int attn_max_spans();

// Fused chain round (chain.hip).
hipError_t launch_chain(const gdn_chain_args& c, hipStream_t s);
int chain_dyn_lds(int N, int dk);

}  // namespace gdn
