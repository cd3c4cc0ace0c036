// Commit by reconstruction (TreeWY, "Speculative Verification for Gated
// DeltaNet Hybrids", section 3 "Reconstruct on commit", Eq. 3):
//
//   S_a = g_a S_0 + sum over i on the root path of a (a included) of (g_a / g_i) vt_i k_i^T
//
// g_a / g_i = exp(sum of the log gates strictly after i on the path) and g_a =
// exp of the whole path's sum. The path is taken from its root in tiles of 16
// nodes, so the sum is the same recurrence tile by tile:
//
//   S <- exp(sum of the tile's log gates) S + sum over i in the tile of exp(sum of its log gates after i) vt_i k_i^T
//
// starting from S_0, all in fp32. One workgroup per (path, head, 32 rows of S):
// it reads S_0 once, the path's pseudo-values, keys and gates, and writes S_a
// once. The kernel is bound by those two state streams (HBM), so it stays on
// plain fp32 FMAs with 16-byte loads and stores, and holds the rows of S in one
// set of registers (eight workgroups fit on a CU).
#include "gdn_internal.h"

namespace gdn {
namespace {

// S_0 and S_a are streamed once: nontemporal loads and stores keep them from
// displacing cached data (measured 15% faster on 64 paths x 32 heads).
typedef float f32x4n __attribute__((ext_vector_type(4)));
constexpr int kRows = 32;      // rows of S per workgroup
constexpr int kPathTile = 16;  // path nodes staged in LDS at a time
constexpr int kThreads = 256;
constexpr int kPer4 = kRows * 128 / 4 / kThreads;  // float4 groups of the block per thread (d_k <= 128)

struct CommitArgs {
  const void* k;
  const void* g;
  const int* parent;
  const int* seq_start;
  const float* init;
  const float* pv;
  const int* path_ptr;
  const int* path_nodes;
  const int* path_seq;
  float* out;
  unsigned long long* err;
  int H, Dk, Dv, n_seq, T;
  int n_path;
  int own_err;  // 1: workgroup (0, 0, 0) checks every path and stores the error word itself
};

__device__ inline float upc(__bf16 x) { return (float)x; }
__device__ inline float upc(float x) { return x; }

__global__ void k_reset(unsigned long long* err) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *err = kNoError;
}

// Is path p a parent chain from a root of its sequence down to its last node?
// Every index is checked before it is used; the nodes' loads do not wait for
// the verdict on the nodes before them.
__device__ inline bool path_ok(const CommitArgs& a, int p) {
  const int seq = a.path_seq[p];
  const int beg = a.path_ptr[p], end = a.path_ptr[p + 1];
  if (seq < 0 || seq >= a.n_seq || end < beg) return false;
  if (end == beg) return true;
  const int s_0 = a.seq_start[seq], s_1 = a.seq_start[seq + 1];
  if (s_0 < 0 || s_1 > a.T || s_1 <= s_0) return false;
  bool ok = true;
  int want = -1;
#pragma unroll 4
  for (int j = beg; j < end; ++j) {
    const int t = a.path_nodes[j];
    const bool in = t >= s_0 && t < s_1;
    ok &= in && a.parent[in ? t : s_0] == want;
    want = t;
  }
  return ok;
}

// The error word of a call with few paths: the smallest bad path, found by one
// workgroup (one path per thread at a time) and stored without atomics, so the
// word needs no reset before the call.
__device__ inline void check_all_paths(const CommitArgs& a) {
  __shared__ int s_first;
  if (threadIdx.x == 0) s_first = 0x7fffffff;
  __syncthreads();
  for (int p = threadIdx.x; p < a.n_path; p += blockDim.x)
    if (!path_ok(a, p)) atomicMin(&s_first, p);
  __syncthreads();
  if (threadIdx.x == 0)
    *a.err = s_first == 0x7fffffff ? kNoError
                                   : (((unsigned long long)(unsigned)GDN_DEV_PATH << 32) | (unsigned)s_first);
}

// One workgroup per (path, head, 32 rows of S). The rows of S_0 are requested
// first, so that they arrive while the path is staged. The path is staged in
// LDS 16 nodes at a time from its root: each node is checked (in its sequence,
// parent = previous node) in the same pass that loads its key, pseudo-values
// and gate. Until the check is decided, a node's index is clamped into [0, T)
// for those loads, so that they need not wait for the sequence's range; the
// verdict is taken before any store.
template <typename E>
__global__ void __launch_bounds__(kThreads, 8) k_commit(CommitArgs a) {
  constexpr int kEPer = 16 / sizeof(E);  // key elements per 16-byte piece
  __shared__ __attribute__((aligned(16))) float sK[kPathTile][128 + 4];
  __shared__ __attribute__((aligned(16))) float sV[kPathTile][kRows];
  __shared__ float sG[kPathTile];
  __shared__ float sW[kPathTile + 1];  // the nodes' weights, then the tile's decay
  const int p = blockIdx.x, h = blockIdx.y, vb = blockIdx.z;
  const int tid = threadIdx.x;
  const int Dk = a.Dk, H = a.H, Dv = a.Dv;
  const int per_row4 = Dk / 4;
  const int n4 = kRows * per_row4;  // float4 groups in the block
  const int rows = min(kRows, Dv - vb * kRows);
  const size_t SS = (size_t)Dv * Dk;
  const int seq = a.path_seq[p];
  const int beg = a.path_ptr[p], end = a.path_ptr[p + 1];
  const bool bad_path = (seq < 0 || seq >= a.n_seq || end < beg);
  bool bad = bad_path;
  // S starts as the S_0 rows of this block (zeros without initial states)
  float4 acc[kPer4];
  const float* S0 = (!bad_path && a.init) ? a.init + ((size_t)seq * H + h) * SS : nullptr;
#pragma unroll
  for (int i = 0; i < kPer4; ++i) {
    const int gidx = tid + kThreads * i;
    const int r = gidx / per_row4, d = (gidx % per_row4) * 4;
    f32x4n v = {0.f, 0.f, 0.f, 0.f};
    if (S0 && gidx < n4 && r < rows) v = __builtin_nontemporal_load(reinterpret_cast<const f32x4n*>(S0 + (size_t)(vb * kRows + r) * Dk + d));
    acc[i] = make_float4(v[0], v[1], v[2], v[3]);
  }
  const E* kg = reinterpret_cast<const E*>(a.k);
  const E* gg = reinterpret_cast<const E*>(a.g);
  const int s_0 = bad_path ? 0 : a.seq_start[seq], s_1 = bad_path ? 0 : a.seq_start[seq + 1];
  const int last = a.T - 1;  // a.T > 0 whenever a path has nodes that pass the check
  const int kpieces = Dk / kEPer;  // 16-byte pieces of a key row
  const int vpieces = rows / 4;    // float4 pieces of the block's pseudo-value rows
  const int n_nodes = (bad_path || a.T <= 0) ? 0 : end - beg;
  for (int tile_beg = beg; tile_beg < beg + n_nodes; tile_beg += kPathTile) {
    const int nt = min(kPathTile, beg + n_nodes - tile_beg);
    if (tid < nt) {  // check the node and load its gate
      const int j = tile_beg + tid;
      const int t = a.path_nodes[j];
      const int want = (j == beg) ? -1 : a.path_nodes[j - 1];
      const int tc = min(max(t, 0), last);
      bad |= !(t >= s_0 && t < s_1 && a.parent[tc] == want);
      sG[tid] = upc(gg[(size_t)tc * H + h]);
    }
    if (tid < nt * kpieces) {  // one 16-byte piece of a key row per thread
      const int j = tid / kpieces, c = tid % kpieces;
      const int tc = min(max(a.path_nodes[tile_beg + j], 0), last);
      const uint4 raw = *reinterpret_cast<const uint4*>(kg + ((size_t)tc * H + h) * Dk + c * kEPer);
      const E* e = reinterpret_cast<const E*>(&raw);
#pragma unroll
      for (int x = 0; x < kEPer; x += 4)
        *reinterpret_cast<float4*>(&sK[j][c * kEPer + x]) = make_float4(upc(e[x]), upc(e[x + 1]), upc(e[x + 2]), upc(e[x + 3]));
    }
    if (tid < nt * (kRows / 4)) {  // one float4 of a pseudo-value row per thread
      const int j = tid / (kRows / 4), c = tid % (kRows / 4);
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c < vpieces) {
        const int tc = min(max(a.path_nodes[tile_beg + j], 0), last);
        v = *reinterpret_cast<const float4*>(a.pv + ((size_t)tc * H + h) * Dv + vb * kRows + 4 * c);
      }
      *reinterpret_cast<float4*>(&sV[j][4 * c]) = v;
    }
    __syncthreads();
    if (tid == 0) {  // weights exp(sum of the tile's log gates after node j), from the tile's end
      float sigma = 0.f;
      for (int j = nt - 1; j >= 0; --j) {
        sW[j] = __expf(sigma);
        sigma += sG[j];
      }
      sW[kPathTile] = __expf(sigma);
    }
    __syncthreads();
    const float dec = sW[kPathTile];
#pragma unroll
    for (int i = 0; i < kPer4; ++i) {
      const int gidx = tid + kThreads * i;
      if (gidx < n4) {
        const int r = gidx / per_row4, d = (gidx % per_row4) * 4;
        float4 s = acc[i];
        s.x *= dec;
        s.y *= dec;
        s.z *= dec;
        s.w *= dec;
        for (int j = 0; j < nt; ++j) {
          const float wv = sW[j] * sV[j][r];
          const float4 kk = *reinterpret_cast<const float4*>(&sK[j][d]);
          s.x += wv * kk.x;
          s.y += wv * kk.y;
          s.z += wv * kk.z;
          s.w += wv * kk.w;
        }
        acc[i] = s;
      }
    }
    __syncthreads();
  }
  // a non-empty path needs a non-empty sequence inside [0, T)
  if (!bad_path && end > beg && (s_1 <= s_0 || s_0 < 0 || s_1 > a.T)) bad = true;
  if (a.own_err && p == 0 && h == 0 && vb == 0) check_all_paths(a);
  if (__syncthreads_or(bad)) {
    if (tid == 0 && !a.own_err) raise_error(a.err, GDN_DEV_PATH, p);
    return;
  }
  float* dst = a.out + ((size_t)p * H + h) * SS;
#pragma unroll
  for (int i = 0; i < kPer4; ++i) {
    const int gidx = tid + kThreads * i;
    const int r = gidx / per_row4, d = (gidx % per_row4) * 4;
    if (gidx < n4 && r < rows) {
      const f32x4n ov = {acc[i].x, acc[i].y, acc[i].z, acc[i].w};
      __builtin_nontemporal_store(ov, reinterpret_cast<f32x4n*>(dst + (size_t)(vb * kRows + r) * Dk + d));
    }
  }
}

}  // namespace

hipError_t launch_commit(const gdn_tree_commit_args& c, unsigned long long* err, hipStream_t s) {
  CommitArgs a;
  a.k = c.k;
  a.g = c.log_gate;
  a.parent = c.parent_idx;
  a.seq_start = c.seq_start;
  a.init = c.init_state;
  a.pv = c.pseudo_v;
  a.path_ptr = c.path_ptr;
  a.path_nodes = c.path_nodes;
  a.path_seq = c.path_seq;
  a.out = c.out_state;
  a.err = err;
  a.H = c.dims.H;
  a.Dk = c.dims.Dk;
  a.Dv = c.dims.Dv;
  a.n_seq = c.dims.n_seq;
  a.T = (int)c.dims.T;
  a.n_path = c.n_path;
  // With up to kOwnErrPaths paths one workgroup of the commit decides the error
  // word by itself; otherwise the word is reset first and raised by atomics.
  constexpr int kOwnErrPaths = 1024;
  a.own_err = c.n_path > 0 && c.n_path <= kOwnErrPaths;
  if (!a.own_err) hipLaunchKernelGGL(k_reset, dim3(1), dim3(64), 0, s, err);
  if (c.n_path > 0) {
    dim3 grid(c.n_path, c.dims.H, (c.dims.Dv + kRows - 1) / kRows);
    if (c.dims.dtype == GDN_BF16) hipLaunchKernelGGL(k_commit<__bf16>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_commit<float>, grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace gdn
