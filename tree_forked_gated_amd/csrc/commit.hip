// Commit by reconstruction (TreeWY, "Speculative Verification for Gated
// DeltaNet Hybrids", section 3 "Reconstruct on commit", Eq. 3):
//
//   S_a = g_a S_0 + sum over i on the root path of a (a included) of (g_a / g_i) vt_i k_i^T
//
// g_a / g_i = exp(sum of the log gates strictly after i on the path), summed
// from a backwards in fp32; g_a = exp of the whole path's sum. One workgroup
// per (path, head, 32 rows of S): it reads S_0 once, the path's pseudo-values,
// keys and gates, and writes S_a once. The kernel is bound by those two state
// streams (HBM), so it stays on plain fp32 FMAs with float4 loads and stores.
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

template <typename E>
__device__ inline float upc(E x) { return (float)x; }

__global__ void k_reset(unsigned long long* err) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *err = kNoError;
}

// Is path p a parent chain from a root of its sequence down to its last node?
// Every index is checked before it is used.
__device__ inline bool path_ok(const CommitArgs& a, int p) {
  const int seq = a.path_seq[p];
  const int beg = a.path_ptr[p], end = a.path_ptr[p + 1];
  if (seq < 0 || seq >= a.n_seq || end < beg) return false;
  if (end == beg) return true;
  const int s_0 = a.seq_start[seq], s_1 = a.seq_start[seq + 1];
  if (s_0 < 0 || s_1 > a.T || s_1 <= s_0) return false;
  for (int j = beg; j < end; ++j) {
    const int t = a.path_nodes[j];
    const int want = (j == beg) ? -1 : a.path_nodes[j - 1];
    if (t < s_0 || t >= s_1 || a.parent[t] != want) return false;
  }
  return true;
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

// One workgroup per (path, head, 32 rows of S). The rows of S_0 are loaded
// first, so that they arrive while the path is summed. The path is staged in
// LDS 16 nodes at a time, from the accepted node backwards: each node is
// checked (in its sequence, parent = previous node) in the same pass that loads
// its key, pseudo-values and gate, with the index held in range until the
// check is decided, just before the stores.
template <typename E>
__global__ void __launch_bounds__(kThreads, 6) k_commit(CommitArgs a) {
  __shared__ float sK[kPathTile][128 + 4];
  __shared__ float sV[kPathTile][kRows];
  __shared__ float sG[kPathTile];
  __shared__ float sW[kPathTile];
  __shared__ float sSigma;
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
  // S_0 rows of this block (zeros without initial states)
  float4 s0[kPer4];
  const float* S0 = (!bad_path && a.init) ? a.init + ((size_t)seq * H + h) * SS : nullptr;
#pragma unroll
  for (int i = 0; i < kPer4; ++i) {
    const int gidx = tid + kThreads * i;
    const int r = gidx / per_row4, d = (gidx % per_row4) * 4;
    f32x4n v = {0.f, 0.f, 0.f, 0.f};
    if (S0 && gidx < n4 && r < rows) v = __builtin_nontemporal_load(reinterpret_cast<const f32x4n*>(S0 + (size_t)(vb * kRows + r) * Dk + d));
    s0[i] = make_float4(v[0], v[1], v[2], v[3]);
  }
  const E* kg = reinterpret_cast<const E*>(a.k);
  const E* gg = reinterpret_cast<const E*>(a.g);
  int s_0 = bad_path ? 0 : a.seq_start[seq], s_1 = bad_path ? 0 : a.seq_start[seq + 1];
  // a non-empty path needs a non-empty sequence inside [0, T); nothing is loaded otherwise
  const bool no_tokens = !bad_path && end > beg && (s_1 <= s_0 || s_0 < 0 || s_1 > a.T);
  if (no_tokens) s_0 = s_1 = 0;
  bad |= no_tokens;
  float4 acc[kPer4];
#pragma unroll
  for (int i = 0; i < kPer4; ++i) acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (tid == 0) sSigma = 0.f;
  __syncthreads();
  for (int tile_end = (bad_path || no_tokens) ? beg : end; tile_end > beg; tile_end -= kPathTile) {
    const int tile_beg = max(beg, tile_end - kPathTile);
    const int nt = tile_end - tile_beg;
    if (tid < nt) {  // check the node and load its gate
      const int j = tile_beg + tid;
      const int t = a.path_nodes[j];
      const int want = (j == beg) ? -1 : a.path_nodes[j - 1];
      const bool ok = t >= s_0 && t < s_1 && a.parent[t] == want;
      bad |= !ok;
      sG[tid] = ok ? upc<E>(gg[(size_t)t * H + h]) : 0.f;
    }
    for (int idx = tid; idx < nt * Dk; idx += kThreads) {
      const int j = idx / Dk, d = idx % Dk;
      int t = a.path_nodes[tile_beg + j];
      t = (t >= s_0 && t < s_1) ? t : s_0;  // in range until the check is decided
      sK[j][d] = upc<E>(kg[((size_t)t * H + h) * Dk + d]);
    }
    for (int idx = tid; idx < nt * kRows; idx += kThreads) {
      const int j = idx / kRows, r = idx % kRows;
      int t = a.path_nodes[tile_beg + j];
      t = (t >= s_0 && t < s_1) ? t : s_0;
      sV[j][r] = r < rows ? a.pv[((size_t)t * H + h) * Dv + vb * kRows + r] : 0.f;
    }
    __syncthreads();
    if (tid == 0) {  // weights exp(sum of log gates after node j), accumulated from a backwards
      float sigma = sSigma;
      for (int j = nt - 1; j >= 0; --j) {
        sW[j] = __expf(sigma);
        sigma += sG[j];
      }
      sSigma = sigma;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPer4; ++i) {
      const int gidx = tid + kThreads * i;
      if (gidx < n4) {
        const int r = gidx / per_row4, d = (gidx % per_row4) * 4;
        float4 s = acc[i];
        for (int j = nt - 1; j >= 0; --j) {
          const float wv = sW[j] * sV[j][r];
          s.x += wv * sK[j][d];
          s.y += wv * sK[j][d + 1];
          s.z += wv * sK[j][d + 2];
          s.w += wv * sK[j][d + 3];
        }
        acc[i] = s;
      }
    }
    __syncthreads();
  }
  if (a.own_err && p == 0 && h == 0 && vb == 0) check_all_paths(a);
  if (__syncthreads_or(bad)) {
    if (tid == 0 && !a.own_err) raise_error(a.err, GDN_DEV_PATH, p);
    return;
  }
  const float ga = __expf(sSigma);
  float* dst = a.out + ((size_t)p * H + h) * SS;
#pragma unroll
  for (int i = 0; i < kPer4; ++i) {
    const int gidx = tid + kThreads * i;
    const int r = gidx / per_row4, d = (gidx % per_row4) * 4;
    if (gidx < n4 && r < rows) {
      float4 o = acc[i];
      o.x += ga * s0[i].x;
      o.y += ga * s0[i].y;
      o.z += ga * s0[i].z;
      o.w += ga * s0[i].w;
      f32x4n ov = {o.x, o.y, o.z, o.w};
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
