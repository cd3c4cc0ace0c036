// Commit by reconstruction (TreeWY, "Speculative Verification for Gated
// DeltaNet Hybrids", section 3 "Reconstruct on commit", Eq. 3):
//
//   S_a = g_a S_0 + sum over i on the root path of a (a included) of (g_a / g_i) vt_i k_i^T
//
// g_a / g_i = exp(sum of the log gates strictly after i on the path), summed
// from a backwards in fp32; g_a = exp of the whole path's sum. One workgroup
// per (path, head, 16 rows of S): it reads S_0 once, the path's pseudo-values,
// keys and gates, and writes S_a once. The kernel is bound by those two state
// streams (HBM), so it stays on plain fp32 FMAs with float4 loads and stores.
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kRows = 16;   // rows of S per workgroup
constexpr int kPathTile = 64;

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
  int H, Dk, Dv, n_seq;
};

template <typename E>
__device__ inline float upc(E x) { return (float)x; }

__global__ void k_reset(unsigned long long* err) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *err = kNoError;
}

template <typename E>
__global__ void __launch_bounds__(256) k_commit(CommitArgs a) {
  __shared__ float sK[kPathTile][128 + 4];
  __shared__ float sV[kPathTile][kRows];
  __shared__ float sW[kPathTile];
  __shared__ float sSigma;
  const int p = blockIdx.x, h = blockIdx.y, vb = blockIdx.z;
  const int tid = threadIdx.x;
  const int seq = a.path_seq[p];
  const int beg = a.path_ptr[p], end = a.path_ptr[p + 1];
  bool bad = (seq < 0 || seq >= a.n_seq || end < beg);
  if (!bad) {
    const int s0 = a.seq_start[seq], s1 = a.seq_start[seq + 1];
    for (int j = beg + tid; j < end; j += blockDim.x) {
      const int t = a.path_nodes[j];
      const int want = (j == beg) ? -1 : a.path_nodes[j - 1];
      if (t < s0 || t >= s1 || a.parent[t] != want) bad = true;
    }
  }
  if (__syncthreads_or(bad)) {
    if (tid == 0) raise_error(a.err, GDN_DEV_PATH, p);
    return;
  }
  const int Dk = a.Dk, H = a.H, Dv = a.Dv;
  const E* kg = reinterpret_cast<const E*>(a.k);
  const E* gg = reinterpret_cast<const E*>(a.g);
  // this thread's elements of the 16 x Dk block, four consecutive columns each
  const int per_row4 = Dk / 4;
  const int n4 = kRows * per_row4;  // float4 groups in the block
  constexpr int kMax4 = kRows * 128 / 4 / 256;  // at most 2 groups per thread
  float4 acc[kMax4];
  for (int i = 0; i < kMax4; ++i) acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (tid == 0) sSigma = 0.f;
  __syncthreads();
  // walk the path backwards in tiles of 64 nodes
  for (int tile_end = end; tile_end > beg; tile_end -= kPathTile) {
    const int tile_beg = max(beg, tile_end - kPathTile);
    const int nt = tile_end - tile_beg;
    for (int idx = tid; idx < nt * Dk; idx += blockDim.x) {
      const int j = idx / Dk, d = idx % Dk;
      const int t = a.path_nodes[tile_beg + j];
      sK[j][d] = upc<E>(kg[((size_t)t * H + h) * Dk + d]);
    }
    for (int idx = tid; idx < nt * kRows; idx += blockDim.x) {
      const int j = idx / kRows, r = idx % kRows;
      const int t = a.path_nodes[tile_beg + j];
      sV[j][r] = a.pv[((size_t)t * H + h) * Dv + vb * kRows + r];
    }
    if (tid == 0) {  // weights exp(sum of log gates after node j), accumulated from a backwards
      float sigma = sSigma;
      for (int j = nt - 1; j >= 0; --j) {
        sW[j] = __expf(sigma);
        sigma += upc<E>(gg[(size_t)a.path_nodes[tile_beg + j] * H + h]);
      }
      sSigma = sigma;
    }
    __syncthreads();
    for (int i = 0; i < kMax4; ++i) {
      const int gidx = tid + 256 * i;
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
  const float ga = __expf(sSigma);
  const size_t SS = (size_t)Dv * Dk;
  const float* S0 = a.init ? a.init + ((size_t)seq * H + h) * SS : nullptr;
  float* dst = a.out + ((size_t)p * H + h) * SS;
  for (int i = 0; i < kMax4; ++i) {
    const int gidx = tid + 256 * i;
    if (gidx < n4) {
      const int r = gidx / per_row4, d = (gidx % per_row4) * 4;
      const size_t off = (size_t)(vb * kRows + r) * Dk + d;
      float4 s0 = S0 ? *reinterpret_cast<const float4*>(S0 + off) : make_float4(0.f, 0.f, 0.f, 0.f);
      float4 o = acc[i];
      o.x += ga * s0.x;
      o.y += ga * s0.y;
      o.z += ga * s0.z;
      o.w += ga * s0.w;
      *reinterpret_cast<float4*>(dst + off) = o;
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
  hipLaunchKernelGGL(k_reset, dim3(1), dim3(64), 0, s, err);
  if (c.n_path > 0) {
    dim3 grid(c.n_path, c.dims.H, c.dims.Dv / kRows);
    if (c.dims.dtype == GDN_BF16) hipLaunchKernelGGL(k_commit<__bf16>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_commit<float>, grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace gdn
