// One speculative round of chain drafts in one kernel: commit the previous
// round's accepted tokens, then verify the new chain draft from that state
// (TreeWY, "Speculative Verification for Gated DeltaNet Hybrids", section 4
// "Implementation": a chain verifies and commits in one fused, graph-capturable
// kernel). The committed state is written to memory only at a flush (the
// deferred write of ReplaySSM, which TreeWY's section 1 and appendix D discuss):
// between flushes the accepted tokens' pseudo-values, keys and log gates are
// appended to a short history, and each round rebuilds its starting state from
// the checkpoint and that history with TreeWY Eq. 3:
//
//   S = g S_ckpt + sum over path tokens i of (g / g_i) vt_i k_i^T,
//
// path = history, then the previous draft's accepted prefix; g_i the product of
// alpha over the path up to i, g over all of it. The draft is then verified by
// the per-token recurrence of Eq. 1 with the key rewrite (chains are short),
// in fp32 on the state held in registers:
//
//   vt_t = beta_t (v_t - alpha_t S k_t),  S <- alpha_t S + vt_t k_t^T,  o_t = S q_t.
//
// One workgroup per (sequence, head, 32 rows of S); a thread holds 16 (d_k /
// 8) consecutive columns of one row. Every launch shape depends only on the
// sizes; the accepted counts and history lengths are device data.
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kRows = 32;   // rows of S (d_v) per workgroup
constexpr int kThr = 256;   // 8 threads per row
constexpr int kTileP = 16;  // path tokens staged in LDS at a time

struct ChainArgs {
  float* ckpt;
  float* hist_pv;
  void* hist_k;
  float* hist_g;
  const int* hist_len_in;
  int* hist_len_out;
  const float* prev_pv;
  const void* prev_k;
  const void* prev_g;
  const int* accepted;
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* b;
  void* out;
  float* pv;
  float* state_out;
  unsigned long long* err;
  int n_seq, N, H, Dv, cap, flush;
};

template <typename E>
__device__ inline float upc(E x) { return (float)x; }

// One workgroup checks every sequence's counts and stores the error word
// (smallest bad sequence) with a plain store: no reset is needed before a call.
__device__ void check_all(const ChainArgs& a) {
  __shared__ int s_bad;
  if (threadIdx.x == 0) s_bad = 0x7fffffff;
  __syncthreads();
  for (int s = threadIdx.x; s < a.n_seq; s += blockDim.x) {
    const int acc = a.accepted[s], hl = a.hist_len_in[s];
    if (acc < 0 || acc > a.N || hl < 0 || hl > a.cap) atomicMin(&s_bad, s);
  }
  __syncthreads();
  if (threadIdx.x == 0)
    *a.err = s_bad == 0x7fffffff ? kNoError
                                 : (((unsigned long long)(unsigned)GDN_DEV_CHAIN << 32) | (unsigned)s_bad);
}

template <typename E, int DK>
__global__ void __launch_bounds__(kThr) k_chain_step(const ChainArgs a) {
  constexpr int CPT = DK / 8;  // columns per thread
  __shared__ float sK[kTileP][DK + 4];
  __shared__ float sV[kTileP][kRows];
  __shared__ float sG[kTileP];
  __shared__ float sW[kTileP];
  __shared__ float sSigma;
  extern __shared__ float dyn[];  // draft: k [N][DK], q [N][DK], v [N][kRows], gate [N], beta [N]
  const int s = blockIdx.x, h = blockIdx.y, vb = blockIdx.z;
  const int tid = threadIdx.x, r = tid >> 3, cq = tid & 7;
  const int H = a.H, Dv = a.Dv, N = a.N;
  const int rows = min(kRows, Dv - vb * kRows);
  const bool row_ok = r < rows;
  const int v0 = vb * kRows;
  if (s == 0 && h == 0 && vb == 0) check_all(a);
  const int acc = a.accepted[s], hl = a.hist_len_in[s];
  if (acc < 0 || acc > N || hl < 0 || hl > a.cap) return;  // reported by check_all
  const size_t SS = (size_t)Dv * DK;
  const E* pk = reinterpret_cast<const E*>(a.prev_k);
  const E* pg = reinterpret_cast<const E*>(a.prev_g);
  E* hk = reinterpret_cast<E*>(a.hist_k);

  // the checkpoint rows
  float S[CPT];
  const float* ck = a.ckpt + ((size_t)s * H + h) * SS + (size_t)(v0 + r) * DK + cq * CPT;
#pragma unroll
  for (int i = 0; i < CPT; i += 4) {
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row_ok) x = *reinterpret_cast<const float4*>(ck + i);
    S[i] = x.x;
    S[i + 1] = x.y;
    S[i + 2] = x.z;
    S[i + 3] = x.w;
  }

  // commit (Eq. 3) over the path: history slots [0, hl), then draft tokens [0, acc)
  const int L = hl + acc;
  float accum[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) accum[i] = 0.f;
  if (tid == 0) sSigma = 0.f;
  __syncthreads();
  for (int tile_end = L; tile_end > 0; tile_end -= kTileP) {
    const int tile_beg = max(0, tile_end - kTileP);
    const int nt = tile_end - tile_beg;
    if (tid < nt) {
      const int j = tile_beg + tid;
      sG[tid] = j < hl ? a.hist_g[((size_t)s * a.cap + j) * H + h]
                       : upc<E>(pg[((size_t)s * N + (j - hl)) * H + h]);
    }
    for (int idx = tid; idx < nt * DK; idx += kThr) {
      const int jj = idx / DK, d = idx % DK, j = tile_beg + jj;
      sK[jj][d] = j < hl ? upc<E>(hk[(((size_t)s * a.cap + j) * H + h) * DK + d])
                         : upc<E>(pk[(((size_t)s * N + (j - hl)) * H + h) * DK + d]);
    }
    for (int idx = tid; idx < nt * kRows; idx += kThr) {
      const int jj = idx / kRows, rr = idx % kRows, j = tile_beg + jj;
      float x = 0.f;
      if (rr < rows)
        x = j < hl ? a.hist_pv[(((size_t)s * a.cap + j) * H + h) * Dv + v0 + rr]
                   : a.prev_pv[(((size_t)s * N + (j - hl)) * H + h) * Dv + v0 + rr];
      sV[jj][rr] = x;
    }
    __syncthreads();
    if (tid == 0) {  // exp(sum of the log gates after token j), accumulated from the path's end
      float sigma = sSigma;
      for (int jj = nt - 1; jj >= 0; --jj) {
        sW[jj] = __expf(sigma);
        sigma += sG[jj];
      }
      sSigma = sigma;
    }
    __syncthreads();
    for (int jj = nt - 1; jj >= 0; --jj) {
      const float wv = sW[jj] * sV[jj][r];
#pragma unroll
      for (int i = 0; i < CPT; ++i) accum[i] += wv * sK[jj][cq * CPT + i];
    }
    __syncthreads();
  }
  const float gall = __expf(sSigma);
#pragma unroll
  for (int i = 0; i < CPT; ++i) S[i] = gall * S[i] + accum[i];

  // flush the committed state, or keep the accepted tokens as history
  const bool flush = a.flush || L > a.cap;
  float* stores[2] = {flush ? a.ckpt : nullptr, a.state_out};
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    if (!stores[w] || !row_ok) continue;
    float* dst = stores[w] + ((size_t)s * H + h) * SS + (size_t)(v0 + r) * DK + cq * CPT;
#pragma unroll
    for (int i = 0; i < CPT; i += 4) *reinterpret_cast<float4*>(dst + i) = make_float4(S[i], S[i + 1], S[i + 2], S[i + 3]);
  }
  if (!flush) {
    for (int idx = tid; idx < acc * kRows; idx += kThr) {
      const int i = idx / kRows, rr = idx % kRows;
      if (rr < rows)
        a.hist_pv[(((size_t)s * a.cap + hl + i) * H + h) * Dv + v0 + rr] =
            a.prev_pv[(((size_t)s * N + i) * H + h) * Dv + v0 + rr];
    }
    if (vb == 0) {
      for (int idx = tid; idx < acc * DK; idx += kThr) {
        const int i = idx / DK, d = idx % DK;
        hk[(((size_t)s * a.cap + hl + i) * H + h) * DK + d] = pk[(((size_t)s * N + i) * H + h) * DK + d];
      }
      if (tid < acc) a.hist_g[((size_t)s * a.cap + hl + tid) * H + h] = upc<E>(pg[((size_t)s * N + tid) * H + h]);
    }
  }
  if (h == 0 && vb == 0 && tid == 0) a.hist_len_out[s] = flush ? 0 : L;

  // verify the new draft from S
  float* dK = dyn;
  float* dQ = dK + (size_t)N * DK;
  float* dV = dQ + (size_t)N * DK;
  float* dG = dV + (size_t)N * kRows;
  float* dB = dG + N;
  const E* qg = reinterpret_cast<const E*>(a.q);
  const E* kg = reinterpret_cast<const E*>(a.k);
  const E* vg = reinterpret_cast<const E*>(a.v);
  const E* gg = reinterpret_cast<const E*>(a.g);
  const E* bg = reinterpret_cast<const E*>(a.b);
  for (int idx = tid; idx < N * DK; idx += kThr) {
    const int t = idx / DK, d = idx % DK;
    const size_t o = (((size_t)s * N + t) * H + h) * DK + d;
    dK[idx] = upc<E>(kg[o]);
    dQ[idx] = upc<E>(qg[o]);
  }
  for (int idx = tid; idx < N * kRows; idx += kThr) {
    const int t = idx / kRows, rr = idx % kRows;
    dV[idx] = rr < rows ? upc<E>(vg[(((size_t)s * N + t) * H + h) * Dv + v0 + rr]) : 0.f;
  }
  for (int t = tid; t < N; t += kThr) {
    dG[t] = upc<E>(gg[((size_t)s * N + t) * H + h]);
    dB[t] = upc<E>(bg[((size_t)s * N + t) * H + h]);
  }
  __syncthreads();
  E* og = reinterpret_cast<E*>(a.out);
  for (int t = 0; t < N; ++t) {
    const float* kt = dK + (size_t)t * DK + cq * CPT;
    const float* qt = dQ + (size_t)t * DK + cq * CPT;
    float u = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) u += S[i] * kt[i];
    u += __shfl_xor(u, 1);
    u += __shfl_xor(u, 2);
    u += __shfl_xor(u, 4);
    const float al = __expf(dG[t]);
    const float vt = dB[t] * (dV[t * kRows + r] - al * u);
    float o = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      S[i] = al * S[i] + vt * kt[i];
      o += S[i] * qt[i];
    }
    o += __shfl_xor(o, 1);
    o += __shfl_xor(o, 2);
    o += __shfl_xor(o, 4);
    if (cq == 0 && row_ok) {
      const size_t ro = (((size_t)s * N + t) * H + h) * Dv + v0 + r;
      og[ro] = (E)o;
      a.pv[ro] = vt;
    }
  }
}

}  // namespace

int chain_dyn_lds(int N, int dk) { return (int)sizeof(float) * (2 * N * dk + N * kRows + 2 * N); }

hipError_t launch_chain(const gdn_chain_args& c, hipStream_t s) {
  ChainArgs a;
  a.ckpt = c.ckpt;
  a.hist_pv = c.hist_pv;
  a.hist_k = c.hist_k;
  a.hist_g = c.hist_g;
  a.hist_len_in = c.hist_len_in;
  a.hist_len_out = c.hist_len_out;
  a.prev_pv = c.prev_pv;
  a.prev_k = c.prev_k;
  a.prev_g = c.prev_g;
  a.accepted = c.accepted;
  a.q = c.q;
  a.k = c.k;
  a.v = c.v;
  a.g = c.log_gate;
  a.b = c.beta;
  a.out = c.out;
  a.pv = c.pseudo_v;
  a.state_out = c.state_out;
  a.err = (unsigned long long*)c.workspace;
  a.n_seq = c.dims.n_seq;
  a.N = c.dims.N;
  a.H = c.dims.H;
  a.Dv = c.dims.Dv;
  a.cap = c.dims.hist_cap;
  a.flush = (c.flags & GDN_CHAIN_FLUSH) ? 1 : 0;
  if (c.dims.n_seq == 0) return hipSuccess;
  const dim3 grid(c.dims.n_seq, c.dims.H, (c.dims.Dv + kRows - 1) / kRows);
  const int dyn = chain_dyn_lds(c.dims.N, c.dims.Dk);
  const bool bf = c.dims.dtype == GDN_BF16;
  switch (c.dims.Dk) {
#define CASE(DKV)                                                                                        \
  case DKV:                                                                                              \
    if (bf) hipLaunchKernelGGL((k_chain_step<__bf16, DKV>), grid, dim3(kThr), dyn, s, a);               \
    else hipLaunchKernelGGL((k_chain_step<float, DKV>), grid, dim3(kThr), dyn, s, a);                  \
    break;
    CASE(32)
    CASE(64)
    CASE(128)
#undef CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gdn
