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
// 8) columns of one row, in four groups of four (each 16-byte access of a row's
// eight threads covers 128 contiguous bytes). Every launch shape depends only on the
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

// Sum over the eight threads of a row (lanes 8 i .. 8 i + 7), the same value in
// each: DPP lane moves (quad permutations for xor 1 and xor 2, then the mirror
// within eight lanes), ALU operations instead of LDS permutes.
__device__ __forceinline__ float row_sum8(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));  // row_half_mirror
  return x;
}

// Lane i of each row of 16 lanes receives lane i + n's x (0 past the row's end).
__device__ __forceinline__ float from_lane_above(float x, int n) {
  const int v = __float_as_int(x);
  switch (n) {
    case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x101, 0xF, 0xF, true));  // row_shl:1
    case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x102, 0xF, 0xF, true));  // row_shl:2
    case 4: return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x104, 0xF, 0xF, true));  // row_shl:4
    default: return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x108, 0xF, 0xF, true));  // row_shl:8
  }
}

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

// 16-byte vector of E as floats.
template <typename E>
struct Vec16;
template <>
struct Vec16<float> {
  static constexpr int n = 4;
  __device__ static void load(const float* p, float* dst) {
    const float4 x = *reinterpret_cast<const float4*>(p);
    dst[0] = x.x, dst[1] = x.y, dst[2] = x.z, dst[3] = x.w;
  }
};
template <>
struct Vec16<__bf16> {
  static constexpr int n = 8;
  __device__ static void load(const __bf16* p, float* dst) {
    const uint4 x = *reinterpret_cast<const uint4*>(p);
    const unsigned w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dst[2 * i] = __uint_as_float(w[i] << 16);
      dst[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

// Path tokens [j0, j0 + nt) of the commit: history slots below hl, then tokens of
// the previous draft. Keys and pseudo-value rows are read in 16-byte pieces.
template <typename E, int DK>
__device__ inline void stage_path(const ChainArgs& a, int s, int h, int v0, int rows, int hl, int j0, int nt,
                                  float (*sK)[DK + 4], float (*sV)[kRows], float* sG) {
  constexpr int VE = Vec16<E>::n;
  const int tid = threadIdx.x, H = a.H, N = a.N, Dv = a.Dv;
  const E* pk = reinterpret_cast<const E*>(a.prev_k);
  const E* pg = reinterpret_cast<const E*>(a.prev_g);
  const E* hk = reinterpret_cast<const E*>(a.hist_k);
  for (int idx = tid; idx < nt * (DK / VE); idx += kThr) {
    const int jj = idx / (DK / VE), part = idx % (DK / VE), j = j0 + jj;
    const E* src = j < hl ? hk + (((size_t)s * a.cap + j) * H + h) * DK : pk + (((size_t)s * N + (j - hl)) * H + h) * DK;
    Vec16<E>::load(src + part * VE, &sK[jj][part * VE]);
  }
  for (int idx = tid; idx < nt * (kRows / 4); idx += kThr) {
    const int jj = idx / (kRows / 4), c4 = idx % (kRows / 4), j = j0 + jj;
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (4 * c4 < rows) {
      const float* src = j < hl ? a.hist_pv + (((size_t)s * a.cap + j) * H + h) * Dv
                                : a.prev_pv + (((size_t)s * N + (j - hl)) * H + h) * Dv;
      x = *reinterpret_cast<const float4*>(src + v0 + 4 * c4);
    }
    *reinterpret_cast<float4*>(&sV[jj][4 * c4]) = x;
  }
  if (tid < nt) {
    const int j = j0 + tid;
    sG[tid] = j < hl ? a.hist_g[((size_t)s * a.cap + j) * H + h] : upc<E>(pg[((size_t)s * N + (j - hl)) * H + h]);
  }
}

template <typename E, int DK>
__global__ void __launch_bounds__(kThr, 8) k_chain_step(const ChainArgs a) {
  constexpr int CPT = DK / 8;  // columns per thread
  constexpr int VE = Vec16<E>::n;
  __shared__ float sK[kTileP][DK + 4];
  __shared__ float sV[kTileP][kRows];
  __shared__ float sG[kTileP];
  __shared__ float sW[kTileP + 1];  // the tokens' weights, then the tile's decay
  extern __shared__ float dyn[];  // draft: k [N][DK], q [N][DK], v [N][kRows], gate [N], beta [N]
  const int s = blockIdx.x, h = blockIdx.y, vb = blockIdx.z;
  const int tid = threadIdx.x, r = tid >> 3, cq = tid & 7;
  const int H = a.H, Dv = a.Dv, N = a.N;
  const int rows = min(kRows, Dv - vb * kRows);
  const bool row_ok = r < rows;
  const int v0 = vb * kRows;
  if (s == 0 && h == 0 && vb == 0) check_all(a);
  // The accepted count and the history length are checked only after the loads
  // that do not depend on them (checkpoint rows, draft) have been issued, so
  // that their round trip overlaps those loads.
  const int acc = a.accepted[s], hl = a.hist_len_in[s];
  const size_t SS = (size_t)Dv * DK;
  E* hk = reinterpret_cast<E*>(a.hist_k);

  // every independent load first: the checkpoint rows, the draft, the path's last tile.
  // Element 4 i4 + e of a thread is column 4 cq + 32 i4 + e of its row, so that
  // the eight threads of a row read 128 contiguous bytes per instruction.
  float S[CPT];
  const float* ck = a.ckpt + ((size_t)s * H + h) * SS + (size_t)(v0 + r) * DK + 4 * cq;
#pragma unroll
  for (int i = 0; i < CPT; i += 4) {
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row_ok) x = *reinterpret_cast<const float4*>(ck + 8 * i);
    S[i] = x.x;
    S[i + 1] = x.y;
    S[i + 2] = x.z;
    S[i + 3] = x.w;
  }
  float* dK = dyn;
  float* dQ = dK + (size_t)N * DK;
  float* dV = dQ + (size_t)N * DK;
  float* dG = dV + (size_t)N * kRows;
  float* dB = dG + N;
  {
    const E* qg = reinterpret_cast<const E*>(a.q);
    const E* kg = reinterpret_cast<const E*>(a.k);
    const E* vg = reinterpret_cast<const E*>(a.v);
    const E* gg = reinterpret_cast<const E*>(a.g);
    const E* bg = reinterpret_cast<const E*>(a.b);
    for (int idx = tid; idx < 2 * N * (DK / VE); idx += kThr) {
      const int which = idx / (N * (DK / VE)), rem = idx % (N * (DK / VE));
      const int t = rem / (DK / VE), part = rem % (DK / VE);
      const size_t o = (((size_t)s * N + t) * H + h) * DK + part * VE;
      Vec16<E>::load((which ? qg : kg) + o, (which ? dQ : dK) + (size_t)t * DK + part * VE);
    }
    constexpr int VPR = kRows / VE;  // 16-byte pieces of a 32-column value row
    for (int idx = tid; idx < N * VPR; idx += kThr) {
      const int t = idx / VPR, part = idx % VPR;
      float* dst = dV + (size_t)t * kRows + part * VE;
      if (part * VE < rows) Vec16<E>::load(vg + (((size_t)s * N + t) * H + h) * Dv + v0 + part * VE, dst);
      else
        for (int i = 0; i < VE; ++i) dst[i] = 0.f;
    }
    for (int t = tid; t < N; t += kThr) {
      dG[t] = upc<E>(gg[((size_t)s * N + t) * H + h]);
      dB[t] = upc<E>(bg[((size_t)s * N + t) * H + h]);
    }
  }
  if (acc < 0 || acc > N || hl < 0 || hl > a.cap) return;  // reported by check_all
  // commit (Eq. 3) over the path: history slots [0, hl), then draft tokens [0, acc)
  const int L = hl + acc;
  const bool flush = a.flush || L > a.cap;
  // the accepted tokens join the history (unless this round flushes), copied
  // from the previous draft's pseudo-values, keys and gates
  if (!flush) {
    const E* pk = reinterpret_cast<const E*>(a.prev_k);
    const E* pg = reinterpret_cast<const E*>(a.prev_g);
    for (int idx = tid; idx < acc * (kRows / 4); idx += kThr) {
      const int i = idx / (kRows / 4), c4 = idx % (kRows / 4);
      if (4 * c4 < rows)
        *reinterpret_cast<float4*>(a.hist_pv + (((size_t)s * a.cap + hl + i) * H + h) * Dv + v0 + 4 * c4) =
            *reinterpret_cast<const float4*>(a.prev_pv + (((size_t)s * N + i) * H + h) * Dv + v0 + 4 * c4);
    }
    if (vb == 0) {
      for (int idx = tid; idx < acc * (DK / VE); idx += kThr) {
        const int i = idx / (DK / VE), part = idx % (DK / VE);
        *reinterpret_cast<uint4*>(hk + (((size_t)s * a.cap + hl + i) * H + h) * DK + part * VE) =
            *reinterpret_cast<const uint4*>(pk + (((size_t)s * N + i) * H + h) * DK + part * VE);
      }
      if (tid < acc) a.hist_g[((size_t)s * a.cap + hl + tid) * H + h] = upc<E>(pg[((size_t)s * N + tid) * H + h]);
    }
  }
  // The path is taken from its start in tiles of kTileP tokens, which regroups
  // Eq. 3 tile by tile: S <- exp(sum of the tile's log gates) S + sum over the
  // tile of exp(sum of its log gates after j) vt_j k_j^T, from the checkpoint.
  for (int j0 = 0; j0 < L; j0 += kTileP) {
    const int nt = min(kTileP, L - j0);
    stage_path<E, DK>(a, s, h, v0, rows, hl, j0, nt, sK, sV, sG);
    __syncthreads();
    static_assert(kTileP == 16, "the suffix scan runs over one row of 16 lanes");
    if (tid < 64) {  // inclusive suffix sums of the tile's log gates over lanes 0..15
      const float gv = tid < nt ? sG[tid] : 0.f;
      float x = gv;
#pragma unroll
      for (int o = 1; o < kTileP; o <<= 1) x += from_lane_above(x, o);
      if (tid < nt) sW[tid] = __expf(x - gv);
      if (tid == 0) sW[kTileP] = __expf(x);
    }
    __syncthreads();
    const float dec = sW[kTileP];
#pragma unroll
    for (int i = 0; i < CPT; ++i) S[i] *= dec;
    for (int jj = 0; jj < nt; ++jj) {
      const float wv = sW[jj] * sV[jj][r];
#pragma unroll
      for (int i = 0; i < CPT; ++i) S[i] += wv * sK[jj][4 * cq + 8 * (i & ~3) + (i & 3)];
    }
    __syncthreads();
  }

  __syncthreads();  // the draft in LDS is complete (an empty path runs no tile above)

  // flush the committed state (or keep the accepted tokens as history, above)
  float* stores[2] = {flush ? a.ckpt : nullptr, a.state_out};
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    if (!stores[w] || !row_ok) continue;
    float* dst = stores[w] + ((size_t)s * H + h) * SS + (size_t)(v0 + r) * DK + 4 * cq;
#pragma unroll
    for (int i = 0; i < CPT; i += 4)
      *reinterpret_cast<float4*>(dst + 8 * i) = make_float4(S[i], S[i + 1], S[i + 2], S[i + 3]);
  }
  if (h == 0 && vb == 0 && tid == 0) a.hist_len_out[s] = flush ? 0 : L;

  // verify the new draft from S
  E* og = reinterpret_cast<E*>(a.out);
  for (int t = 0; t < N; ++t) {
    const float* kt = dK + (size_t)t * DK + 4 * cq;
    const float* qt = dQ + (size_t)t * DK + 4 * cq;
    float u = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) u += S[i] * kt[8 * (i & ~3) + (i & 3)];
    u = row_sum8(u);
    const float al = __expf(dG[t]);
    const float vt = dB[t] * (dV[t * kRows + r] - al * u);
    float o = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = 8 * (i & ~3) + (i & 3);
      S[i] = al * S[i] + vt * kt[c];
      o += S[i] * qt[c];
    }
    o = row_sum8(o);
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
