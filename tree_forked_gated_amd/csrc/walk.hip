// Chunked tree-WY walk of the gated delta rule on gfx950.
//
// Math (TreeWY, "Speculative Verification for Gated DeltaNet Hybrids",
// section 3: "Key rewrite", Eq. 2 "Verifying a draft", Eq. 3 "Reconstruct on
// commit"), applied to one chunk of n <= 64 tokens whose in-chunk parents
// precede them and whose out-of-chunk entries all start from one state S_e:
//
//   G_i        chunk-local path sum of log gates (G_i = G_{p(i)} + g_i, 0 at the entry)
//   M[i][j]    1 iff j is an ancestor of i or i itself (a causal mask on a chain)
//   A[i][j]    beta_i exp(G_i - G_j) (k_i . k_j) for j a strict ancestor of i, else 0
//   T          (I + A)^{-1}          (unit lower triangular; parents come first)
//   W          T diag(beta e^G) K    U = T diag(beta) V
//   Vt         U - W S_e^T           (the pseudo-values, one per token)
//   O          diag(e^G) Q S_e^T + (M . exp(G_i - G_j) . Q K^T) Vt
//   S_a        e^{G_a} S_e + sum over j ancestor-or-self of a of exp(G_a - G_j) vt_j k_j^T
//
// With S_e the committed state and the whole draft tree in one chunk this is
// TreeWY's Eq. 2 and Eq. 3 verbatim; with a causal mask it is the chain WY
// form those equations generalise. Forks (Flide, "Accelerating Decision
// Inference with Exact State Forking", sections 3.2.2 and 3.5): a segment that
// starts at a fork reads its entry state from the fork token's slot, which the
// chunk holding that token wrote once with the S_a formula; no state is ever
// copied per branch.
//
// One workgroup (four wave64s) walks one (segment, head, Dv tile) item chunk
// by chunk, holding S in registers (fp32) and its bf16 or fp32 image in LDS.
// Items of one dependency level are taken from an atomic counter by a
// persistent grid. All products use MFMA 16x16 tiles: v_mfma_f32_16x16x32_bf16
// for bf16 inputs, v_mfma_f32_16x16x4_f32 for fp32 inputs and for the
// triangular solve. The reduction order of every output element depends only
// on its chunk, never on the Dv tile or on other items, so results are bitwise
// independent of the batch around a sequence.
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename E>
struct Op;

template <>
struct Op<__bf16> {
  static constexpr int KS = 32;  // k extent of one MFMA
  // acc += A[0:16, 0:32] * B[0:16, 0:32]^T with A, B in LDS, rows k-contiguous
  __device__ static inline void mma(f32x4& acc, const __bf16* A, int lda, const __bf16* B, int ldb, int lane) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(A + (lane & 15) * lda + 8 * (lane >> 4));
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(B + (lane & 15) * ldb + 8 * (lane >> 4));
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
  }
  __device__ static inline __bf16 cvt(float x) { return (__bf16)x; }
  __device__ static inline float up(__bf16 x) { return (float)x; }
  __device__ static inline void st4(__bf16* p, f32x4 v) {
    bf16x4 o;
    o[0] = (__bf16)v[0];
    o[1] = (__bf16)v[1];
    o[2] = (__bf16)v[2];
    o[3] = (__bf16)v[3];
    *reinterpret_cast<bf16x4*>(p) = o;
  }
};

template <>
struct Op<float> {
  static constexpr int KS = 4;
  __device__ static inline void mma(f32x4& acc, const float* A, int lda, const float* B, int ldb, int lane) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[(lane & 15) * lda + (lane >> 4)], B[(lane & 15) * ldb + (lane >> 4)],
                                               acc, 0, 0, 0);
  }
  __device__ static inline float cvt(float x) { return x; }
  __device__ static inline float up(float x) { return x; }
  __device__ static inline void st4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
};

template <typename E, int KLEN>
__device__ inline void contract(f32x4& acc, const E* A, int lda, const E* B, int ldb, int lane) {
#pragma unroll
  for (int k0 = 0; k0 < KLEN; k0 += Op<E>::KS) Op<E>::mma(acc, A + k0, lda, B + k0, ldb, lane);
}

template <typename E>
__device__ inline void contract_n(f32x4& acc, const E* A, int lda, const E* B, int ldb, int klen, int lane) {
  for (int k0 = 0; k0 < klen; k0 += Op<E>::KS) Op<E>::mma(acc, A + k0, lda, B + k0, ldb, lane);
}

template <typename E>
__device__ inline int round_k(int x) {
  return (x + Op<E>::KS - 1) / Op<E>::KS * Op<E>::KS;
}

// LDS carve-up (bytes). Regions that are never live at the same time share
// memory: Q then the negated W; A and T (fp32) then the two transposed
// pseudo-value images.
template <typename E, int DK, int BV>
struct Cfg {
  static constexpr int ES = sizeof(E);
  static constexpr int PAD = 16 / ES;
  static constexpr int LDK = DK + PAD;      // [*][DK] tiles
  static constexpr int LDM = kChunk + PAD;  // [*][64] tiles
  static constexpr int LDF = kChunk + 4;    // fp32 [64][64] tiles
  static constexpr int LDY = 17;
  static constexpr int KB = DK / 16, VB = BV / 16;
  static constexpr int oKr = 0;
  static constexpr int oKt = oKr + kChunk * LDK * ES;
  static constexpr int oQW = oKt + DK * LDM * ES;
  static constexpr int oVt = oQW + kChunk * LDK * ES;
  static constexpr int oSb = oVt + BV * LDM * ES;
  static constexpr int oPb = oSb + BV * LDK * ES;
  static constexpr int oAT = oPb + kChunk * LDM * ES;
  static constexpr int szAT = 2 * kChunk * LDF * 4;
  static constexpr int oTT = oAT + szAT;
  static constexpr int oY = oTT + 2 * kChunk * LDM * ES;
  static constexpr int oG = oY + 3 * 16 * LDY * 4;
  static constexpr int oEG = oG + kChunk * 4;
  static constexpr int oB = oEG + kChunk * 4;
  static constexpr int oMask = oB + kChunk * 4;
  static constexpr int oOrow = oMask + kChunk * 8;
  static constexpr int oReq = oOrow + kChunk * 4;
  static constexpr int bytes = oReq + 16;
  static_assert(2 * BV * LDM * ES <= szAT, "pseudo-value images must fit the solve region");
  static_assert(bytes <= 160 * 1024, "LDS budget");
  static_assert(DK % 16 == 0 && BV % 16 == 0, "16-wide tiles");
  static_assert((kChunk * (DK / (16 / ES))) % kThreads == 0, "row loads tile the workgroup");
};

struct WalkArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* b;
  const int* parent;
  const float* init;
  void* out;
  float* state_out;
  float* pv;
  Meta m;
  int H, Dv, NT, level, out_all;
};

__constant__ int kPairRb[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ int kPairCb[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

template <typename E, int DK, int BV>
__global__ void __launch_bounds__(kThreads, 1) k_walk(WalkArgs a) {
  using C = Cfg<E, DK, BV>;
  using O = Op<E>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  E* sKr = reinterpret_cast<E*>(smem + C::oKr);
  E* sKt = reinterpret_cast<E*>(smem + C::oKt);
  E* sQW = reinterpret_cast<E*>(smem + C::oQW);
  E* sVt = reinterpret_cast<E*>(smem + C::oVt);
  E* sSb = reinterpret_cast<E*>(smem + C::oSb);
  E* sPb = reinterpret_cast<E*>(smem + C::oPb);
  float* sAf = reinterpret_cast<float*>(smem + C::oAT);
  float* sTf = sAf + kChunk * C::LDF;
  E* sVnt = reinterpret_cast<E*>(smem + C::oAT);
  E* sVwt = sVnt + BV * C::LDM;
  E* sTw = reinterpret_cast<E*>(smem + C::oTT);
  E* sTu = sTw + kChunk * C::LDM;
  float* sY = reinterpret_cast<float*>(smem + C::oY);
  float* sG = reinterpret_cast<float*>(smem + C::oG);
  float* sEG = reinterpret_cast<float*>(smem + C::oEG);
  float* sB = reinterpret_cast<float*>(smem + C::oB);
  unsigned long long* sMask = reinterpret_cast<unsigned long long*>(smem + C::oMask);
  int* sOrow = reinterpret_cast<int*>(smem + C::oOrow);
  unsigned long long* sReq = reinterpret_cast<unsigned long long*>(smem + C::oReq);
  int* sItem = reinterpret_cast<int*>(smem + C::oReq + 8);

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const Meta& m = a.m;
  if (*m.err != kNoError) return;  // structural error: nothing is computed
  const int lvl = a.level;
  const int count = m.level_count[lvl];
  const int base = m.level_ptr[lvl];
  const int per_seg = a.H * a.NT;
  const long long total = (long long)count * per_seg;
  const size_t SS = (size_t)a.Dv * DK;
  const E* qg = reinterpret_cast<const E*>(a.q);
  const E* kg = reinterpret_cast<const E*>(a.k);
  const E* vg = reinterpret_cast<const E*>(a.v);
  const E* gg = reinterpret_cast<const E*>(a.g);
  const E* bg = reinterpret_cast<const E*>(a.b);
  E* og = reinterpret_cast<E*>(a.out);

  constexpr int ST = C::VB * C::KB;  // state tiles of one item
  constexpr int NSW = (ST + 3) / 4;  // state tiles per wave
  constexpr int NOW = C::VB;         // output / pseudo-value tiles per wave (row block = wave)
  constexpr int VEC = 16 / sizeof(E);

  for (;;) {
    __syncthreads();
    if (tid == 0) *sItem = atomicAdd(&m.walk_ctr[lvl * kSchedInts], 1);
    __syncthreads();
    const long long item = *sItem;
    if (item >= total) break;
    const int seg = m.level_items[base + (int)(item / per_seg)];
    const int rem = (int)(item % per_seg);
    const int h = rem / a.NT, tile = rem % a.NT;
    const int v0 = tile * BV;
    const int start = m.seg_start[seg], len = m.seg_len[seg], sq = m.seg_seq[seg];
    const int mode = m.seg_mode[seg], slot = m.seg_slot[seg];
    const float* Sin = slot >= 0 ? m.fork_states + ((size_t)slot * a.H + h) * SS
                                 : (a.init ? a.init + ((size_t)sq * a.H + h) * SS : nullptr);

    // entry state: fp32 registers (accumulator layout) and its operand image in LDS
    f32x4 S[NSW];
#pragma unroll
    for (int i = 0; i < NSW; ++i) {
      const int t = w + 4 * i;
      if (t < ST) {
        const int vb = t / C::KB, db = t % C::KB;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = vb * 16 + 4 * (lane >> 4) + r, col = db * 16 + (lane & 15);
          const float x = Sin ? Sin[(size_t)(v0 + row) * DK + col] : 0.f;
          S[i][r] = x;
          sSb[row * C::LDK + col] = O::cvt(x);
        }
      }
    }

    const int nch = mode ? 1 : (len + kChunk - 1) / kChunk;
    for (int c = 0; c < nch; ++c) {
      const int t0 = start + c * kChunk;
      const int n = min(kChunk, len - c * kChunk);
      const bool need_exit = (!mode) && (c + 1 < nch);

      // ---------------------------------------------------------------- load
      {
        constexpr int PR = DK / VEC;
        for (int p = tid; p < kChunk * PR; p += kThreads) {
          const int row = p / PR, col = (p % PR) * VEC;
          uint4 kv = make_uint4(0, 0, 0, 0), qv = make_uint4(0, 0, 0, 0);
          if (row < n) {
            const size_t off = ((size_t)(t0 + row) * a.H + h) * DK + col;
            kv = *reinterpret_cast<const uint4*>(kg + off);
            qv = *reinterpret_cast<const uint4*>(qg + off);
          }
          *reinterpret_cast<uint4*>(sKr + row * C::LDK + col) = kv;
          *reinterpret_cast<uint4*>(sQW + row * C::LDK + col) = qv;
          const E* ke = reinterpret_cast<const E*>(&kv);
#pragma unroll
          for (int j = 0; j < VEC; ++j) sKt[(col + j) * C::LDM + row] = ke[j];
        }
        constexpr int PV = BV / VEC;
        for (int p = tid; p < kChunk * PV; p += kThreads) {
          const int row = p / PV, col = (p % PV) * VEC;
          uint4 vv = make_uint4(0, 0, 0, 0);
          if (row < n) vv = *reinterpret_cast<const uint4*>(vg + ((size_t)(t0 + row) * a.H + h) * a.Dv + v0 + col);
          const E* ve = reinterpret_cast<const E*>(&vv);
#pragma unroll
          for (int j = 0; j < VEC; ++j) sVt[(col + j) * C::LDM + row] = ve[j];
        }
        if (tid < kChunk) {
          const int i = tid, t = t0 + i;
          const bool valid = i < n;
          float bi = 0.f, gi = 0.f;
          int ptr;
          unsigned long long mask;
          if (valid) {
            bi = O::up(bg[(size_t)t * a.H + h]);
            gi = O::up(gg[(size_t)t * a.H + h]);
          }
          if (mode) {
            const int pg = valid ? a.parent[t] : -1;
            ptr = (pg >= t0 && pg < t) ? pg - t0 : -1;
            mask = m.tree_mask[(size_t)sq * kChunk + i];
          } else {
            ptr = i - 1;
            mask = (i == kChunk - 1) ? ~0ull : ((2ull << i) - 1ull);
          }
          // chunk-local path sums of log gates by pointer jumping
          float G = gi;
          int pj = ptr;
#pragma unroll
          for (int r = 0; r < 6; ++r) {
            const int src = pj >= 0 ? pj : i;
            const float pG = __shfl(G, src);
            const int pp = __shfl(pj, src);
            if (pj >= 0) {
              G += pG;
              pj = pp;
            }
          }
          sG[i] = G;
          sEG[i] = __expf(G);
          sB[i] = bi;
          sMask[i] = mask;
          int orow = -1;
          bool req = false;
          if (valid) {
            if (a.out_all) orow = t;
            else {
              const int om = m.out_map[t];
              orow = om != kUnmapped ? om : -1;
            }
            req = (m.fork_slot[t] >= 0) || (m.state_map[t] != kUnmapped);
          }
          sOrow[i] = orow;
          const unsigned long long rq = __ballot(req);
          if (i == 0) *sReq = rq;
        }
      }
      __syncthreads();

      // -------------------------------------- phase 1: P, A and the Q S_e^T part of O
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int job = w + 4 * i;
        const int kind = job & 1;  // 0: P from Q K^T, 1: A from K K^T
        const int pair = job >> 1;
        const int rb = kPairRb[pair], cb = kPairCb[pair];
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        contract<E, DK>(acc, (kind ? sKr : sQW) + rb * 16 * C::LDK, C::LDK, sKr + cb * 16 * C::LDK, C::LDK, lane);
        const int j = cb * 16 + (lane & 15);
        const float Gj = sG[j];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ii = rb * 16 + 4 * (lane >> 4) + r;
          const bool anc = (sMask[ii] >> j) & 1ull;
          if (kind == 0) {
            const float val = anc ? __expf(sG[ii] - Gj) * acc[r] : 0.f;
            sPb[ii * C::LDM + j] = O::cvt(val);
          } else {
            const float val = (anc && ii != j) ? sB[ii] * __expf(sG[ii] - Gj) * acc[r] : 0.f;
            sAf[ii * C::LDF + j] = val;
          }
        }
      }
      for (int idx = tid; idx < kChunk * kChunk; idx += kThreads) {
        const int ii = idx >> 6, j = idx & 63;
        if ((j >> 4) > (ii >> 4)) sPb[ii * C::LDM + j] = O::cvt(0.f);
      }
      f32x4 accO[NOW];
#pragma unroll
      for (int i = 0; i < NOW; ++i) {
        accO[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        contract<E, DK>(accO[i], sQW + w * 16 * C::LDK, C::LDK, sSb + i * 16 * C::LDK, C::LDK, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) accO[i][r] *= sEG[w * 16 + 4 * (lane >> 4) + r];
      }
      __syncthreads();

      // ------------------------------------ phase 2: T = (I + A)^{-1}, blocked, fp32
      if (lane < 16) {  // diagonal block w: forward substitution, one column per lane
        const int b = w;
        float x[16];
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) {
          float acc = (ii == lane) ? 1.f : 0.f;
#pragma unroll
          for (int mm = 0; mm < ii; ++mm) acc -= sAf[(16 * b + ii) * C::LDF + 16 * b + mm] * x[mm];
          x[ii] = acc;
        }
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) sTf[(16 * b + ii) * C::LDF + 16 * b + lane] = x[ii];
      }
      __syncthreads();
      for (int gap = 1; gap < 4; ++gap) {  // T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj, i - j = gap
        const bool act = w < 4 - gap;
        const int bi = w + gap, bj = w;
        float* Yw = sY + w * 16 * C::LDY;
        if (act) {
          f32x4 y = {0.f, 0.f, 0.f, 0.f};
          for (int k0 = 16 * bj; k0 < 16 * bi; k0 += 4)
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(sAf[(16 * bi + (lane & 15)) * C::LDF + k0 + (lane >> 4)],
                                                     sTf[(k0 + (lane >> 4)) * C::LDF + 16 * bj + (lane & 15)], y, 0, 0,
                                                     0);
#pragma unroll
          for (int r = 0; r < 4; ++r) Yw[(4 * (lane >> 4) + r) * C::LDY + (lane & 15)] = y[r];
        }
        __syncthreads();
        if (act) {
          f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k0 = 0; k0 < 16; k0 += 4)
            z = __builtin_amdgcn_mfma_f32_16x16x4f32(sTf[(16 * bi + (lane & 15)) * C::LDF + 16 * bi + k0 + (lane >> 4)],
                                                     Yw[(k0 + (lane >> 4)) * C::LDY + (lane & 15)], z, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) sTf[(16 * bi + 4 * (lane >> 4) + r) * C::LDF + 16 * bj + (lane & 15)] = -z[r];
        }
        __syncthreads();
      }
      for (int idx = tid; idx < kChunk * kChunk; idx += kThreads) {
        const int ii = idx >> 6, j = idx & 63;
        const float t = ((j >> 4) <= (ii >> 4)) ? sTf[ii * C::LDF + j] : 0.f;
        sTw[ii * C::LDM + j] = O::cvt(t * sB[j] * sEG[j]);
        sTu[ii * C::LDM + j] = O::cvt(t * sB[j]);
      }
      __syncthreads();

      // ------------------------------------------- phase 3: W = T diag(beta e^G) K (negated)
#pragma unroll
      for (int i = 0; i < C::KB; ++i) {
        const int rb = (w + i) & 3, db = i;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        contract_n<E>(acc, sTw + rb * 16 * C::LDM, C::LDM, sKt + db * 16 * C::LDM, C::LDM, round_k<E>(16 * (rb + 1)),
                      lane);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sQW[(rb * 16 + 4 * (lane >> 4) + r) * C::LDK + db * 16 + (lane & 15)] = O::cvt(-acc[r]);
      }
      __syncthreads();

      // ------------------------------------------- phase 4: pseudo-values Vt = U - W S_e^T
      f32x4 accV[NOW];
#pragma unroll
      for (int i = 0; i < NOW; ++i) {
        const int rb = w, vb = i;
        accV[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        contract_n<E>(accV[i], sTu + rb * 16 * C::LDM, C::LDM, sVt + vb * 16 * C::LDM, C::LDM,
                      round_k<E>(16 * (rb + 1)), lane);
        contract<E, DK>(accV[i], sQW + rb * 16 * C::LDK, C::LDK, sSb + vb * 16 * C::LDK, C::LDK, lane);
        if (a.pv) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = rb * 16 + 4 * (lane >> 4) + r;
            if (row < n) a.pv[((size_t)(t0 + row) * a.H + h) * a.Dv + v0 + vb * 16 + (lane & 15)] = accV[i][r];
          }
        }
        O::st4(sVnt + (vb * 16 + (lane & 15)) * C::LDM + rb * 16 + 4 * (lane >> 4), accV[i]);
      }
      __syncthreads();

      // ------------------------------------------- phase 5: O += P Vt, write the rows asked for
#pragma unroll
      for (int i = 0; i < NOW; ++i) {
        const int rb = w, vb = i;
        contract_n<E>(accO[i], sPb + rb * 16 * C::LDM, C::LDM, sVnt + vb * 16 * C::LDM, C::LDM,
                      round_k<E>(16 * (rb + 1)), lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int orow = sOrow[rb * 16 + 4 * (lane >> 4) + r];
          if (orow >= 0) og[((size_t)orow * a.H + h) * a.Dv + v0 + vb * 16 + (lane & 15)] = O::cvt(accO[i][r]);
        }
      }

      // ------------------------------- phase 6: states at fork / requested tokens, chunk exit
      unsigned long long todo = *sReq;
      if (need_exit) todo |= 1ull << (n - 1);
      while (todo) {
        const int p = __builtin_ctzll(todo);
        todo &= todo - 1ull;
        const unsigned long long mk = sMask[p];
        const float Gp = sG[p];
#pragma unroll
        for (int i = 0; i < NOW; ++i) {
          const int rb = w, vb = i;
          f32x4 wv;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int mrow = rb * 16 + 4 * (lane >> 4) + r;
            wv[r] = ((mk >> mrow) & 1ull) ? accV[i][r] * __expf(Gp - sG[mrow]) : 0.f;
          }
          O::st4(sVwt + (vb * 16 + (lane & 15)) * C::LDM + rb * 16 + 4 * (lane >> 4), wv);
        }
        __syncthreads();
        const float cS = sEG[p];
        const bool is_exit = need_exit && p == n - 1;
        const int ml = round_k<E>(p + 1);
        const int tp = t0 + p;
        float* dst_slot = nullptr;
        float* dst_row = nullptr;
        if ((*sReq >> p) & 1ull) {
          const int fs = m.fork_slot[tp];
          const int sr = m.state_map[tp];
          if (fs >= 0) dst_slot = m.fork_states + ((size_t)fs * a.H + h) * SS;
          if (sr != kUnmapped) dst_row = a.state_out + ((size_t)sr * a.H + h) * SS;
        }
#pragma unroll
        for (int i = 0; i < NSW; ++i) {
          const int t = w + 4 * i;
          if (t < ST) {
            const int vb = t / C::KB, db = t % C::KB;
            f32x4 acc;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = cS * S[i][r];
            contract_n<E>(acc, sVwt + vb * 16 * C::LDM, C::LDM, sKt + db * 16 * C::LDM, C::LDM, ml, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = vb * 16 + 4 * (lane >> 4) + r, col = db * 16 + (lane & 15);
              const size_t off = (size_t)(v0 + row) * DK + col;
              if (dst_slot) dst_slot[off] = acc[r];
              if (dst_row) dst_row[off] = acc[r];
              if (is_exit) sSb[row * C::LDK + col] = O::cvt(acc[r]);
            }
            if (is_exit) S[i] = acc;
          }
        }
        __syncthreads();
      }
    }
  }
}

template <typename E, int DK, int BV>
hipError_t run(const WalkArgs& wa, int levels, hipStream_t s) {
  auto kern = k_walk<E, DK, BV>;
  constexpr int bytes = Cfg<E, DK, BV>::bytes;
  int cus = 0, occ = 1;
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), bytes, kThreads, &occ);
  if (e != hipSuccess) return e;
  e = current_device_cus(&cus);
  if (e != hipSuccess) return e;
  const int grid = cus * occ;
  for (int l = 0; l < levels; ++l) {
    WalkArgs x = wa;
    x.level = l;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), bytes, s, x);
  }
  return hipGetLastError();
}

}  // namespace

// bf16 with d_k = 128 always runs the pipelined walk (walk_pipe.hip)
#define GDN_WALK_CASES(X)                                                                                        \
  X(GDN_BF16, __bf16, 32, 16) X(GDN_BF16, __bf16, 32, 32) X(GDN_BF16, __bf16, 32, 64) X(GDN_BF16, __bf16, 64, 16) \
  X(GDN_BF16, __bf16, 64, 32) X(GDN_BF16, __bf16, 64, 64) X(GDN_F32, float, 16, 16) X(GDN_F32, float, 16, 32)     \
  X(GDN_F32, float, 32, 16) X(GDN_F32, float, 32, 32) X(GDN_F32, float, 64, 16) X(GDN_F32, float, 64, 32)

bool walk_supported(int dtype, int dk, int bv) {
  if (walk_pipe_supported(dtype, dk, bv)) return true;
#define X(DT, E, DKV, BVV) \
  if (dtype == DT && dk == DKV && bv == BVV) return true;
  GDN_WALK_CASES(X)
#undef X
  return false;
}

int walk_lds_bytes(int dtype, int dk, int bv) {
#define X(DT, E, DKV, BVV) \
  if (dtype == DT && dk == DKV && bv == BVV) return Cfg<E, DKV, BVV>::bytes;
  GDN_WALK_CASES(X)
#undef X
  return -1;
}

hipError_t launch_walk(const gdn_tree_fwd_args& fa, const Meta& m, int bv, hipStream_t s) {
  if (walk_pipe_supported(fa.dims.dtype, fa.dims.Dk, bv)) return launch_walk_pipe(fa, m, bv, s);
  WalkArgs wa;
  wa.q = fa.q;
  wa.k = fa.k;
  wa.v = fa.v;
  wa.g = fa.log_gate;
  wa.b = fa.beta;
  wa.parent = fa.parent_idx;
  wa.init = fa.init_state;
  wa.out = fa.out;
  wa.state_out = fa.state_out;
  wa.pv = fa.pseudo_v;
  wa.m = m;
  wa.H = fa.dims.H;
  wa.Dv = fa.dims.Dv;
  wa.NT = fa.dims.Dv / bv;
  wa.level = 0;
  wa.out_all = fa.out_rows == nullptr;
  const int dt = fa.dims.dtype, dk = fa.dims.Dk, L = fa.dims.max_levels;
#define X(DT, E, DKV, BVV) \
  if (dt == DT && dk == DKV && bv == BVV) return run<E, DKV, BVV>(wa, L, s);
  GDN_WALK_CASES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace gdn
