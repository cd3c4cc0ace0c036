// Chunked tree-WY walk for bf16 inputs with d_k = 128 on gfx950 (MFMA path).
//
// Per chunk of n <= 64 tokens with entry state S_e (d_v x d_k), chunk-local
// path sums of log gates G and ancestor-or-self mask M (TreeWY, "Speculative
// Verification for Gated DeltaNet Hybrids", section 3: "Key rewrite", Eq. 2
// "Verifying a draft" and Eq. 3 "Reconstruct on commit"):
//
//   A[i][j] = beta_i exp(G_i - G_j) (k_i . k_j)   j a strict ancestor of i
//   R       = diag(beta) (V - diag(e^G) K S_e^T)   right-hand side of Eq. 2
//   (I + A) Vt = R                                  pseudo-values, one per token
//   O       = diag(e^G) Q S_e^T + (M . exp(G_i - G_j) . Q K^T) Vt
//   S_a     = e^{G_a} S_e + sum over j ancestor-or-self of a of exp(G_a - G_j) vt_j k_j^T
//
// Eq. 2 is solved by blocks of 16 tokens: the four 16 x 16 diagonal blocks of
// I + A are inverted by forward substitution in fp32, and the pseudo-values of
// block b follow from those of the blocks before it,
//   Vt_b = (I + A_bb)^{-1} (R_b - sum over m < b of A_bm Vt_m).
//
// One workgroup walks one (segment, head, d_v tile) item chunk by chunk. Each
// of its waves owns 16 columns of the d_v tile and holds those 16 rows of S in
// fp32 registers. A wave keeps the chunk's K (and Q, when the chunk has rows to
// output) as MFMA fragments in registers and computes from them its share of
// the A and P = M . exp . Q K^T tiles, K S_e^T and Q S_e^T for its columns,
// the block substitution, the outputs and the state update. The last wave
// takes the four diagonal tiles and inverts their blocks, one block per
// quarter of its lanes. Products that contract over tokens take their operands
// straight from accumulators: a 16 x 16 accumulator block is the B operand
// (and, read as its transpose, the A operand) of a 16x16x16 MFMA, and two of
// them side by side form the operand of a 16x16x32 MFMA whose k index runs
// over the two blocks' rows in the same order on both sides.
//
// The next chunk's q, k, v are copied from HBM into the second of two LDS
// buffers by direct-to-LDS loads issued at the start of a chunk, so they are
// in flight while the current chunk computes; no register holds them. K and Q
// rows are stored unpadded with their 16-byte pieces permuted by an XOR of the
// row index, which keeps both the row-fragment reads and the transposed reads
// (ds_read_b64_tr_b16) free of bank conflicts. Wave 0 also prepares each
// chunk's token tables (gate sums, masks, output and state rows) and takes
// items in a fixed per-XCD order, one unit record ahead. Barriers wait on LDS
// only. Chunks that have no row to output skip Q and P entirely (selective
// readout, Flide "Accelerating Decision Inference with Exact State Forking",
// section 3.3.3).
//
// Reduction orders depend only on the chunk's own tokens (never on the d_v
// tile width, the grid or other items), so results are bitwise independent of
// the batch around a sequence and of the d_v tile.
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int DK = 128;
constexpr int kXcd = kWalkQueues;  // workgroup b runs on XCD b % 8 of an MI355X
constexpr float kLog2e = 1.4426950408889634f;

template <int BV>
struct Lay {
  static constexpr int NS = BV / 16;  // waves, one per 16 columns
  static constexpr int NTHR = NS * 64;
  static constexpr int WI = NS - 1;   // the wave that takes the diagonal tiles
  static constexpr int LDA = 64 + 4;  // fp32 row stride of A
  static constexpr int LDP = 64 + 8;  // bf16 row stride of P
  static constexpr int LDD = 16 + 4;  // bf16 row stride of the diagonal inverses
  static constexpr int LDI = BV + 8;  // bf16 row stride of the state image [d][v]
  static constexpr int VPR = BV / 8;  // 16-byte pieces per V row
  static constexpr int RPI = 64 / VPR;  // V rows per direct-to-LDS instruction
  // one input buffer (two of them alternate between chunks)
  static constexpr int bK = 0;                 // bf16 [64][128], pieces permuted per row
  static constexpr int bQ = bK + 64 * DK * 2;  // same
  static constexpr int bV = bQ + 64 * DK * 2;  // bf16 [64][BV]
  static constexpr int bG2 = bV + 64 * BV * 2; // float[64] G log2(e)
  static constexpr int bEG = bG2 + 256;        // float[64] exp(G)
  static constexpr int bB = bEG + 256;         // float[64] beta
  static constexpr int bMl = bB + 256;         // u32[64] ancestor-or-self mask, tokens 0..31
  static constexpr int bMh = bMl + 256;        // u32[64] same, tokens 32..63
  static constexpr int bOR = bMh + 256;        // int[64] output row or -1
  static constexpr int bFS = bOR + 256;        // int[64] fork slot or -1
  static constexpr int bSR = bFS + 256;        // int[64] state row or -1
  static constexpr int bD = bSR + 256;         // descriptor of the chunk in this buffer
  static constexpr int BUF = bD + 64;
  static constexpr int oND = 2 * BUF;                  // descriptors of the chunks to load, by parity
  static constexpr int oA = oND + 128;                 // fp32 [64][LDA]
  static constexpr int oP = oA + 64 * LDA * 4;         // bf16 [64][LDP]
  static constexpr int oDI = oP + 64 * LDP * 2;        // bf16 [4][16][LDD]
  static constexpr int oIMG = oDI + 4 * 16 * LDD * 2;  // bf16 [DK][LDI]
  static constexpr int bytes = oIMG + DK * LDI * 2;
  static_assert(bytes <= 160 * 1024, "LDS budget");
  static_assert(BUF % 16 == 0 && bV % 16 == 0 && bG2 % 16 == 0 && oA % 16 == 0 && oIMG % 16 == 0, "alignment");
};

struct Desc {
  int valid;         // 0: no chunk (the walk is over)
  int t0, n;         // first token, tokens in the chunk
  int h, v0;         // head, first column of the d_v tile
  int mode;          // 1: tree chunk (a whole sequence of <= 64 tokens)
  int sq;            // sequence
  int first;         // first chunk of its item: the waves load the entry state
  int need_exit;     // the chunk-exit state feeds a next chunk of the same segment
  int has_out;       // some token of the chunk has an output row
  unsigned req_lo, req_hi;  // tokens whose state is asked for (fork slot or state row)
  const float* sin;  // entry state rows of this tile (row v0), or null for zeros
  int pad[2];
};
static_assert(sizeof(Desc) <= 64, "descriptor");

struct Args {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* g;
  const __bf16* b;
  const int* parent;
  const float* init;
  __bf16* out;
  float* state_out;
  float* pv;
  float* fork_states;
  const int4* unit_info;
  const int* out_map;
  const int* state_map;
  const int* fork_slot;
  const unsigned long long* tree_mask;
  const unsigned long long* err;
  const int* level_count;
  const int* level_ptr;
  int H, Dv, NT, level, out_all;
};

__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ inline void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 16 bytes per lane from global memory (sbase + voff) straight into LDS: lane
// i's bytes land at lds_base + 16 i. Issued as inline assembly so that the
// compiler does not treat the copy as a pending write to all of LDS (it would
// otherwise wait for it before every LDS access); completion is awaited
// explicitly with wait_vm(). M0 holds the LDS base for the instruction; nothing
// else in this kernel uses M0.
__device__ inline void dma16(const void* sbase, unsigned voff, const void* lds_base) {
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)((const lds_void*)lds_base));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(l), "v"(voff), "s"(sbase)
               : "memory");
}

// 16-byte piece p of row r of a K or Q tile sits at slot p ^ kq_swz(r).
__device__ inline int kq_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// V rows of 8 pieces (d_v tile of 64) are permuted too; narrower rows need not be.
template <int BV>
__device__ inline int v_swz(int r) { return BV == 64 ? ((r & 3) << 1) : 0; }

__device__ inline i16x4 tr_read(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

__device__ inline bf16x8 cat8(i16x4 lo, i16x4 hi) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ inline bf16x4 to_bf4(f32x4 x) {
  bf16x4 r;
  r[0] = (__bf16)x[0];
  r[1] = (__bf16)x[1];
  r[2] = (__bf16)x[2];
  r[3] = (__bf16)x[3];
  return r;
}

__device__ inline bf16x4 neg_bf4(float4 x) {
  bf16x4 r;
  r[0] = (__bf16)(-x.x);
  r[1] = (__bf16)(-x.y);
  r[2] = (__bf16)(-x.z);
  r[3] = (__bf16)(-x.w);
  return r;
}

__device__ inline float bf_up(unsigned short x) { return __uint_as_float((unsigned)x << 16); }

__device__ inline f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }
__device__ inline f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0); }

template <typename T>
__device__ inline T lds_at(const unsigned char* base, int byte_off) {
  return *reinterpret_cast<const T*>(base + byte_off);
}

// --------------------------------------------------------------- item feed
// Wave 0 walks the level's items in a fixed order: the workgroups of one XCD
// share the units (segment, head) whose index is congruent to the XCD mod 8,
// so all d_v tiles of a unit read its q and k through the same L2, and the
// k-th workgroup of the XCD takes the XCD's items k, k + G, k + 2 G, ... (G
// workgroups per XCD). The unit record of the next item is loaded while the
// current one is walked.

struct Feed {
  int start, len, mode, sq, slot, h, tile, nch, c;
  bool cur;     // an item is being walked
  int li;       // XCD-local index of the next item to start
  int4 info_v;  // unit record of that item (in flight until the next vmcnt(0))
  bool nx_valid;
};

__device__ inline void feed_prefetch(Feed& f, const Args& a, int xcd, int count, int base) {
  const long long u = (long long)xcd + (long long)kXcd * (f.li / a.NT);
  f.nx_valid = u < (long long)count * a.H;
  f.info_v = make_int4(0, 0, 0, -1);
  if (f.nx_valid) f.info_v = a.unit_info[base + (int)(u / a.H)];
}

// The descriptor of the next chunk to load (valid = 0 when the level is done).
// Reads the prefetched unit record: call it only after a vmcnt(0).
template <int BV>
__device__ inline Desc feed_next(Feed& f, const Args& a, int xcd, int count, int base, int per_xcd) {
  Desc d;
  d.valid = 0;
  if (!(f.cur && f.c < f.nch)) {
    f.cur = false;
    if (!f.nx_valid) return d;
    const long long u = (long long)xcd + (long long)kXcd * (f.li / a.NT);
    f.start = __builtin_amdgcn_readfirstlane(f.info_v.x);
    f.len = __builtin_amdgcn_readfirstlane(f.info_v.y);
    const int ms = __builtin_amdgcn_readfirstlane(f.info_v.z);
    f.mode = ms & 1;
    f.sq = ms >> 1;
    f.slot = __builtin_amdgcn_readfirstlane(f.info_v.w);
    f.h = (int)(u % a.H);
    f.tile = f.li % a.NT;
    f.nch = f.mode ? 1 : (f.len + kChunk - 1) / kChunk;
    f.c = 0;
    f.cur = true;
    f.li += per_xcd;
    feed_prefetch(f, a, xcd, count, base);
  }
  const size_t SS = (size_t)a.Dv * DK;
  d.valid = 1;
  d.t0 = f.start + f.c * kChunk;
  d.n = min(kChunk, f.len - f.c * kChunk);
  d.h = f.h;
  d.v0 = f.tile * BV;
  d.mode = f.mode;
  d.sq = f.sq;
  d.first = f.c == 0;
  d.need_exit = (!f.mode) && (f.c + 1 < f.nch);
  d.has_out = 0;
  d.req_lo = d.req_hi = 0;
  d.sin = nullptr;
  if (d.first) {
    const float* s = f.slot >= 0 ? a.fork_states + ((size_t)f.slot * a.H + f.h) * SS
                                 : (a.init ? a.init + ((size_t)f.sq * a.H + f.h) * SS : nullptr);
    d.sin = s ? s + (size_t)d.v0 * DK : nullptr;
  }
  f.c += 1;
  return d;
}

// A descriptor read from LDS, with every field made wave-uniform.
__device__ inline Desc uniform_desc(const Desc& s) {
  Desc d;
  d.valid = __builtin_amdgcn_readfirstlane(s.valid);
  d.t0 = __builtin_amdgcn_readfirstlane(s.t0);
  d.n = __builtin_amdgcn_readfirstlane(s.n);
  d.h = __builtin_amdgcn_readfirstlane(s.h);
  d.v0 = __builtin_amdgcn_readfirstlane(s.v0);
  d.mode = __builtin_amdgcn_readfirstlane(s.mode);
  d.sq = __builtin_amdgcn_readfirstlane(s.sq);
  d.first = __builtin_amdgcn_readfirstlane(s.first);
  d.need_exit = __builtin_amdgcn_readfirstlane(s.need_exit);
  d.has_out = 0;
  d.req_lo = d.req_hi = 0;
  const unsigned long long p = (unsigned long long)s.sin;
  d.sin = (const float*)(((unsigned long long)__builtin_amdgcn_readfirstlane((unsigned)(p >> 32)) << 32) |
                         (unsigned)__builtin_amdgcn_readfirstlane((unsigned)p));
  return d;
}

__device__ inline void put_desc(unsigned char* p, const Desc& d, int lane) {
  if (lane == 0) *reinterpret_cast<Desc*>(p) = d;
}

// ------------------------------------------------------------ chunk loads

// This wave's share of the direct-to-LDS copies of chunk d into buffer buf.
// Rows at or beyond d.n are zero-filled.
template <int BV>
__device__ inline void issue_chunk_loads(const Args& a, const Desc& d, unsigned char* buf, int w, int lane) {
  using L = Lay<BV>;
  constexpr int kKQ = 16;  // instructions per K (or Q) tile: 4 rows each
  constexpr int kAll = 2 * kKQ + L::VPR;
  const unsigned H = a.H, Dv = a.Dv;
  const int g4 = lane >> 4, l16 = lane & 15;
  const bool full = d.n == kChunk;
  // K, Q: row 4 blk + g4, slot l16 holds piece l16 ^ kq_swz(row)
  const unsigned kq_row0 = (((unsigned)d.t0 + g4) * H + d.h) * (DK * 2);
  const unsigned kq_step = 4u * H * (DK * 2);  // bytes per instruction (4 rows)
  // V: row blk * RPI + lane / VPR, slot lane % VPR
  const int vr = lane / L::VPR, vs = lane % L::VPR;
  const unsigned v_row0 = (((unsigned)d.t0 + vr) * H + d.h) * (Dv * 2) + (unsigned)d.v0 * 2 +
                          (unsigned)((vs ^ v_swz<BV>(vr)) * 16);
  const unsigned v_step = (unsigned)L::RPI * H * (Dv * 2);
  for (int ins = w; ins < kAll; ins += L::NS) {
    unsigned char* dst;
    const void* sbase;
    unsigned voff;
    int row;
    if (ins < 2 * kKQ) {
      const bool isK = ins < kKQ;
      const int blk = isK ? ins : ins - kKQ;
      row = 4 * blk + g4;
      dst = buf + (isK ? L::bK : L::bQ) + blk * 1024;
      sbase = reinterpret_cast<const unsigned char*>(isK ? a.k : a.q) + (size_t)blk * kq_step;
      voff = kq_row0 + (unsigned)((l16 ^ ((g4 << 2) | (blk & 3))) * 16);
    } else {
      const int blk = ins - 2 * kKQ;
      row = blk * L::RPI + vr;
      dst = buf + L::bV + blk * 1024;
      sbase = reinterpret_cast<const unsigned char*>(a.v) + (size_t)blk * v_step;
      voff = v_row0;
    }
    if (full || row < d.n) dma16(sbase, voff, dst);
    else *reinterpret_cast<uint4*>(dst + lane * 16) = make_uint4(0, 0, 0, 0);
  }
}

// Raw per-token values of a chunk (one token per lane), converted only after
// the chunk's wait_vm() so that no compiler wait lands among the copies.
struct TokenRegs {
  unsigned short g, b;  // bf16 bits
  int par, om, sm, fs;
};

__device__ inline TokenRegs load_tokens(const Args& a, const Desc& d, int lane) {
  TokenRegs r;
  r.g = 0;
  r.b = 0;
  r.par = -1;
  r.om = kUnmapped;
  r.sm = kUnmapped;
  r.fs = -1;
  if (d.valid && lane < d.n) {
    const int t = d.t0 + lane;
    r.g = reinterpret_cast<const unsigned short*>(a.g)[(size_t)t * a.H + d.h];
    r.b = reinterpret_cast<const unsigned short*>(a.b)[(size_t)t * a.H + d.h];
    if (d.mode) r.par = a.parent[t];
    r.om = a.out_all ? t : a.out_map[t];
    r.sm = a.state_map[t];
    r.fs = a.fork_slot[t];
  }
  return r;
}

// Wave 0: token tables of chunk d into buffer buf.
template <int BV>
__device__ inline void store_tokens(const Args& a, Desc d, const TokenRegs& r, unsigned char* buf, int lane) {
  using L = Lay<BV>;
  if (!d.valid) {
    put_desc(buf + L::bD, d, lane);
    return;
  }
  // chunk-local path sums of log gates: a prefix sum on a chain, pointer
  // jumping over in-chunk parents in a tree chunk (six rounds cover 64 levels)
  const int i = lane;
  const bool valid = i < d.n;
  float G = bf_up(r.g);
  unsigned long long mask;
  if (d.mode) {
    int pj = (valid && r.par >= d.t0 && r.par < d.t0 + i) ? r.par - d.t0 : -1;
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      const int src = pj >= 0 ? pj : i;
      const float pG = __shfl(G, src);
      const int pp = __shfl(pj, src);
      if (pj >= 0) {
        G += pG;
        pj = pp;
      }
    }
    mask = a.tree_mask[(size_t)d.sq * kChunk + i];
  } else {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_up(G, off);
      if (i >= off) G += o;
    }
    mask = (i == 63) ? ~0ull : ((2ull << i) - 1ull);
  }
  const int orow = (valid && r.om != kUnmapped) ? r.om : -1;
  const int fs = valid ? r.fs : -1;
  const int sr = (valid && r.sm != kUnmapped) ? r.sm : -1;
  reinterpret_cast<float*>(buf + L::bG2)[i] = G * kLog2e;
  reinterpret_cast<float*>(buf + L::bEG)[i] = __expf(G);
  reinterpret_cast<float*>(buf + L::bB)[i] = bf_up(r.b);
  reinterpret_cast<unsigned*>(buf + L::bMl)[i] = (unsigned)mask;
  reinterpret_cast<unsigned*>(buf + L::bMh)[i] = (unsigned)(mask >> 32);
  reinterpret_cast<int*>(buf + L::bOR)[i] = orow;
  reinterpret_cast<int*>(buf + L::bFS)[i] = fs;
  reinterpret_cast<int*>(buf + L::bSR)[i] = sr;
  const unsigned long long rq = __ballot(fs >= 0 || sr >= 0);
  d.has_out = __ballot(orow >= 0) != 0ull;
  d.req_lo = (unsigned)rq;
  d.req_hi = (unsigned)(rq >> 32);
  put_desc(buf + L::bD, d, lane);
}

// ------------------------------------------------------------------ kernel

template <int BV>
__global__ void __launch_bounds__(Lay<BV>::NTHR, 1) k_walk_mfma(const Args a) {
  using L = Lay<BV>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int g4 = lane >> 4, l16 = lane & 15;
  if (*a.err != kNoError) return;  // structural error: nothing is computed
  const int count = a.level_count[a.level];
  const int base = a.level_ptr[a.level];
  const int xcd = blockIdx.x % kXcd;
  const unsigned HDv = (unsigned)a.H * a.Dv;

  // P is only written on and below its diagonal blocks; the products read
  // whole 32-token k-steps, so the blocks above must hold zeros.
  for (int e = tid; e < 64 * L::LDP; e += L::NTHR) reinterpret_cast<__bf16*>(smem + L::oP)[e] = (__bf16)0.f;

  // ---- per-lane LDS byte offsets (buffer-relative for K, Q, V)
  int oKQ[4];  // A/B fragment of K or Q rows 0..15 (row block rb adds 4096 rb)
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) oKQ[ks] = l16 * 256 + (((4 * ks + g4) ^ kq_swz(l16)) << 4);
  int oKT[8];  // transposed read of K rows 4 g4 + l16/4 (block pairs add 8192, second block 4096)
  {
    const int r0 = 4 * g4 + (l16 >> 2);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      oKT[dt] = r0 * 256 + (((2 * dt + ((l16 & 3) >> 1)) ^ kq_swz(r0)) << 4) + ((l16 & 1) << 3);
  }
  int oV;  // transposed read of V rows 4 g4 + l16/4, columns 16 w .. +15 (row block rb adds 32 BV rb)
  {
    const int vrow = 4 * g4 + (l16 >> 2), vcol = 16 * w + (l16 & 3) * 4;
    oV = L::bV + vrow * BV * 2 + (((vcol >> 3) ^ v_swz<BV>(vrow)) << 4) + ((vcol & 7) << 1);
  }
  const int oSb = L::oIMG + (8 * g4 + (l16 >> 2)) * L::LDI * 2 + (16 * w + (l16 & 3) * 4) * 2;
  const int oImgW = L::oIMG + l16 * L::LDI * 2 + (16 * w + 4 * g4) * 2;
  const int oPr = L::oP + (l16 * L::LDP + 4 * g4) * 2;
  const int oAr = L::oA + (l16 * L::LDA + 4 * g4) * 4;
  const int oDr = L::oDI + (l16 * L::LDD + 4 * g4) * 2;
  const int oAw = L::oA + (4 * g4 * L::LDA + l16) * 4;
  const int oPw = L::oP + (4 * g4 * L::LDP + l16) * 2;

  // ---- prologue: describe the first two chunks, load the first into buffer 0
  const int per_xcd = gridDim.x / kXcd;
  Feed f;
  f.cur = false;
  f.li = blockIdx.x / kXcd;
  f.nx_valid = false;
  Desc* nds = reinterpret_cast<Desc*>(smem + L::oND);  // [2]: descriptors of chunks to load, by chunk parity
  if (w == 0) {
    feed_prefetch(f, a, xcd, count, base);
    wait_vm();
    put_desc(reinterpret_cast<unsigned char*>(nds + 0), feed_next<BV>(f, a, xcd, count, base, per_xcd), lane);
    wait_vm();
    put_desc(reinterpret_cast<unsigned char*>(nds + 1), feed_next<BV>(f, a, xcd, count, base, per_xcd), lane);
  }
  lds_barrier();
  TokenRegs tr;
  {
    const Desc nd = uniform_desc(nds[0]);
    if (w == 0) tr = load_tokens(a, nd, lane);
    if (nd.valid) issue_chunk_loads<BV>(a, nd, smem, w, lane);
    wait_vm();
    if (w == 0) store_tokens<BV>(a, nd, tr, smem, lane);
  }
  lds_barrier();

  // the wave's 16 x 128 rows of S in the accumulator layout:
  // lane holds S[16 w + 4 g4 + r][16 dt + l16]
  f32x4 S[8];
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) S[dt] = zero;
  const size_t SS = (size_t)a.Dv * DK;

  for (int it = 0;; ++it) {
    const unsigned char* buf = smem + (it & 1) * L::BUF;
    unsigned char* nbuf = smem + ((it + 1) & 1) * L::BUF;
    const Desc* dp = reinterpret_cast<const Desc*>(buf + L::bD);
    if (!__builtin_amdgcn_readfirstlane(dp->valid)) break;
    // descriptor fields are the same for every lane: keep them scalar
    const int t0 = __builtin_amdgcn_readfirstlane(dp->t0), n = __builtin_amdgcn_readfirstlane(dp->n);
    const int h = __builtin_amdgcn_readfirstlane(dp->h), v0 = __builtin_amdgcn_readfirstlane(dp->v0);
    const int mode = __builtin_amdgcn_readfirstlane(dp->mode);
    const bool has_out = __builtin_amdgcn_readfirstlane(dp->has_out);
    const bool need_exit = __builtin_amdgcn_readfirstlane(dp->need_exit);
    const bool first = __builtin_amdgcn_readfirstlane(dp->first);
    const unsigned req_lo = __builtin_amdgcn_readfirstlane(dp->req_lo), req_hi = __builtin_amdgcn_readfirstlane(dp->req_hi);
    const Desc nd = uniform_desc(nds[(it + 1) & 1]);
    const int bo = (it & 1) * L::BUF;  // byte offset of this chunk's buffer

    // ---------------------------------------------------- stage 1: on-chip work
    // entry state of a new item first: its loads must not queue behind the copies
    if (first) {
      const unsigned long long sp = (unsigned long long)dp->sin;
      const float* sin = (const float*)(((unsigned long long)__builtin_amdgcn_readfirstlane((unsigned)(sp >> 32)) << 32) |
                                        (unsigned)__builtin_amdgcn_readfirstlane((unsigned)sp));
      if (sin) {
        const float* row = sin + (size_t)(16 * w + 4 * g4) * DK + l16;
        float t[8][4];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) t[dt][r] = __builtin_nontemporal_load(row + (size_t)r * DK + 16 * dt);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) S[dt] = f32x4{t[dt][0], t[dt][1], t[dt][2], t[dt][3]};
      } else {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) S[dt] = zero;
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<bf16x4*>(smem + oImgW + dt * 16 * L::LDI * 2) = to_bf4(S[dt]);
    }
    // token values of the next chunk, then start copying it into the other buffer
    if (w == 0) tr = load_tokens(a, nd, lane);
    if (nd.valid) issue_chunk_loads<BV>(a, nd, nbuf, w, lane);

    // K fragments of this chunk and the state image as B operands
    bf16x8 Kf[4][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const unsigned char* kb = smem + bo + L::bK + oKQ[ks];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) Kf[rb][ks] = lds_at<bf16x8>(kb, rb * 4096);
    }
    bf16x8 Sb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const unsigned char* p = smem + oSb + ks * 32 * L::LDI * 2;
      Sb[ks] = cat8(tr_read(p), tr_read(p + 4 * L::LDI * 2));
    }
    // K S_e^T for the wave's columns
    f32x4 X[4], O[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      X[rb] = zero;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) X[rb] = mma32(Kf[rb][ks], Sb[ks], X[rb]);
    }
    // Row block by row block: Q fragments (when the chunk has outputs), Q S_e^T,
    // and the A and P tiles of (row block, column block) pairs. The diagonal
    // pairs and the inversion go to wave WI, the six off-diagonal pairs
    // round-robin to the others (all of them to wave 0 when it is alone).
    const float* sG2 = reinterpret_cast<const float*>(buf + L::bG2);
    const float* sB = reinterpret_cast<const float*>(buf + L::bB);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      bf16x8 Qr[4];
      if (has_out) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) Qr[ks] = lds_at<bf16x8>(smem + bo + L::bQ + oKQ[ks], rb * 4096);
        O[rb] = zero;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) O[rb] = mma32(Qr[ks], Sb[ks], O[rb]);
      }
      const int i0 = 16 * rb + 4 * g4;
      const float4 g2i4 = *reinterpret_cast<const float4*>(sG2 + i0);
      const float4 bi4 = *reinterpret_cast<const float4*>(sB + i0);
      const float gi[4] = {g2i4.x, g2i4.y, g2i4.z, g2i4.w};
      const float bb[4] = {bi4.x, bi4.y, bi4.z, bi4.w};
#pragma unroll
      for (int cb = 0; cb <= rb; ++cb) {
        const bool diag = cb == rb;
        const int pix = rb * (rb - 1) / 2 + cb;  // index among the off-diagonal pairs
        const bool mine = diag ? (w == L::WI) : (L::NS == 1 || (w != L::WI && pix % (L::NS - 1) == w));
        if (!mine) continue;
        f32x4 accA = zero, accP = zero;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) accA = mma32(Kf[rb][ks], Kf[cb][ks], accA);
        if (has_out) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) accP = mma32(Qr[ks], Kf[cb][ks], accP);
        }
        const int j = 16 * cb + l16;
        const float g2j = sG2[j];
        // decay exp(G_i - G_j) where j is an ancestor-or-self of i, else 0
        float e[4];
        if (!mode) {  // chain: every earlier token is an ancestor
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x = __builtin_amdgcn_exp2f(gi[r] - g2j);
            e[r] = (!diag || 4 * g4 + r >= l16) ? x : 0.f;
          }
        } else {
          const uint4 mk = *reinterpret_cast<const uint4*>(buf + (cb >= 2 ? L::bMh : L::bMl) + i0 * 4);
          const unsigned mm[4] = {mk.x, mk.y, mk.z, mk.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x = __builtin_amdgcn_exp2f(gi[r] - g2j);
            e[r] = ((mm[r] >> (j & 31)) & 1u) ? x : 0.f;
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float av = bb[r] * e[r] * accA[r];
          *reinterpret_cast<float*>(smem + oAw + ((16 * rb + r) * L::LDA + 16 * cb) * 4) =
              (!diag || 4 * g4 + r != l16) ? av : 0.f;
          if (has_out)
            *reinterpret_cast<__bf16*>(smem + oPw + ((16 * rb + r) * L::LDP + 16 * cb) * 2) = (__bf16)(e[r] * accP[r]);
        }
      }
    }
    if (w == L::WI) {
      // inverse of the diagonal block g4 of I + A, column l16, by forward substitution (fp32)
      const float* blkA = reinterpret_cast<const float*>(smem + L::oA) + 16 * g4 * L::LDA + 16 * g4;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float nr[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 t = *reinterpret_cast<const float4*>(blkA + r * L::LDA + 4 * q);
          nr[4 * q] = t.x;
          nr[4 * q + 1] = t.y;
          nr[4 * q + 2] = t.z;
          nr[4 * q + 3] = t.w;
        }
        float acc = (r == l16) ? 1.f : 0.f;
#pragma unroll
        for (int c = 0; c < r; ++c) acc -= nr[c] * x[c];
        x[r] = acc;
      }
      __bf16* dst = reinterpret_cast<__bf16*>(smem + L::oDI) + 16 * g4 * L::LDD + l16;
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[r * L::LDD] = (__bf16)x[r];
    }
    // R = beta (V - e^G K S^T) in place of X, and the e^G Q S^T part of O
    const float* sEG = reinterpret_cast<const float*>(buf + L::bEG);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const bf16x4 vb = __builtin_bit_cast(bf16x4, tr_read(smem + bo + oV + rb * 32 * BV));
      const float4 eg = *reinterpret_cast<const float4*>(sEG + 16 * rb + 4 * g4);
      const float4 bi = *reinterpret_cast<const float4*>(sB + 16 * rb + 4 * g4);
      X[rb][0] = bi.x * ((float)vb[0] - eg.x * X[rb][0]);
      X[rb][1] = bi.y * ((float)vb[1] - eg.y * X[rb][1]);
      X[rb][2] = bi.z * ((float)vb[2] - eg.z * X[rb][2]);
      X[rb][3] = bi.w * ((float)vb[3] - eg.w * X[rb][3]);
      if (has_out) {
        O[rb][0] *= eg.x;
        O[rb][1] *= eg.y;
        O[rb][2] *= eg.z;
        O[rb][3] *= eg.w;
      }
    }
    wait_vm();  // the next chunk's copies, token values and unit record have landed
    if (w == 0) {
      Desc nn;
      nn.valid = 0;
      if (nd.valid) nn = feed_next<BV>(f, a, xcd, count, base, per_xcd);
      put_desc(reinterpret_cast<unsigned char*>(nds + (it & 1)), nn, lane);
    }
    lds_barrier();

    // ------------------------------------------ stage 2: substitution and outputs
    auto dinv = [&](int b) { return lds_at<bf16x4>(smem + oDr, b * 16 * L::LDD * 2); };
    auto ablk = [&](int b, int mb) { return neg_bf4(lds_at<float4>(smem + oAr, (16 * b * L::LDA + 16 * mb) * 4)); };
    f32x4 Vt[4];
    bf16x4 Vb[4];
    Vt[0] = mma16(dinv(0), to_bf4(X[0]), zero);
    Vb[0] = to_bf4(Vt[0]);
    {
      f32x4 y = mma16(ablk(1, 0), Vb[0], X[1]);
      Vt[1] = mma16(dinv(1), to_bf4(y), zero);
      Vb[1] = to_bf4(Vt[1]);
    }
    {
      f32x4 y = mma16(ablk(2, 0), Vb[0], X[2]);
      y = mma16(ablk(2, 1), Vb[1], y);
      Vt[2] = mma16(dinv(2), to_bf4(y), zero);
      Vb[2] = to_bf4(Vt[2]);
    }
    {
      f32x4 y = mma16(ablk(3, 0), Vb[0], X[3]);
      y = mma16(ablk(3, 1), Vb[1], y);
      y = mma16(ablk(3, 2), Vb[2], y);
      Vt[3] = mma16(dinv(3), to_bf4(y), zero);
      Vb[3] = to_bf4(Vt[3]);
    }
    const unsigned col = (unsigned)v0 + 16 * w + l16;
    const unsigned hcol = (unsigned)h * a.Dv + col;
    if (a.pv) {
      float* pvb = a.pv + ((unsigned)t0 + 4 * g4) * HDv + hcol;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n == kChunk || 16 * rb + 4 * g4 + r < n) pvb[(16 * rb + r) * HDv] = Vt[rb][r];
    }
    if (has_out) {
      const bool all_rows = a.out_all && n == kChunk;
      // O += P Vt over pairs of 16-token blocks (blocks of P above the diagonal are zero)
      const int* sOR = reinterpret_cast<const int*>(buf + L::bOR);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
        for (int mp = 0; mp < 2; ++mp) {
          if (2 * mp > rb) continue;
          const unsigned char* prow = smem + oPr + (16 * rb * L::LDP + 32 * mp) * 2;
          const bf16x8 pa = cat8(lds_at<i16x4>(prow, 0), lds_at<i16x4>(prow, 32));
          const bf16x8 vb = __builtin_shufflevector(Vb[2 * mp], Vb[2 * mp + 1], 0, 1, 2, 3, 4, 5, 6, 7);
          O[rb] = mma32(pa, vb, O[rb]);
        }
        if (all_rows) {  // every token of a full chunk is an output row, in stream order
          __bf16* ob = a.out + ((unsigned)t0 + 4 * g4) * HDv + hcol;
#pragma unroll
          for (int r = 0; r < 4; ++r) ob[(16 * rb + r) * HDv] = (__bf16)O[rb][r];
        } else {
          const int4 orow = *reinterpret_cast<const int4*>(sOR + 16 * rb + 4 * g4);
          const int ors[4] = {orow.x, orow.y, orow.z, orow.w};
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (ors[r] >= 0) a.out[(unsigned)ors[r] * HDv + hcol] = (__bf16)O[rb][r];
        }
      }
    }
    // states after requested tokens (fork slots, state rows) and at the chunk exit
    unsigned long long todo = ((unsigned long long)req_hi << 32) | req_lo;
    if (need_exit) todo |= 1ull << (n - 1);
    if (todo) {
      const int* sFS = reinterpret_cast<const int*>(buf + L::bFS);
      const int* sSR = reinterpret_cast<const int*>(buf + L::bSR);
      do {
        const int p = __builtin_ctzll(todo);
        todo &= todo - 1ull;
        const unsigned mlo = reinterpret_cast<const unsigned*>(buf + L::bMl)[p];
        const unsigned mhi = reinterpret_cast<const unsigned*>(buf + L::bMh)[p];
        const float g2p = sG2[p];
        bf16x4 Wb[4];
        // masked, decayed pseudo-values exp(G_p - G_j) vt_j for j ancestor-or-self of p; on a
        // chain the last token needs no mask (rows past n are zero)
        const bool nomask = !mode && p == n - 1;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const float4 g2 = *reinterpret_cast<const float4*>(sG2 + 16 * mb + 4 * g4);
          const float gj[4] = {g2.x, g2.y, g2.z, g2.w};
          f32x4 wv;
          if (nomask) {
#pragma unroll
            for (int r = 0; r < 4; ++r) wv[r] = Vt[mb][r] * __builtin_amdgcn_exp2f(g2p - gj[r]);
          } else {
            const unsigned mword = mb >= 2 ? mhi : mlo;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int j = 16 * mb + 4 * g4 + r;
              const bool anc = mode ? ((mword >> (j & 31)) & 1u) : (j <= p);
              wv[r] = anc ? Vt[mb][r] * __builtin_amdgcn_exp2f(g2p - gj[r]) : 0.f;
            }
          }
          Wb[mb] = to_bf4(wv);
        }
        const float cS = sEG[p];
        const bool is_exit = need_exit && p == n - 1;
        const int fs = sFS[p], sr = sSR[p];
        float* dst_slot = fs >= 0 ? a.fork_states + ((size_t)fs * a.H + h) * SS : nullptr;
        float* dst_row = sr >= 0 ? a.state_out + ((size_t)sr * a.H + h) * SS : nullptr;
        const bool two = p >= 32;
        const bf16x8 w01 = __builtin_shufflevector(Wb[0], Wb[1], 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 w23 = __builtin_shufflevector(Wb[2], Wb[3], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          f32x4 acc;
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] = cS * S[dt][r];
          // B operand: K[j][16 dt + l16] for j in blocks 2 mp and 2 mp + 1, rows 4 g4 .. 4 g4 + 3 of each
          const unsigned char* kp = smem + bo + L::bK + oKT[dt];
          acc = mma32(w01, cat8(tr_read(kp), tr_read(kp + 4096)), acc);
          if (two) acc = mma32(w23, cat8(tr_read(kp + 8192), tr_read(kp + 8192 + 4096)), acc);
          const size_t off = (size_t)(v0 + 16 * w + 4 * g4) * DK + 16 * dt + l16;
          if (dst_slot) {
#pragma unroll
            for (int r = 0; r < 4; ++r) dst_slot[off + (size_t)r * DK] = acc[r];
          }
          if (dst_row) {
#pragma unroll
            for (int r = 0; r < 4; ++r) dst_row[off + (size_t)r * DK] = acc[r];
          }
          if (is_exit) {
            S[dt] = acc;
            *reinterpret_cast<bf16x4*>(smem + oImgW + dt * 16 * L::LDI * 2) = to_bf4(acc);
          }
        }
      } while (todo);
    }
    // wave 0: token tables of the next chunk
    if (w == 0) store_tokens<BV>(a, nd, tr, nbuf, lane);
    lds_barrier();
  }
}

template <int BV>
hipError_t run(const Args& wa, int levels, hipStream_t s) {
  auto kern = k_walk_mfma<BV>;
  constexpr int bytes = Lay<BV>::bytes;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     bytes);
  if (e != hipSuccess) return e;
  int dev = 0, cus = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // one workgroup per CU (bounded by LDS), persistent over the level's items;
  // a multiple of the XCD count so that every XCD has the same number of workgroups
  const int grid = cus >= kXcd ? cus / kXcd * kXcd : kXcd;
  for (int l = 0; l < levels; ++l) {
    Args x = wa;
    x.level = l;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(Lay<BV>::NTHR), bytes, s, x);
  }
  return hipGetLastError();
}

}  // namespace

bool walk_mfma_supported(int dtype, int dk, int bv) {
  return dtype == GDN_BF16 && dk == DK && (bv == 16 || bv == 32 || bv == 64);
}

bool walk_mfma_fits(const gdn_tree_dims& d) {
  // the kernel addresses q, k, v, out and pseudo_v with 32-bit element offsets
  const long long per_token = (long long)d.H * (d.Dk > d.Dv ? d.Dk : d.Dv);
  return d.T * per_token < (1ll << 30);
}

hipError_t launch_walk_mfma(const gdn_tree_fwd_args& fa, const Meta& m, int bv, hipStream_t s) {
  Args wa;
  wa.q = reinterpret_cast<const __bf16*>(fa.q);
  wa.k = reinterpret_cast<const __bf16*>(fa.k);
  wa.v = reinterpret_cast<const __bf16*>(fa.v);
  wa.g = reinterpret_cast<const __bf16*>(fa.log_gate);
  wa.b = reinterpret_cast<const __bf16*>(fa.beta);
  wa.parent = fa.parent_idx;
  wa.init = fa.init_state;
  wa.out = reinterpret_cast<__bf16*>(fa.out);
  wa.state_out = fa.state_out;
  wa.pv = fa.pseudo_v;
  wa.fork_states = m.fork_states;
  wa.unit_info = m.unit_info;
  wa.out_map = m.out_map;
  wa.state_map = m.state_map;
  wa.fork_slot = m.fork_slot;
  wa.tree_mask = m.tree_mask;
  wa.err = m.err;
  wa.level_count = m.level_count;
  wa.level_ptr = m.level_ptr;
  wa.H = fa.dims.H;
  wa.Dv = fa.dims.Dv;
  wa.NT = fa.dims.Dv / bv;
  wa.level = 0;
  wa.out_all = fa.out_rows == nullptr;
  const int L = fa.dims.max_levels;
  switch (bv) {
    case 16: return run<16>(wa, L, s);
    case 32: return run<32>(wa, L, s);
    case 64: return run<64>(wa, L, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn
