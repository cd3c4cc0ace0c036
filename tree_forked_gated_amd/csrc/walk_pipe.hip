// Chunked tree-WY walk for bf16 inputs with d_k = 128 on gfx950: a software
// pipeline over chunks with specialised waves.
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
// I + A are inverted in fp32, and Vt_b = (I + A_bb)^{-1} (R_b - sum over m < b
// of A_bm Vt_m).
//
// Only the products with S_e depend on the previous chunk. A workgroup walks
// one (segment, head, d_v tile) item after another and splits each chunk's
// work by that line:
//
// * state waves (one per 16 columns of the d_v tile, per 32 in a tile of 64)
//   hold their rows of S in
//   fp32 registers and do everything that involves S: K S_e^T, R, the block
//   substitution, Q S_e^T and P Vt, the outputs and pseudo-values, and the
//   states after requested tokens and at the chunk exit;
// * two helper waves work one chunk ahead: from that chunk's K and Q they form
//   the A tiles, the inverses of the diagonal blocks and the masked, decayed
//   P = M . exp . Q K^T, and leave them in LDS as ready MFMA operands. They
//   also copy q two chunks ahead and v one chunk ahead from HBM into LDS
//   (direct-to-LDS loads), and k two chunks ahead in a tile of 64 columns (in
//   narrower tiles the state waves copy k); the first helper also walks the
//   item list and the second prepares each chunk's token tables.
//
// One barrier per chunk separates the stages. The state is kept transposed in
// the MFMA accumulator layout, with its d_k index permuted so that the
// accumulators, converted to bf16, are directly the B operands of K S_e^T and
// Q S_e^T; the update takes its K^T operand with transposing LDS reads.
//
// Reduction orders depend only on the chunk's own tokens (never on the d_v
// tile width, the grid or other items), so results are bitwise independent of
// the batch around a sequence and of the d_v tile.
#include "gdn_internal.h"

namespace gdn {
namespace {

// Stage stamps, in a measurement build only (compiled with -DGDN_WALK_STAMPS;
// the library itself has none): s_memtime at the stage boundaries of every wave
// of the first kStampWg workgroups, over the first kStampIts chunks of the
// first level launch, read back with gdn_walk_stamps(). Lane 0 stores them
// with ordinary vector stores.
#ifdef GDN_WALK_STAMPS
constexpr int kStampWg = 8, kStampWaves = 4, kStampIts = 128, kStampPts = 10;
__device__ unsigned long long g_walk_stamps[kStampWg * kStampWaves * kStampIts * kStampPts];
#define WALK_STAMP(IT, S)                                                                                   \
  do {                                                                                                      \
    const int w_ = (int)(threadIdx.x >> 6), i_ = (IT);                                                     \
    if (blockIdx.x < kStampWg && a.level == 0 && i_ >= 0 && i_ < kStampIts && (threadIdx.x & 63) == 0 &&    \
        w_ < kStampWaves)                                                                                   \
      g_walk_stamps[(((int)blockIdx.x * kStampWaves + w_) * kStampIts + i_) * kStampPts + (S)] =           \
          __builtin_amdgcn_s_memtime();                                                                     \
  } while (0)
#else
#define WALK_STAMP(IT, S) \
  do {                    \
  } while (0)
#endif

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
// Global-memory view of a state row. The entry-state pointer comes from a
// descriptor in LDS, so the compiler cannot tell its address space; through a
// generic pointer the loads would be flat loads, which also count against the
// LDS wait counter and would hold up every later LDS wait.
typedef __attribute__((address_space(1))) const f32x4 gf32x4;

constexpr int DK = 128;
constexpr int kXcd = kWalkQueues;  // workgroup b runs on XCD b % 8 of an MI355X
constexpr float kLog2e = 1.4426950408889634f;

// Token tables of one chunk (byte offsets): 64 entries each.
constexpr int tG2 = 0;      // float G log2(e)
constexpr int tEG = 256;    // float exp(G)
constexpr int tB = 512;     // float beta
constexpr int tDX = 768;    // float exp(G_{n-1} - G_j) for j < n, else 0 (decay to the chunk exit)
constexpr int tMl = 1024;   // u32 ancestor-or-self mask, tokens 0..31
constexpr int tMh = 1280;   // u32 same, tokens 32..63
constexpr int tOR = 1536;   // int output row or -1
constexpr int tFS = 1792;   // int fork slot or -1
constexpr int tSR = 2048;   // int state row or -1
constexpr int tD = 2304;    // chunk descriptor
constexpr int kTB = 2368;

// Products of one chunk, laid out as per-lane MFMA operands (byte offsets).
constexpr int pNA = 0;              // 6 blocks x 64 lanes x 8 B: -A_bm (m < b), 16x16x16 A operands
constexpr int kDIS = 640;           // stride between diagonal inverses (512 B used)
constexpr int pDI = 3072;           // 4 blocks: (I + A_bb)^{-1}, 16x16x16 A operands
constexpr int kPR = pDI + 4 * kDIS;
// P of one chunk: 6 pairs x 64 lanes x 16 B (row block x 32 tokens), 16x16x32 operands.
// It lives one iteration longer than the other products: the state waves
// finish a chunk's output during the next chunk.
constexpr int kPP = 6 * 1024;
// fp32 staging of one helper's diagonal blocks of A, transposed: [4][16][kLTR] + pad
constexpr int kLTR = 20;
constexpr int kLTS = 16 * kLTR + 4;

template <int BV>
struct Cfg {
  static constexpr int NB = BV == 64 ? 2 : 1;  // 16-column blocks per state wave
  static constexpr int NS = BV / (16 * NB);    // state waves
  static constexpr int NW = NS + 2;            // plus two helpers
  static constexpr int NTHR = 64 * NW;
  static constexpr int VPR = BV / 8;    // 16-byte pieces per V row
  static constexpr int RPI = 64 / VPR;  // V rows per direct-to-LDS instruction
  static constexpr int VT = 64 * BV * 2;
  static constexpr int oKQ = 0;                  // [3] K tile (16 KB) then Q tile (16 KB)
  static constexpr int oTB = oKQ + 3 * 32768;    // [3] token tables
  static constexpr int oV = oTB + 3 * kTB;       // [2] V tiles bf16 [64][BV]
  static constexpr int oPR = oV + 2 * VT;        // [2] -A blocks and diagonal inverses
  static constexpr int oPP = oPR + 2 * kPR;      // [3] P
  static constexpr int oLT = oPP + 3 * kPP;      // diagonal-block staging
  static constexpr int oND = oLT + 4 * kLTS * 4; // [2] descriptors of chunks to copy, by parity
  static constexpr int bytes = oND + 128;
  static_assert(bytes <= 160 * 1024, "LDS budget");
  static_assert(oTB % 16 == 0 && oV % 16 == 0 && oPR % 16 == 0 && oPP % 16 == 0 && oLT % 16 == 0 && oND % 16 == 0,
                "alignment");
};

struct Desc {
  int valid;         // 0: no chunk (the walk is over)
  int t0, n;         // first token, tokens in the chunk
  int h, v0;         // head, first column of the d_v tile
  int mode;          // 1: tree chunk (a whole sequence of <= 64 tokens)
  int sq;            // sequence
  int first;         // first chunk of its item: the state waves load the entry state
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
  int* walk_ctr;  // per level: items claimed so far per XCD (zeroed by the plan), fewest and most chunks of an item
  int H, Dv, NT, level, out_all;
};

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// 16 bytes per lane from global memory (sbase + voff) straight into LDS: lane
// i's bytes land at lds_addr + 16 i. Issued as inline assembly so that the
// compiler does not treat the copy as a pending write to all of LDS (it would
// otherwise wait for it before every LDS access); completion is awaited
// explicitly with wait_vm(). M0 holds the LDS base for the instruction; nothing
// else in this kernel uses M0.
__device__ __forceinline__ void dma16(const void* sbase, unsigned voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_addr), "v"(voff), "s"(sbase)
               : "memory");
}

// LDS address of a byte of the kernel's shared buffer (32-bit, wave-uniform).
__device__ __forceinline__ uint32_t lds_addr_of(const unsigned char* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)((const lds_void*)p));
}

// 16-byte piece p of row r of a K or Q tile sits at slot p ^ kq_swz(r).
__device__ __forceinline__ int kq_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// V rows of 8 pieces (d_v tile of 64) are permuted too; narrower rows need not be.
template <int BV>
__device__ __forceinline__ int v_swz(int r) { return BV == 64 ? ((r & 3) << 1) : 0; }

__device__ __forceinline__ i16x4 tr_read(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

__device__ __forceinline__ bf16x8 cat8(i16x4 lo, i16x4 hi) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ bf16x8 cat8b(bf16x4 lo, bf16x4 hi) { return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7); }

__device__ __forceinline__ bf16x4 to_bf4(f32x4 x) {
  bf16x4 r;
  r[0] = (__bf16)x[0];
  r[1] = (__bf16)x[1];
  r[2] = (__bf16)x[2];
  r[3] = (__bf16)x[3];
  return r;
}

__device__ __forceinline__ float bf_up(unsigned short x) { return __uint_as_float((unsigned)x << 16); }

__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0); }

template <typename T>
__device__ __forceinline__ T lds_at(const unsigned char* base, int byte_off) {
  return *reinterpret_cast<const T*>(base + byte_off);
}

__device__ __forceinline__ int rfl(int x) { return __builtin_amdgcn_readfirstlane(x); }

// --------------------------------------------------------------- item feed
// The workgroups of one XCD share the units (segment, head) whose index is
// congruent to the XCD mod 8, so all d_v tiles of a unit read its q and k
// through the same L2. The k-th workgroup of an XCD starts with the XCD's item
// k. After that, in a level whose items all have the same chunk count, it takes
// items k + G, k + 2 G, ... (G workgroups per XCD); in any other level it claims
// its next item from the XCD's counter, only shortly before it needs it: the
// level lists segments longest first, so long and short items balance like a
// longest-first list schedule, and claims are spread out in time (contended
// claims on one counter are slow). A claim takes two feed calls to become
// usable (the index arrives, then the unit record it names), so the next item
// is claimed when one chunk of the current item is left to feed, and the one
// after it as well when the current item is short (items of one or two chunks
// then follow each other without a stall). Only the first of the two waiting
// items has its unit record requested, which keeps one record and one index in
// flight.

struct Feed {
  int start, len, ms, slot;  // unit record of the current item: first token, length, mode | sequence << 1, fork slot
  int h, tile, nch, c;       // its head, d_v tile, chunks, chunks fed so far
  int u0, tile0;             // unit and d_v tile of the first waiting item once its index is known
  int nst;                   // items taken so far in the fixed stride
  int fl;                    // kFeedDone | kFeedDyn | stage of the first waiting item | kFeedWait1
};
// Stages of the first waiting item (bits 0-1 of fl): none, index in flight,
// index known and unit record requested.
constexpr int kFeedIdx = 1, kFeedRec = 2, kFeedStage = 3;
constexpr int kFeedWait1 = 4;  // a second item is waiting (its index in flight)
constexpr int kFeedDyn = 8;    // items are claimed from the counter (else taken in a fixed stride)
constexpr int kFeedDone = 16;  // the level has no item left for this workgroup

struct FeedRegs {
  int raw0, raw1;  // indices of the waiting items in lane 0 (a claim is in flight until the next vmcnt(0))
  int4 info0;      // unit record of the first waiting item (likewise)
};

// Index of the workgroup's next item after its first.
__device__ __forceinline__ int feed_claim(Feed& f, const Args& a, int xcd, int lane) {
  const int G = (int)(gridDim.x / kXcd);
  if (!(f.fl & kFeedDyn)) return (int)(blockIdx.x / kXcd) + G * ++f.nst;
  int v = 0;
  if (lane == 0) v = atomicAdd(a.walk_ctr + a.level * kSchedInts + xcd, 1) + G;
  return v;
}

// First waiting item, index -> record: reads its index and requests its unit
// record. Unit indices stay below count * H <= T * H < 2^31 (checked on the
// host); a unit past the level's last one ends the level.
__device__ __forceinline__ void feed_advance(Feed& f, FeedRegs& r, const Args& a, int xcd, int count, int base) {
  if ((f.fl & kFeedStage) != kFeedIdx) return;
  const unsigned idx = (unsigned)rfl(r.raw0);
  const unsigned q = idx / (unsigned)a.NT;
  const unsigned u = (unsigned)xcd + (unsigned)kXcd * q;
  f.u0 = (int)u;
  f.tile0 = (int)(idx - q * (unsigned)a.NT);
  r.info0 = make_int4(0, 0, 0, -1);
  if (u < (unsigned)count * (unsigned)a.H) r.info0 = a.unit_info[base + (int)(u / (unsigned)a.H)];
  f.fl += kFeedRec - kFeedIdx;
}

// The workgroup's first item waits with its index known (its rank among the
// XCD's workgroups).
__device__ __forceinline__ void feed_init(Feed& f, FeedRegs& r, const Args& a) {
  f = Feed{};
  const int* sc = a.walk_ctr + a.level * kSchedInts + kWalkQueues;
  f.fl = kFeedIdx | (sc[0] != sc[1] ? kFeedDyn : 0);
  r.raw0 = (int)(blockIdx.x / kXcd);
  r.raw1 = 0;
  r.info0 = make_int4(0, 0, 0, -1);
}

// The descriptor of the next chunk to load (valid = 0 when the level is done).
// Called once per helper iteration, after its vmcnt(0), so that what the
// previous call requested has arrived.
template <int BV>
__device__ __forceinline__ Desc feed_next(Feed& f, FeedRegs& r, const Args& a, int xcd, int count, int base,
                                          int lane) {
  Desc d = {};  // every field defined, also when the level is done
  if (f.fl & kFeedDone) return d;
  const bool sw = f.c >= f.nch;  // the current item is over (or none has started)
  if (sw && !(f.fl & kFeedStage)) {  // nothing waiting: claim now (the advance below waits for it)
    r.raw0 = feed_claim(f, a, xcd, lane);
    f.fl |= kFeedIdx;
  }
  feed_advance(f, r, a, xcd, count, base);
  if (sw) {
    const unsigned u = (unsigned)f.u0;
    if (u >= (unsigned)count * (unsigned)a.H) {  // claims run past the level's items
      f.fl |= kFeedDone;
      return d;
    }
    f.start = rfl(r.info0.x);
    f.len = rfl(r.info0.y);
    f.ms = rfl(r.info0.z);
    f.slot = rfl(r.info0.w);
    f.h = (int)(u % (unsigned)a.H);
    f.tile = f.tile0;
    f.nch = (f.ms & 1) ? 1 : (f.len + kChunk - 1) / kChunk;
    f.c = 0;
    // the second waiting item moves up; its claim was made in an earlier call
    f.fl = (f.fl & ~(kFeedStage | kFeedWait1)) | ((f.fl & kFeedWait1) ? kFeedIdx : 0);
    r.raw0 = r.raw1;
    feed_advance(f, r, a, xcd, count, base);
  }
  const size_t SS = (size_t)a.Dv * DK;
  const int mode = f.ms & 1, sq = f.ms >> 1;
  d.valid = 1;
  d.t0 = f.start + f.c * kChunk;
  d.n = min(kChunk, f.len - f.c * kChunk);
  d.h = f.h;
  d.v0 = f.tile * BV;
  d.mode = mode;
  d.sq = sq;
  d.first = f.c == 0;
  d.need_exit = (!mode) && (f.c + 1 < f.nch);
  d.has_out = 0;
  d.req_lo = d.req_hi = 0;
  d.sin = nullptr;
  if (d.first) {
    const float* s = f.slot >= 0 ? a.fork_states + ((size_t)f.slot * a.H + f.h) * SS
                                 : (a.init ? a.init + ((size_t)sq * a.H + f.h) * SS : nullptr);
    d.sin = s ? s + (size_t)d.v0 * DK : nullptr;
  }
  f.c += 1;
  const int rem = f.nch - f.c;
  const int need = rem == 0 ? (f.nch <= 2 ? 2 : 1) : (rem == 1 ? 1 : 0);
  if (need >= 1 && !(f.fl & kFeedStage)) {
    r.raw0 = feed_claim(f, a, xcd, lane);
    f.fl |= kFeedIdx;
  }
  if (need >= 2 && !(f.fl & kFeedWait1)) {
    r.raw1 = feed_claim(f, a, xcd, lane);
    f.fl |= kFeedWait1;
  }
  return d;
}

// The fields of a descriptor the state waves use, wave-uniform.
struct SDesc {
  int valid, t0, n, h, v0, mode, has_out, need_exit, first;
  unsigned req_lo, req_hi;
};

__device__ __forceinline__ SDesc load_sdesc(const unsigned char* p) {
  const Desc* dp = reinterpret_cast<const Desc*>(p);
  SDesc d;
  d.valid = rfl(dp->valid);
  d.t0 = rfl(dp->t0);
  d.n = rfl(dp->n);
  d.h = rfl(dp->h);
  d.v0 = rfl(dp->v0);
  d.mode = rfl(dp->mode);
  d.has_out = rfl(dp->has_out);
  d.need_exit = rfl(dp->need_exit);
  d.first = rfl(dp->first);
  d.req_lo = (unsigned)rfl((int)dp->req_lo);
  d.req_hi = (unsigned)rfl((int)dp->req_hi);
  return d;
}

// A descriptor read from LDS, with every field made wave-uniform.
__device__ __forceinline__ Desc uniform_desc(const Desc& s) {
  Desc d;
  d.valid = rfl(s.valid);
  d.t0 = rfl(s.t0);
  d.n = rfl(s.n);
  d.h = rfl(s.h);
  d.v0 = rfl(s.v0);
  d.mode = rfl(s.mode);
  d.sq = rfl(s.sq);
  d.first = rfl(s.first);
  d.need_exit = rfl(s.need_exit);
  d.has_out = rfl(s.has_out);
  d.req_lo = (unsigned)rfl((int)s.req_lo);
  d.req_hi = (unsigned)rfl((int)s.req_hi);
  const unsigned long long p = (unsigned long long)s.sin;
  d.sin = (const float*)(((unsigned long long)(unsigned)rfl((int)(p >> 32)) << 32) | (unsigned)rfl((int)p));
  return d;
}

__device__ __forceinline__ void put_desc(unsigned char* p, const Desc& d, int lane) {
  if (lane == 0) *reinterpret_cast<Desc*>(p) = d;
}

// ------------------------------------------------------------ chunk loads

// Direct-to-LDS copies of 4-row blocks [b0, b1) of the K (or Q) rows of
// chunk d into the tile at tile (LDS). Lane (g4, l16) copies row
// 4 blk + g4, 16-byte piece l16 ^ kq_swz(row), into slot l16 of that row. Rows
// at or beyond d.n are zero-filled. The global address advances from the
// block's first row, so no per-block pointer outlives an iteration.
template <int B0, int B1>
__device__ __forceinline__ void issue_rows(const Args& a, const Desc& d, const __bf16* x, unsigned char* tile, int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
  const unsigned rs = (unsigned)a.H * (DK * 2);  // bytes per token row
  const unsigned char* src = reinterpret_cast<const unsigned char*>(x) + ((size_t)d.t0 * a.H + d.h) * (DK * 2) +
                             (size_t)(4 * B0) * rs;
  unsigned vo[4];  // the piece permutation depends on blk & 3
#pragma unroll
  for (int k = 0; k < 4; ++k) vo[k] = g4 * rs + (unsigned)((l16 ^ ((g4 << 2) | k)) << 4);
  const size_t step = (size_t)4 * rs;
  if (d.n == kChunk) {
    const uint32_t l0 = lds_addr_of(tile);
#pragma unroll
    for (int blk = B0; blk < B1; ++blk) {
      dma16(src, vo[blk & 3], l0 + blk * 1024);
      src += step;
    }
  } else {
#pragma unroll
    for (int blk = B0; blk < B1; ++blk) {
      if (4 * blk + g4 < d.n) dma16(src, vo[blk & 3], lds_addr_of(tile + blk * 1024));
      else *reinterpret_cast<uint4*>(tile + blk * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
      src += step;
    }
  }
}

// The V tile of chunk d into vb: pieces of RPI rows each; lane takes row
// ins * RPI + lane / VPR, slot lane % VPR.
template <int BV>
__device__ __forceinline__ void issue_v(const Args& a, const Desc& d, unsigned char* vb, int lane) {
  using C = Cfg<BV>;
  const int vr = lane / C::VPR, vs = lane % C::VPR;
  const unsigned rs = (unsigned)a.H * (unsigned)(a.Dv * 2);
  const unsigned vo = vr * rs + (unsigned)((vs ^ v_swz<BV>(vr)) * 16);
  const unsigned char* src = reinterpret_cast<const unsigned char*>(a.v) + ((size_t)d.t0 * a.H + d.h) * (size_t)(a.Dv * 2) +
                             (size_t)d.v0 * 2;
  const size_t step = (size_t)C::RPI * rs;
#pragma unroll
  for (int ins = 0; ins < C::VPR; ++ins) {
    const int row = ins * C::RPI + vr;
    if (d.n == kChunk || row < d.n) dma16(src, vo, lds_addr_of(vb + ins * 1024));
    else *reinterpret_cast<uint4*>(vb + ins * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
    src += step;
  }
}

// The entry state rows of the next chunk's d_v tile (BV rows of d_k fp32,
// contiguous, BV * 512 bytes) are pulled into L2 while the current chunk runs,
// so that the state waves' own loads of those rows hit L2: each lane loads one
// word of a different 128-byte line, the two helpers taking alternate halves
// (one or two loads per helper instead of BV / 4 direct-to-LDS copies). The
// words are consumed only after the helper's own wait for its copies, so the
// loads never hold the wave up.
struct Touch {
  unsigned w0, w1;
};
typedef __attribute__((address_space(1))) const unsigned gu32;
template <int BV>
__device__ __forceinline__ Touch prefetch_entry(const float* sin, int hid, int lane) {
  constexpr int kPer = BV * 2;  // lines per helper: BV rows x 4 lines / 2
  Touch t = {0u, 0u};
  if (lane < kPer) t.w0 = *(gu32*)(sin + (size_t)(hid * kPer + lane) * 32);
  if (kPer > 64 && lane + 64 < kPer) t.w1 = *(gu32*)(sin + (size_t)(hid * kPer + 64 + lane) * 32);
  return t;
}
__device__ __forceinline__ void consume(const Touch& t) { asm volatile("" ::"v"(t.w0), "v"(t.w1)); }

// Helper 0 copies K (tiles of 64 columns) and the first kQSplit blocks of 4 rows
// of Q, helper 1 the rest of Q (helper 0 also inverts the diagonal blocks and
// feeds the items, so it takes fewer copies). Measured on the chain walk while
// helper 0 also copied K there: 2 blocks 2% faster than 4, 0, 6 or 8.
constexpr int kQSplit = 2;
// With tiles of 16 or 32 columns the helpers set the pace of a chunk while the
// state waves wait at the barrier, so there the state waves copy the K rows of
// the chunk two ahead themselves (state_loop, from chunk 2 on) and helper 0
// copies only its Q rows.
template <int BV>
constexpr bool kStateCopiesK = Cfg<BV>::NB == 1;
template <bool WITH_K = true>
__device__ __forceinline__ void issue_kq(const Args& a, const Desc& d, unsigned char* kq, int hid, int lane) {
  if (hid == 0) {
    if (WITH_K) issue_rows<0, 16>(a, d, a.k, kq, lane);
    issue_rows<0, kQSplit>(a, d, a.q, kq + 16384, lane);
  } else {
    issue_rows<kQSplit, 16>(a, d, a.q, kq + 16384, lane);
  }
}

// Raw per-token values of a chunk (one token per lane), converted only after
// the wait that follows the copies so that no compiler wait lands among them.
struct TokenRegs {
  unsigned short g, b;  // bf16 bits
  int par, om, sm, fs;
  unsigned long long tm;  // ancestor-or-self mask of the token in a tree chunk
};

__device__ __forceinline__ TokenRegs load_tokens(const Args& a, const Desc& d, int lane) {
  TokenRegs r;
  r.g = 0;
  r.b = 0;
  r.par = -1;
  r.om = kUnmapped;
  r.sm = kUnmapped;
  r.fs = -1;
  r.tm = 0;
  // the mask rows of a tree chunk are loaded here, with the other token values,
  // so that their latency hides behind the chunk's products
  if (d.valid && d.mode) r.tm = a.tree_mask[(size_t)d.sq * kChunk + lane];
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

// Inclusive prefix sum over the 64 lanes of a wave: shifts within rows of 16
// lanes, then the last lane of a row added to the rows after it.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_prefix_sum(float x) {
  x = dpp_add<0x111, 0xf>(x);  // row_shr:1
  x = dpp_add<0x112, 0xf>(x);  // row_shr:2
  x = dpp_add<0x114, 0xf>(x);  // row_shr:4
  x = dpp_add<0x118, 0xf>(x);  // row_shr:8
  x = dpp_add<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x = dpp_add<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

// Token tables of chunk d into tb (second helper).
__device__ __forceinline__ void store_tokens(const Args& a, Desc d, const TokenRegs& r, unsigned char* tb, int lane) {
  if (!d.valid) {
    put_desc(tb + tD, d, lane);
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
    mask = r.tm;
  } else {
    G = wave_prefix_sum(G);
    mask = (i == 63) ? ~0ull : ((2ull << i) - 1ull);
  }
  const float g2 = G * kLog2e;
  const float g2last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g2), d.n - 1));
  const int orow = (valid && r.om != kUnmapped) ? r.om : -1;
  const int fs = valid ? r.fs : -1;
  const int sr = (valid && r.sm != kUnmapped) ? r.sm : -1;
  reinterpret_cast<float*>(tb + tG2)[i] = g2;
  reinterpret_cast<float*>(tb + tEG)[i] = __expf(G);
  reinterpret_cast<float*>(tb + tB)[i] = bf_up(r.b);
  reinterpret_cast<float*>(tb + tDX)[i] = valid ? __builtin_amdgcn_exp2f(g2last - g2) : 0.f;
  reinterpret_cast<unsigned*>(tb + tMl)[i] = (unsigned)mask;
  reinterpret_cast<unsigned*>(tb + tMh)[i] = (unsigned)(mask >> 32);
  reinterpret_cast<int*>(tb + tOR)[i] = orow;
  reinterpret_cast<int*>(tb + tFS)[i] = fs;
  reinterpret_cast<int*>(tb + tSR)[i] = sr;
  const unsigned long long rq = __ballot(fs >= 0 || sr >= 0);
  d.has_out = __ballot(orow >= 0) != 0ull;
  d.req_lo = (unsigned)rq;
  d.req_hi = (unsigned)(rq >> 32);
  put_desc(tb + tD, d, lane);
}

// ---------------------------------------------------------------- helpers

// The S-independent operands of one chunk. The Gram and Q K^T tiles are
// computed with K of the column block as the A operand, so that the
// accumulator of tile (row block b, column block m) holds row 16 b + l16,
// columns 16 m + 4 g4 .. + 3: exactly the A-operand layout the state waves
// read. Helper 0 (DIAG) takes the four diagonal tiles and inverts the
// diagonal blocks of I + A; helper 1 takes the six tiles below them.
template <bool DIAG, bool HAS_OUT>
__device__ __forceinline__ void products(const unsigned char* kq, const unsigned char* tb, unsigned char* pr,
                                         unsigned char* pp, float* lt, bool tree, int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
  int oF[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) oF[ks] = l16 * 256 + (((4 * ks + g4) ^ kq_swz(l16)) << 4);
  bf16x8 KF[4][4], QF[4][4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) KF[b][ks] = lds_at<bf16x8>(kq + oF[ks], b * 4096);
  if (HAS_OUT) {
#pragma unroll
    for (int rb = DIAG ? 0 : 1; rb < 4; ++rb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) QF[rb][ks] = lds_at<bf16x8>(kq + 16384 + oF[ks], rb * 4096);
  }
  const float* G2 = reinterpret_cast<const float*>(tb + tG2);
  const float* Bt = reinterpret_cast<const float*>(tb + tB);
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int rb = DIAG ? 0 : 1; rb < 4; ++rb) {
    const int i = 16 * rb + l16;
    const float g2i = G2[i], bi = Bt[i];
    const unsigned mw0 = reinterpret_cast<const unsigned*>(tb + tMl)[i];
    const unsigned mw1 = reinterpret_cast<const unsigned*>(tb + tMh)[i];
#pragma unroll
    for (int cb = 0; cb <= rb; ++cb) {
      if (DIAG != (cb == rb)) continue;
      f32x4 ga = zero, gp = zero;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) ga = mma32(KF[cb][ks], KF[rb][ks], ga);
      if (HAS_OUT) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) gp = mma32(KF[cb][ks], QF[rb][ks], gp);
      }
      const float4 gj4 = *reinterpret_cast<const float4*>(G2 + 16 * cb + 4 * g4);
      const float gj[4] = {gj4.x, gj4.y, gj4.z, gj4.w};
      // decay exp(G_i - G_j) where token j is an ancestor-or-self of token i, else 0
      float e[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int jl = 4 * g4 + r;  // j = 16 cb + jl
        const bool in_tree = ((cb >= 2 ? mw1 : mw0) >> ((16 * cb + jl) & 31)) & 1u;
        const bool anc = tree ? in_tree : (cb < rb || jl <= l16);
        e[r] = anc ? __builtin_amdgcn_exp2f(g2i - gj[r]) : 0.f;
      }
      if (!DIAG) {
        bf16x4 na;
#pragma unroll
        for (int r = 0; r < 4; ++r) na[r] = (__bf16)(-(bi * e[r] * ga[r]));
        *reinterpret_cast<bf16x4*>(pr + pNA + ((rb * (rb - 1)) / 2 + cb) * 512 + lane * 8) = na;
      } else {
        // strict lower part of the diagonal block, transposed: lt[rb][j][i]
#pragma unroll
        for (int r = 0; r < 4; ++r)
          lt[rb * kLTS + (4 * g4 + r) * kLTR + l16] = (4 * g4 + r != l16) ? bi * e[r] * ga[r] : 0.f;
      }
      if (HAS_OUT) {
        bf16x4 pv;
#pragma unroll
        for (int r = 0; r < 4; ++r) pv[r] = (__bf16)(e[r] * gp[r]);
        const int pair = (rb <= 1 ? rb : 2 * rb - 2) + (cb >> 1);
        *reinterpret_cast<bf16x4*>(pp + pair * 1024 + lane * 16 + (cb & 1) * 8) = pv;
      }
    }
  }
  if (!DIAG) return;
  wait_lds();
  // Row c = l16 of (I + L)^{-1} for the diagonal block g4, by back substitution
  // on the transposed system (I + L)^T z = e_c, in fp32. The block's entries are
  // read first; each sum runs from the far end so that only its last term waits
  // for the entry just solved.
  const float* L = lt + g4 * kLTS;  // L[r * kLTR + c'] = A[c'][r] of the block
  float Lr[16][16];
#pragma unroll
  for (int r = 0; r < 15; ++r)
#pragma unroll
    for (int q = (r + 1) / 4; q < 4; ++q) {
      const float4 v = *reinterpret_cast<const float4*>(L + r * kLTR + 4 * q);
      Lr[r][4 * q] = v.x;
      Lr[r][4 * q + 1] = v.y;
      Lr[r][4 * q + 2] = v.z;
      Lr[r][4 * q + 3] = v.w;
    }
  float z[16];
#pragma unroll
  for (int r = 15; r >= 0; --r) {
    float acc = (r == l16) ? 1.f : 0.f;
#pragma unroll
    for (int c = 15; c > r; --c) acc -= Lr[r][c] * z[c];
    z[r] = acc;
  }
  unsigned char* d = pr + pDI + g4 * kDIS;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    bf16x4 v;
#pragma unroll
    for (int y = 0; y < 4; ++y) v[y] = (__bf16)z[4 * q + y];
    *reinterpret_cast<bf16x4*>(d + (q * 16 + l16) * 8) = v;
  }
}

__device__ __forceinline__ void chunk_products(int hid, const Desc& c, const unsigned char* kq, const unsigned char* tb,
                                               unsigned char* pr, unsigned char* pp, float* lt, int lane) {
  const bool tree = c.mode != 0;
  if (hid == 0) {
    if (c.has_out) products<true, true>(kq, tb, pr, pp, lt, tree, lane);
    else products<true, false>(kq, tb, pr, pp, lt, tree, lane);
  } else {
    if (c.has_out) products<false, true>(kq, tb, pr, pp, lt, tree, lane);
    else products<false, false>(kq, tb, pr, pp, lt, tree, lane);
  }
}

template <int BV>
__device__ __forceinline__ void helper_loop(const Args& a, unsigned char* smem, int hid, int lane, Feed& ff, FeedRegs& fr, int xcd,
                                            int count, int base) {
  using C = Cfg<BV>;
  Desc* nds = reinterpret_cast<Desc*>(smem + C::oND);
  float* lt = reinterpret_cast<float*>(smem + C::oLT);
  TokenRegs tr;
  // Iteration -1 forms the products of chunk 0 while the state waves wait.
  for (int it = -1;; ++it) {
    if (it >= 0 && !rfl(reinterpret_cast<const Desc*>(smem + C::oTB + (it % 3) * kTB + tD)->valid)) break;
    WALK_STAMP(it + 1, 0);
    const int s1 = (it + 1) % 3, s2 = (it + 2) % 3;
    unsigned char* tb1 = smem + C::oTB + s1 * kTB;
    const Desc nd = uniform_desc(nds[it & 1]);                              // chunk it + 2: K, Q, tables
    const Desc nx = uniform_desc(*reinterpret_cast<const Desc*>(tb1 + tD));  // chunk it + 1: V, products
    if (hid == 1) tr = load_tokens(a, nd, lane);
    // (the state waves copy K rows from their first chunk on, for chunk 2; chunk
    // 1's are copied here, in iteration -1)
    if (nd.valid) {
      if constexpr (kStateCopiesK<BV>) {
        if (it < 0) issue_kq<true>(a, nd, smem + C::oKQ + s2 * 32768, hid, lane);
        else issue_kq<false>(a, nd, smem + C::oKQ + s2 * 32768, hid, lane);
      } else {
        issue_kq(a, nd, smem + C::oKQ + s2 * 32768, hid, lane);
      }
    }
    if (hid == 1 && nx.valid) issue_v<BV>(a, nx, smem + C::oV + ((it + 1) & 1) * C::VT, lane);
    Touch touch = {0u, 0u};
    if (nx.valid && nx.first && nx.sin) touch = prefetch_entry<BV>(nx.sin, hid, lane);
    WALK_STAMP(it + 1, 1);
    if (nx.valid)
      chunk_products(hid, nx, smem + C::oKQ + s1 * 32768, tb1, smem + C::oPR + ((it + 1) & 1) * kPR,
                     smem + C::oPP + s1 * kPP, lt, lane);
    WALK_STAMP(it + 1, 2);
    wait_vm();  // this wave's copies, token values and unit record have landed
    consume(touch);
    WALK_STAMP(it + 1, 3);
    if (hid == 1) store_tokens(a, nd, tr, smem + C::oTB + s2 * kTB, lane);
    if (hid == 0) {
      Desc nn = {};
      if (nd.valid) nn = feed_next<BV>(ff, fr, a, xcd, count, base, lane);
      put_desc(reinterpret_cast<unsigned char*>(nds + ((it + 1) & 1)), nn, lane);
    }
    WALK_STAMP(it + 1, 4);
    lds_barrier();
  }
}

// ------------------------------------------------------------ state waves

// Per-lane LDS offsets of a state wave.
template <int NB>
struct SOff {
  int F[4];    // row fragment of K or Q rows 0..15, 16 B per lane (row block rb adds 4096 rb)
  int KT[8];   // transposed read of K rows 4 g4 + l16/4 for state block dt (rows + 16 add 4096)
  int V[NB];   // transposed read of V rows 4 g4 + l16/4, column block nb (row block rb adds 32 BV rb)
};

// dst = cS src + (K^T rows of the state block) x (decayed pseudo-values w) for
// every 16-column block and d_k tile; dst may be src (each tile depends only on
// its own tile of src).
template <int NB, bool SCALE = true>
__device__ __forceinline__ void state_at(f32x4 (&dst)[NB][8], const f32x4 (&src)[NB][8], float cS, const unsigned char* kq,
                                         const SOff<NB>& o, const bf16x8 (&w01)[NB], const bf16x8 (&w23)[NB]) {
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    // A operand: K^T rows (d_k) of this state block against tokens 0..31 and 32..63
    const unsigned char* kp = kq + o.KT[dt];
    const bf16x8 k01 = cat8(tr_read(kp), tr_read(kp + 4096));
    const bf16x8 k23 = cat8(tr_read(kp + 8192), tr_read(kp + 8192 + 4096));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      f32x4 t;
#pragma unroll
      for (int r = 0; r < 4; ++r) t[r] = SCALE ? cS * src[nb][dt][r] : src[nb][dt][r];
      t = mma32(k01, w01[nb], t);
      dst[nb][dt] = mma32(k23, w23[nb], t);
    }
  }
}

// A state after a requested token to its fork slot and/or state row.
template <int NB>
__device__ __forceinline__ void store_state(const Args& a, const f32x4 (&S)[NB][8], int fs, int sr, int h, int v0w,
                                            int lane) {
  const int g4 = lane >> 4, l16 = lane & 15;
  const size_t SS = (size_t)a.Dv * DK;
  const size_t roff = (size_t)(v0w + l16) * DK + 8 * g4;
  if (fs >= 0) {
    float* dst = a.fork_states + ((size_t)fs * a.H + h) * SS + roff;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<f32x4*>(dst + 16 * nb * DK + 32 * (dt >> 1) + 4 * (dt & 1)) = S[nb][dt];
  }
  if (sr >= 0) {
    float* dst = a.state_out + ((size_t)sr * a.H + h) * SS + roff;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<f32x4*>(dst + 16 * nb * DK + 32 * (dt >> 1) + 4 * (dt & 1)) = S[nb][dt];
  }
}

// Boundary between two stages of a state wave's chunk. For waves of one
// 16-column block a scheduling barrier keeps the compiler from hoisting every
// stage's LDS reads to the top of the chunk (values then went out to AGPRs and
// back; 1-3% slower without it); waves of two blocks schedule better without
// it under the ILP schedule (mixed forest 2.3% faster).
template <int NB>
__device__ __forceinline__ void stage_fence() {
  if constexpr (NB == 1) __builtin_amdgcn_sched_barrier(0);
}

// One chunk on a state wave: K S_e^T, R, the block substitution, the outputs
// and pseudo-values, then the states after requested tokens and at the exit.
// The wave owns NB blocks of 16 columns. ST[nb][dt] (dt = 2 m + bb) holds S^T
// of block nb in the accumulator layout, lane (l16, g4) holding
// S[col][32 m + 8 g4 + 4 bb + r]; Sb[nb][m] is its bf16 B operand (and, as the
// same registers, the A operand of S_e Q^T) for d_k 32 m .. 32 m + 31.
template <int BV, bool HAS_OUT>
__device__ __forceinline__ void state_chunk(const Args& a, const unsigned char* smem, const unsigned char* tb,
                                            const unsigned char* kq, const unsigned char* vt, const unsigned char* pr,
                                            const SOff<Cfg<BV>::NB>& o, f32x4 (&ST)[Cfg<BV>::NB][8],
                                            bf16x8 (&Sb)[Cfg<BV>::NB][4], int it, int t0, int n, int h, int v0w, int mode,
                                            bool need_exit, unsigned long long todo, int lane) {
  constexpr int NB = Cfg<BV>::NB;
  const int g4 = lane >> 4, l16 = lane & 15;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const unsigned HDv = (unsigned)a.H * a.Dv;
  const float* sEG = reinterpret_cast<const float*>(tb + tEG);
  const float* sB = reinterpret_cast<const float*>(tb + tB);

  // K S_e^T for the wave's columns
  f32x4 X[NB][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    bf16x8 KF[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) KF[m] = lds_at<bf16x8>(kq + o.F[m], rb * 4096);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      X[nb][rb] = zero;
#pragma unroll
      for (int m = 0; m < 4; ++m) X[nb][rb] = mma32(KF[m], Sb[nb][m], X[nb][rb]);
    }
  }
  // When the chunk exit is the only state asked for, S is scaled by the exit's
  // decay e^{G_{n-1}} here, next to the matrix products, instead of inside the
  // exit update at the end of the chunk's dependency chain (S itself is not
  // read again before the exit: K S^T and S Q^T use its bf16 copy). Only for
  // waves of one 16-column block: with two, the extra path cost scalar-register
  // spills and made the 64-column walk slower.
  bool prescale = false;
  if constexpr (NB == 1) prescale = need_exit && todo == (1ull << (n - 1));
  if (prescale) {
    const float cs = sEG[n - 1];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) ST[nb][dt][r] *= cs;
  }
  stage_fence<NB>();
  WALK_STAMP(it, 1);
  // e^G S_e Q^T (the output, transposed): lane holds four columns of one token
  f32x4 O[NB][4];
  if (HAS_OUT) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      bf16x8 QF[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) QF[m] = lds_at<bf16x8>(kq + 16384 + o.F[m], rb * 4096);
      const float egt = sEG[16 * rb + l16];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        O[nb][rb] = zero;
#pragma unroll
        for (int m = 0; m < 4; ++m) O[nb][rb] = mma32(Sb[nb][m], QF[m], O[nb][rb]);
#pragma unroll
        for (int r = 0; r < 4; ++r) O[nb][rb][r] *= egt;
      }
    }
  }
  stage_fence<NB>();
  WALK_STAMP(it, 2);
  // R = beta (V - e^G K S^T) in place of X
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const float4 eg = *reinterpret_cast<const float4*>(sEG + 16 * rb + 4 * g4);
    const float4 bi = *reinterpret_cast<const float4*>(sB + 16 * rb + 4 * g4);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bf16x4 vb = __builtin_bit_cast(bf16x4, tr_read(vt + o.V[nb] + rb * 32 * BV));
      X[nb][rb][0] = bi.x * ((float)vb[0] - eg.x * X[nb][rb][0]);
      X[nb][rb][1] = bi.y * ((float)vb[1] - eg.y * X[nb][rb][1]);
      X[nb][rb][2] = bi.z * ((float)vb[2] - eg.z * X[nb][rb][2]);
      X[nb][rb][3] = bi.w * ((float)vb[3] - eg.w * X[nb][rb][3]);
    }
  }
  stage_fence<NB>();
  WALK_STAMP(it, 3);
  // block substitution with the helpers' -A_bm and (I + A_bb)^{-1}
  bf16x4 nA[6], DI[4];
#pragma unroll
  for (int k = 0; k < 6; ++k) nA[k] = lds_at<bf16x4>(pr + pNA + k * 512, lane * 8);
#pragma unroll
  for (int b = 0; b < 4; ++b) DI[b] = lds_at<bf16x4>(pr + pDI + b * kDIS, lane * 8);
  f32x4 Vt[NB][4];
  bf16x4 Vb[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    Vt[nb][0] = mma16(DI[0], to_bf4(X[nb][0]), zero);
    Vb[nb][0] = to_bf4(Vt[nb][0]);
    f32x4 y = mma16(nA[0], Vb[nb][0], X[nb][1]);
    Vt[nb][1] = mma16(DI[1], to_bf4(y), zero);
    Vb[nb][1] = to_bf4(Vt[nb][1]);
    y = mma16(nA[1], Vb[nb][0], X[nb][2]);
    y = mma16(nA[2], Vb[nb][1], y);
    Vt[nb][2] = mma16(DI[2], to_bf4(y), zero);
    Vb[nb][2] = to_bf4(Vt[nb][2]);
    y = mma16(nA[3], Vb[nb][0], X[nb][3]);
    y = mma16(nA[4], Vb[nb][1], y);
    y = mma16(nA[5], Vb[nb][2], y);
    Vt[nb][3] = mma16(DI[3], to_bf4(y), zero);
    Vb[nb][3] = to_bf4(Vt[nb][3]);
  }
  stage_fence<NB>();
  WALK_STAMP(it, 4);
  if (HAS_OUT) {
    // O^T += Vt^T P^T over pairs of 16-token blocks (blocks of P above the
    // diagonal are zero; the helpers' P fragments are the B operands)
    const unsigned char* pp = smem + Cfg<BV>::oPP + (it % 3) * kPP;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
      for (int mp = 0; mp < 2; ++mp) {
        if (2 * mp > rb) continue;
        const int pair = (rb <= 1 ? rb : 2 * rb - 2) + mp;
        const bf16x8 pb = lds_at<bf16x8>(pp + pair * 1024, lane * 16);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) O[nb][rb] = mma32(cat8b(Vb[nb][2 * mp], Vb[nb][2 * mp + 1]), pb, O[nb][rb]);
      }
    }
    // lane (l16, g4) holds columns 4 g4 .. 4 g4 + 3 of block nb for token 16 rb + l16.
    // Row offsets are 64-bit at the chunk (or row) base and 32-bit inside a chunk.
    const unsigned ccol = (unsigned)h * a.Dv + (unsigned)(v0w + 4 * g4);
    if (a.out_all && n == kChunk) {  // every token of a full chunk is an output row, in stream order
      __bf16* oc = a.out + (size_t)t0 * HDv;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          *reinterpret_cast<bf16x4*>(oc + (unsigned)(16 * rb + l16) * HDv + ccol + 16 * nb) = to_bf4(O[nb][rb]);
    } else {
      const int* sOR = reinterpret_cast<const int*>(tb + tOR);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int orow = sOR[16 * rb + l16];
        if (orow >= 0) {
          __bf16* orp = a.out + (size_t)orow * HDv + ccol;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) *reinterpret_cast<bf16x4*>(orp + 16 * nb) = to_bf4(O[nb][rb]);
        }
      }
    }
  }
  stage_fence<NB>();
  WALK_STAMP(it, 5);
  if (a.pv) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float* pvb = a.pv + (size_t)t0 * HDv + (unsigned)(4 * g4) * HDv + (unsigned)h * a.Dv + (unsigned)(v0w + 16 * nb + l16);
      if (n == kChunk) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
          for (int r = 0; r < 4; ++r) pvb[(16 * rb + r) * HDv] = Vt[nb][rb][r];
      } else {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * rb + 4 * g4 + r < n) pvb[(16 * rb + r) * HDv] = Vt[nb][rb][r];
      }
    }
  }
  stage_fence<NB>();
  WALK_STAMP(it, 6);
  // states after requested tokens (fork slots, state rows) and at the chunk exit
  if (!todo) return;
  const float* sG2 = reinterpret_cast<const float*>(tb + tG2);
  do {
    const int p = __builtin_ctzll(todo);
    todo &= todo - 1ull;
    // masked, decayed pseudo-values exp(G_p - G_j) vt_j for j ancestor-or-self of p
    // (zero past p, so the product over tokens 32..63 adds nothing when p < 32);
    // on a chain the last token takes the exit decay table (zero past n)
    float dec[4][4];
    if (!mode && p == n - 1) {
      const float* sDX = reinterpret_cast<const float*>(tb + tDX);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const float4 dx = *reinterpret_cast<const float4*>(sDX + 16 * mb + 4 * g4);
        dec[mb][0] = dx.x;
        dec[mb][1] = dx.y;
        dec[mb][2] = dx.z;
        dec[mb][3] = dx.w;
      }
    } else {
      const unsigned mlo = reinterpret_cast<const unsigned*>(tb + tMl)[p];
      const unsigned mhi = reinterpret_cast<const unsigned*>(tb + tMh)[p];
      const float g2p = sG2[p];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const float4 g2 = *reinterpret_cast<const float4*>(sG2 + 16 * mb + 4 * g4);
        const float gj[4] = {g2.x, g2.y, g2.z, g2.w};
        const unsigned mword = mb >= 2 ? mhi : mlo;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * mb + 4 * g4 + r;
          const bool anc = mode ? ((mword >> (j & 31)) & 1u) : (j <= p);
          dec[mb][r] = anc ? __builtin_amdgcn_exp2f(g2p - gj[r]) : 0.f;
        }
      }
    }
    bf16x8 w01[NB], w23[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      bf16x4 Wb[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        f32x4 wv;
#pragma unroll
        for (int r = 0; r < 4; ++r) wv[r] = Vt[nb][mb][r] * dec[mb][r];
        Wb[mb] = to_bf4(wv);
      }
      w01[nb] = cat8b(Wb[0], Wb[1]);
      w23[nb] = cat8b(Wb[2], Wb[3]);
    }
    const float cS = sEG[p];
    const int fs = reinterpret_cast<const int*>(tb + tFS)[p];
    const int sr = reinterpret_cast<const int*>(tb + tSR)[p];
    if (need_exit && p == n - 1) {
      // the chunk exit (always the last requested token): S is updated in place
      if constexpr (NB == 1) {
        if (prescale) state_at<NB, false>(ST, ST, cS, kq, o, w01, w23);
        else state_at<NB>(ST, ST, cS, kq, o, w01, w23);
      } else {
        state_at<NB>(ST, ST, cS, kq, o, w01, w23);
      }
      store_state<NB>(a, ST, fs, sr, h, v0w, lane);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int m = 0; m < 4; ++m) Sb[nb][m] = cat8b(to_bf4(ST[nb][2 * m]), to_bf4(ST[nb][2 * m + 1]));
    } else {
      f32x4 acc[NB][8];
      state_at<NB>(acc, ST, cS, kq, o, w01, w23);
      store_state<NB>(a, acc, fs, sr, h, v0w, lane);
    }
  } while (todo);
}

// Entry state rows of the wave's columns (or zeros) in the accumulator layout.
template <int NB>
__device__ __forceinline__ void load_entry(const Desc* dp, int ws, int lane, f32x4 (&T)[NB][8]) {
  const int g4 = lane >> 4, l16 = lane & 15;
  const unsigned long long sp = (unsigned long long)dp->sin;
  const float* sin = (const float*)(((unsigned long long)(unsigned)rfl((int)(sp >> 32)) << 32) | (unsigned)rfl((int)sp));
  if (sin) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float* row = sin + (size_t)(16 * NB * ws + 16 * nb + l16) * DK + 8 * g4;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        T[nb][dt] = __builtin_nontemporal_load((const gf32x4*)(row + 32 * (dt >> 1) + 4 * (dt & 1)));
    }
  } else {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) T[nb][dt] = zero;
  }
}

template <int BV>
__device__ __forceinline__ void state_loop(const Args& a, unsigned char* smem, int ws, int lane) {
  using C = Cfg<BV>;
  constexpr int NB = C::NB;
  const int g4 = lane >> 4, l16 = lane & 15;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  SOff<NB> o;
#pragma unroll
  for (int m = 0; m < 4; ++m) o.F[m] = l16 * 256 + (((4 * m + g4) ^ kq_swz(l16)) << 4);
  // lane i of a 16-lane group receives d_k column 32 m + 8 (i / 4) + 4 bb + i % 4 of
  // rows 4 g4 .. 4 g4 + 3 (dt = 2 m + bb)
  {
    const int r0 = 4 * g4 + (l16 >> 2), p = l16 & 3;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o.KT[dt] = r0 * 256 + ((((4 * (dt >> 1) + p) ^ kq_swz(r0))) << 4) + ((dt & 1) << 3);
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int vrow = 4 * g4 + (l16 >> 2), vcol = 16 * NB * ws + 16 * nb + (l16 & 3) * 4;
    o.V[nb] = vrow * BV * 2 + (((vcol >> 3) ^ v_swz<BV>(vrow)) << 4) + ((vcol & 7) << 1);
  }
  f32x4 ST[NB][8];
  bf16x8 Sb[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) ST[nb][dt] = zero;
#pragma unroll
    for (int m = 0; m < 4; ++m) Sb[nb][m] = cat8b(to_bf4(zero), to_bf4(zero));
  }

  lds_barrier();  // the helpers' iteration -1
  // The descriptor of chunk it + 1 is complete during chunk it (the helpers
  // wrote it one iteration earlier), so it is read before the barrier that
  // ends chunk it and the next chunk starts without an LDS round trip.
  SDesc cd = load_sdesc(smem + C::oTB + tD);
  // An item's entry state is loaded before the barrier that precedes its first
  // chunk (the previous item's state is dead by then), so that the load's
  // latency passes while the wave waits at the barrier.
  if (cd.valid && cd.first) load_entry<NB>(reinterpret_cast<const Desc*>(smem + C::oTB + tD), ws, lane, ST);
  for (int it = 0;; ++it) {
    const unsigned char* tb = smem + C::oTB + (it % 3) * kTB;
    if (!cd.valid) break;
    WALK_STAMP(it, 0);
    const int t0 = cd.t0, n = cd.n, h = cd.h, v0 = cd.v0;
    const int mode = cd.mode;
    const bool has_out = cd.has_out, need_exit = cd.need_exit, first = cd.first;
    unsigned long long todo = ((unsigned long long)cd.req_hi << 32) | cd.req_lo;
    if (need_exit) todo |= 1ull << (n - 1);
    const unsigned char* kq = smem + C::oKQ + (it % 3) * 32768;
    const unsigned char* vt = smem + C::oV + (it & 1) * C::VT;
    const unsigned char* pr = smem + C::oPR + (it & 1) * kPR;
    const int v0w = v0 + 16 * NB * ws;  // first column of the wave

    if constexpr (kStateCopiesK<BV>) {
      // The entry state loaded before the barrier is awaited here, by a wait
      // the compiler's own wait insertion sees: the copies below are inline
      // assembly, invisible to it, and a wait it placed later for the state
      // would wait for them too.
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), other counters untouched
    }
    if (first) {  // a new item: its entry state, loaded before the barrier
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int m = 0; m < 4; ++m) Sb[nb][m] = cat8b(to_bf4(ST[nb][2 * m]), to_bf4(ST[nb][2 * m + 1]));
    }
    if constexpr (kStateCopiesK<BV>) {  // K rows of chunk it + 2, split over the state waves
      const Desc nd = uniform_desc(reinterpret_cast<const Desc*>(smem + C::oND)[it & 1]);
      if (nd.valid) {
        unsigned char* k2 = smem + C::oKQ + ((it + 2) % 3) * 32768;
        if constexpr (C::NS == 1) {
          issue_rows<0, 16>(a, nd, a.k, k2, lane);
        } else {
          if (ws == 0) issue_rows<0, 8>(a, nd, a.k, k2, lane);
          else issue_rows<8, 16>(a, nd, a.k, k2, lane);
        }
      }
    }
    if (has_out)
      state_chunk<BV, true>(a, smem, tb, kq, vt, pr, o, ST, Sb, it, t0, n, h, v0w, mode, need_exit, todo, lane);
    else
      state_chunk<BV, false>(a, smem, tb, kq, vt, pr, o, ST, Sb, it, t0, n, h, v0w, mode, need_exit, todo, lane);
    WALK_STAMP(it, 7);
    if constexpr (kStateCopiesK<BV>) wait_vm();  // this wave's copies have landed (before the next entry loads)
    const Desc* dn = reinterpret_cast<const Desc*>(smem + C::oTB + ((it + 1) % 3) * kTB + tD);
    cd = load_sdesc(reinterpret_cast<const unsigned char*>(dn));
    WALK_STAMP(it, 8);
    if (cd.valid && cd.first) load_entry<NB>(dn, ws, lane, ST);
    WALK_STAMP(it, 9);
    lds_barrier();
  }
}

// ------------------------------------------------------------------ kernel

template <int BV>
__global__ void __launch_bounds__(Cfg<BV>::NTHR, 1) k_walk_pipe(const Args a) {
  using C = Cfg<BV>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = rfl(tid >> 6);  // wave index (uniform)
  if (*a.err != kNoError) return;  // structural error: nothing is computed
  const int count = a.level_count[a.level];
  const int base = a.level_ptr[a.level];
  const int xcd = blockIdx.x % kXcd;
  const bool helper = w >= C::NS;
  const int hid = w - C::NS;  // 0 or 1 on the helpers

  // Pairs of P whose second 16-token block lies above the diagonal ((0, 1) and
  // (2, 3)) are never written: clear them once in every P buffer.
  for (int e = tid; e < 3 * 2 * 64; e += C::NTHR) {
    const int slot = e >> 7, which = (e >> 6) & 1, ln = e & 63;
    *reinterpret_cast<uint2*>(smem + C::oPP + slot * kPP + (which ? 3 : 0) * 1024 + ln * 16 + 8) = make_uint2(0, 0);
  }

  // ---- prologue: describe chunks 0 and 1 and copy K, Q and the token tables
  // of chunk 0; the helpers' first loop iteration forms its products
  Desc* nds = reinterpret_cast<Desc*>(smem + C::oND);
  Feed ff;
  FeedRegs fr;
  feed_init(ff, fr, a);
  if (hid == 0) {
#pragma nounroll
    for (int i = 0; i < 2; ++i) {
      put_desc(reinterpret_cast<unsigned char*>(nds + i), feed_next<BV>(ff, fr, a, xcd, count, base, lane), lane);
      wait_vm();
    }
  }
  lds_barrier();
  if (helper) {
    const Desc d0 = uniform_desc(nds[0]);
    TokenRegs tr;
    if (hid == 1) tr = load_tokens(a, d0, lane);
    if (d0.valid) issue_kq(a, d0, smem + C::oKQ, hid, lane);
    wait_vm();
    if (hid == 1) store_tokens(a, d0, tr, smem + C::oTB, lane);
  }
  lds_barrier();

  if (helper) helper_loop<BV>(a, smem, hid, lane, ff, fr, xcd, count, base);
  else state_loop<BV>(a, smem, w, lane);
}

template <int BV>
hipError_t run(const Args& wa, int levels, hipStream_t s) {
  auto kern = k_walk_pipe<BV>;
  constexpr int bytes = Cfg<BV>::bytes;
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), bytes, Cfg<BV>::NTHR, nullptr);
  if (e != hipSuccess) return e;
  int cus = 0;
  e = current_device_cus(&cus);
  if (e != hipSuccess) return e;
  // one workgroup per CU (bounded by LDS), persistent over the level's items;
  // a multiple of the XCD count so that every XCD has the same number of workgroups
  const int grid = cus >= kXcd ? cus / kXcd * kXcd : kXcd;
  for (int l = 0; l < levels; ++l) {
    Args x = wa;
    x.level = l;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(Cfg<BV>::NTHR), bytes, s, x);
  }
  return hipGetLastError();
}

}  // namespace

bool walk_pipe_supported(int dtype, int dk, int bv) {
  return dtype == GDN_BF16 && dk == DK && (bv == 16 || bv == 32 || bv == 64);
}

hipError_t launch_walk_pipe(const gdn_tree_fwd_args& fa, const Meta& m, int bv, hipStream_t s) {
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
  wa.walk_ctr = m.walk_ctr;
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

#ifdef GDN_WALK_STAMPS
// Measurement build only: copies (clear = 0) or zeroes (clear != 0) the stamps.
extern "C" int gdn_walk_stamps(unsigned long long* host, int clear) {
  constexpr size_t n = sizeof(gdn::g_walk_stamps);
  if (clear) {
    static unsigned long long zero[n / sizeof(unsigned long long)];
    return (int)hipMemcpyToSymbol(HIP_SYMBOL(gdn::g_walk_stamps), zero, n);
  }
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(gdn::g_walk_stamps), n);
}
#endif
