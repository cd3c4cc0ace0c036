// ForkAttention for the full-attention layers of a tree-structured flat stream
// (Flide, "Accelerating Decision Inference with Exact State Forking", section
// 3.2.1 "Full-Attention Layers" and section 3.3.1 "GPU-Resident Metadata").
//
// Token t attends to its ancestors-or-self in its own sequence (the visibility
// rule under which every question computes its standalone prompt, section
// 3.2.3). On the segment table of the recurrence's planner (a segment is a
// maximal run of tokens each the child of the one before; a sequence of at most
// 64 tokens is one tree chunk), the keys visible to the queries of one 64-token
// chunk of a segment are key spans:
//
//   * the segment's own prefix [segment start, last query of the chunk], whose
//     tiles before the chunk are fully visible and whose last tile (the chunk
//     itself) is causal, and
//   * for every ancestor segment on the root path, its prefix up to the fork
//     token the path leaves it at, fully visible except for a span's last tile
//     when the fork token is not a tile's last key.
//
// A tree chunk has one tile, masked by its ancestor bits. Other requests'
// tokens are never in a span. The span lists are built on the GPU (one
// planning workgroup, after the recurrence's metadata kernels), so launch
// shapes depend only on the sizes.
//
// The attention kernel is a persistent grid of workgroups that claim (chunk,
// query heads) items, last chunks first. Every wave holds 16 queries of two
// query heads of one key/value group, so that every K and V fragment read from
// LDS feeds two matrix products, and walks the item's key tiles of 64 keys with
// an online softmax: S^T = K Q^T and O^T += V^T P^T on 16x16x32 bf16 matrix
// cores, fp32 softmax state. When a key/value group has a multiple of four
// query heads, a workgroup has eight waves (four query blocks x two head
// pairs), a ring of four K/V tiles and two tiles per step (one barrier per 128
// keys); a chunk of at most 32 queries is then split by key tiles over the
// wave pairs. Otherwise four waves share a double-buffered pair of tiles. K and
// V tiles are copied straight from HBM into LDS; fully visible tiles take no
// mask.
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int D = 128;        // head dimension
constexpr int kT = 64;        // keys per tile, queries per chunk
constexpr int kTileB = kT * D * 2;  // bytes of one K or V tile (bf16)
constexpr int kMaxLevels = 64;  // fork nesting levels an item's span list may hold
constexpr int kMaxSpans = kMaxLevels + 1;  // plus the sequence's cached keys
constexpr int oK = 0;  // K tiles, then V tiles, then the item's spans (int2)
__host__ __device__ constexpr int attn_lds(int nbuf) { return 2 * nbuf * kTileB + 8 * kMaxSpans; }
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.f;  // a row's weights stay below 2^kLazy before its reference moves

struct AttnArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* out;
  const unsigned long long* err;
  const unsigned long long* tree_mask;
  const int4* item_info;  // {first query, queries, mode | sequence << 1, spans}
  const int2* spans;      // [item][max_levels] inclusive key spans; span 0 is the item's own segment
  const int* n_items;
  int* claim;
  const __bf16* k_cache;
  const __bf16* v_cache;
  const int* cache_start;  // null: no cached keys
  int Hq, Hkv, max_levels;
  float c;  // scale * log2(e), positive
};

__device__ __forceinline__ void dma16(const void* sbase, unsigned voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_addr), "v"(voff), "s"(sbase)
               : "memory");
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ uint32_t lds_addr_of(const unsigned char* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)((const lds_void*)p));
}
__device__ __forceinline__ int rfl(int x) { return __builtin_amdgcn_readfirstlane(x); }
// A wave-uniform pointer made explicit (the copies take their base address in scalar registers).
__device__ __forceinline__ const __bf16* rfl_ptr(const __bf16* p) {
  const unsigned long long u = (unsigned long long)p;
  return (const __bf16*)(((unsigned long long)(unsigned)rfl((int)(u >> 32)) << 32) | (unsigned)rfl((int)u));
}
// 16-byte piece p of tile row r sits at slot p ^ swz(r) (spreads the rows over the LDS banks)
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
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
__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }

// Rows [row0, row0 + n) of one key/value head (row stride rs bytes) into a
// tile: wave w copies the 4-row blocks kB w .. kB w + kB - 1 (kB = 16 / NW);
// lane (g4, l16) fills slot l16 of row r = 4 blk + g4 with the row's piece
// l16 ^ swz(r). Rows at or past n are copied from row n - 1 (finite values:
// their keys are masked and their weights are zero), so that every wave issues
// exactly kB copies per tile and the waits can count them.
// vo_full holds the lane's offsets of a full tile (the same for every tile);
// l0 is the tile's LDS address.
template <int NW>
__device__ __forceinline__ void issue_tile(const __bf16* head0, int row0, int n, unsigned rs, uint32_t l0, int w,
                                           int lane, const unsigned (&vo_full)[16 / NW]) {
  constexpr int kB = 16 / NW;
  const int g4 = lane >> 4, l16 = lane & 15;
  const unsigned char* src = reinterpret_cast<const unsigned char*>(rfl_ptr(head0)) + (size_t)rfl(row0) * rs;
  if (n == kT) {
#pragma unroll
    for (int b = 0; b < kB; ++b) dma16(src, vo_full[b], l0 + (kB * w + b) * 1024);
  } else {
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      const int blk = kB * w + b, r = 4 * blk + g4;
      const unsigned vo = (unsigned)min(r, n - 1) * rs + (unsigned)((l16 ^ swz(r)) << 4);
      dma16(src, vo, l0 + blk * 1024);
    }
  }
}

// Wait until at most 0, 1 or 2 tiles' copies (of kPer each) of this wave are in flight.
template <int kPer>
__device__ __forceinline__ void wait_tiles(int pending) {
  static_assert(kPer == 4 || kPer == 8, "copies per tile");
  if (pending == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if (pending == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kPer) : "memory");
  else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kPer) : "memory");
}

// One key tile of an item: its first key, valid keys, and mask kind.
struct Tile {
  int valid, k0, n, kind;  // kind 0: no mask beyond n; 1: causal (the item's own chunk); 2: tree ancestor bits
  int sp, end;             // span index and the span's last key
};

// The tile after (sp, k0) in the item's span list (spans in LDS; span `own` is
// the item's own segment, a span before it the cached keys).
__device__ __forceinline__ Tile next_tile(const int2* sps, int nsp, int own, int sp, int k0, int q0, int tree) {
  Tile t = {0, 0, 0, 0, 0, 0};
  while (sp < nsp) {
    const int2 s = sps[sp];
    if (k0 < 0) k0 = s.x;
    if (k0 <= s.y) {  // every field wave-uniform (the spans are the same for every lane)
      t.valid = 1;
      t.sp = rfl(sp);
      t.k0 = rfl(k0);
      t.end = rfl(s.y);
      t.n = rfl(min(kT, s.y - k0 + 1));
      t.kind = rfl((sp == own && k0 == q0) ? (tree ? 2 : 1) : 0);
      return t;
    }
    ++sp;
    k0 = -1;
  }
  return t;
}

// The tile after t: inside t's span without reading the span list again.
__device__ __forceinline__ Tile after(const Tile& t, const int2* sps, int nsp, int own, int q0, int tree) {
  if (!t.valid) return t;
  const int k0 = t.k0 + kT;
  if (k0 <= t.end) {
    Tile u = t;
    u.k0 = k0;
    u.n = min(kT, t.end - k0 + 1);
    u.kind = (t.sp == own && k0 == q0) ? (tree ? 2 : 1) : 0;
    return u;
  }
  return next_tile(sps, nsp, own, t.sp + 1, -1, q0, tree);
}

// HPW query heads of one key/value group per wave: every K and V fragment read
// from LDS feeds HPW matrix products. NW = 4 waves take 16 queries each (HPW
// heads per item, two workgroups per CU, K/V tiles double-buffered); NW = 8
// waves take 16 queries and one of two head pairs each (2 HPW heads per item
// sharing every K/V tile, one workgroup per CU, a ring of four tiles so that
// three are in flight while one is used).
template <int HPW, int NW, bool CACHE>
__global__ void __launch_bounds__(64 * NW, NW == 8 ? 1 : 2) k_fork_attn(const AttnArgs a) {
  constexpr int kBuf = NW == 8 ? 4 : 2;  // K/V tile buffers
  constexpr int kPer = 2 * (16 / NW);    // copies per wave and tile (K and V)
  constexpr int kHW = HPW * (NW / 4);    // query heads per item
  constexpr int oV_ = kBuf * kTileB, oSp_ = 2 * kBuf * kTileB;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ int s_claim;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = rfl(tid >> 6);
  const int wq = w & 3, wh = w >> 2;  // the wave's query block and head pair
  const int g4 = lane >> 4, l16 = lane & 15;
  if (*a.err != kNoError) return;  // structural error in the tree: nothing is computed
  const int n_items = *a.n_items;
  const int HG = a.Hq / kHW;  // head groups of kHW query heads
  const long long total = (long long)n_items * HG;
  const int G = a.Hq / a.Hkv;
  const unsigned rs_kv = (unsigned)a.Hkv * (D * 2);
  int2* sps = reinterpret_cast<int2*>(smem + oSp_);
  // A-operand rows of the K fragments (row l16 of a 16-key block, d 32 ks + 8 g4 .. + 7)
  int oF[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) oF[ks] = l16 * 256 + (((4 * ks + g4) ^ swz(l16)) << 4);
  // transposed reads of V: lane i of a 16-lane group receives d column 32 m + 8 (i / 4) + 4 bb + i % 4 of
  // keys 4 g4 .. 4 g4 + 3 (dt = 2 m + bb); the accumulator element r of O^T block dt is then
  // d = 32 m + 8 g4 + 4 bb + r for query l16
  int oT[8];
  {
    const int r0 = 4 * g4 + (l16 >> 2), p = l16 & 3;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oT[dt] = r0 * 256 + ((((4 * (dt >> 1) + p) ^ swz(r0))) << 4) + ((dt & 1) << 3);
  }
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const bf16x8 kOnes = __builtin_bit_cast(bf16x8, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
  // the lane's copy offsets within a full tile, and the LDS address of the shared buffer
  unsigned vo_full[16 / NW];
#pragma unroll
  for (int b = 0; b < 16 / NW; ++b) {
    const int r = 4 * ((16 / NW) * w + b) + g4;
    vo_full[b] = (unsigned)r * rs_kv + (unsigned)((l16 ^ swz(r)) << 4);
  }
  const uint32_t lds0 = lds_addr_of(smem);

  for (;;) {
    if (tid == 0) s_claim = atomicAdd(a.claim, 1);
    lds_barrier();  // (also: every wave is done with the previous item's spans and tiles)
    const long long idx = s_claim;
    if (idx >= total) break;
    // items in reverse stream order: a segment's later chunks see more keys,
    // so the longer items tend to go first and the short ones fill the tail
    const int item = n_items - 1 - (int)(idx / HG), hg0 = (int)(idx % HG) * kHW, h0 = hg0 + wh * HPW;
    const int hk = hg0 / G;  // the item's heads share one key/value head (G is a multiple of kHW)
    const int4 inf = a.item_info[item];
    // Every span slot of the item is read together with its record (the table
    // holds max_levels slots per item), so the list does not wait for the
    // record's span count; only the item's own spans reach LDS below.
    const int span_slots = min(a.max_levels, kMaxLevels);
    int2 spv = make_int2(0, 0);
    if (tid < span_slots) spv = a.spans[(size_t)item * a.max_levels + tid];
    const int q0 = rfl(inf.x), nq = rfl(inf.y), tree = rfl(inf.z & 1), sq = rfl(inf.z >> 1);
    // the sequence's cached keys, if any, come first (span 0), then the item's spans
    int own = 0;
    if (CACHE) {
      const int c0 = a.cache_start[sq], c1 = a.cache_start[sq + 1];
      own = rfl(c1 > c0 ? 1 : 0);
      if (own && tid == 0) sps[0] = make_int2(c0, c1 - 1);
    }
    const int nsp = rfl(min(inf.w, kMaxLevels)) + own;
    if (tid < span_slots && tid + own < nsp) sps[tid + own] = spv;
    // Eight waves take two tiles per step (one barrier and one wait per 128
    // keys). A chunk of at most 32 queries is split by key tiles: the waves of
    // query blocks 2 and 3 take the odd tiles of blocks 0 and 1's queries, and
    // hand their softmax states over at the end; otherwise every wave takes both.
    const int S = NW == 8 ? 2 : 1;                 // tiles per step
    const bool split = NW == 8 && nq <= 32;
    const int par = split ? wq >> 1 : 0;           // the wave's tile within a step, when split
    const int qb = split ? wq & 1 : wq;            // the wave's query block
    // this wave's 16 queries of each head as MFMA fragments (zero past the chunk's queries)
    const int qi = 16 * qb + l16;  // query within the chunk
    bf16x8 Qf[HPW][4];
    unsigned long long tmask = 0;
    {
      const bool ok = qi < nq;
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        const __bf16* qrow = a.q + ((size_t)(q0 + (ok ? qi : 0)) * a.Hq + h0 + j) * D;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          bf16x8 x = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks + 8 * g4);
          if (!ok) x = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
          Qf[j][ks] = x;
        }
      }
      if (tree && ok) tmask = a.tree_mask[(size_t)sq * kT + qi];
    }
    const __bf16* k0p = a.k + (size_t)hk * D;
    const __bf16* v0p = a.v + (size_t)hk * D;
    const __bf16* kc0p = CACHE ? a.k_cache + (size_t)hk * D : k0p;
    const __bf16* vc0p = CACHE ? a.v_cache + (size_t)hk * D : v0p;
    lds_barrier();  // spans in LDS
    // a window of kBuf consecutive tiles: the step's S tiles first; the first
    // kBuf - S are copied now (tile g + i of the item goes to buffer (g + i) mod kBuf)
    Tile tw[kBuf];
    tw[0] = next_tile(sps, nsp, own, 0, -1, q0, tree);
#pragma unroll
    for (int i = 1; i < kBuf; ++i) tw[i] = after(tw[i - 1], sps, nsp, own, q0, tree);
    auto issue = [&](const Tile& t, int buf) {
      const bool cc = t.sp < own;
      issue_tile<NW>(cc ? kc0p : k0p, t.k0, t.n, rs_kv, lds0 + oK + buf * kTileB, w, lane, vo_full);
      issue_tile<NW>(cc ? vc0p : v0p, t.k0, t.n, rs_kv, lds0 + oV_ + buf * kTileB, w, lane, vo_full);
    };
#pragma unroll
    for (int i = 0; i < kBuf - 1; ++i)
      if (i < kBuf - S && tw[i].valid) issue(tw[i], i);
    f32x4 O[HPW][8];
    float m[HPW];
    f32x4 L[HPW];  // row sums of the weights, formed on the matrix cores (every element the query's sum)
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) O[j][dt] = zero;
      m[j] = -INFINITY;
      L[j] = zero;
    }
    const bool active = 16 * qb < nq;
    for (int g = 0; tw[0].valid; g += S) {
      // the step's tiles have landed (every wave's copies), and every wave is
      // done with the buffers the next copies go to (the previous step's)
      int pending = 0;
#pragma unroll
      for (int i = 1; i < kBuf - 1; ++i) pending += (i >= S && i < kBuf - S) ? tw[i].valid : 0;
      wait_tiles<kPer>(pending);
      lds_barrier();
#pragma unroll
      for (int i = 1; i < kBuf; ++i)
        if (i >= kBuf - S && tw[i].valid) issue(tw[i], (g + i) & (kBuf - 1));
#pragma unroll
      for (int p = 0; p < S; ++p) {  // unrolled: one tile's scores can overlap the other's softmax
      if (split && p != par) continue;
      const Tile cur = p ? tw[1] : tw[0];
      const int b = (g + p) & (kBuf - 1);
      if (active && cur.valid) {
        const unsigned char* kt = smem + oK + b * kTileB;
        const unsigned char* vt = smem + oV_ + b * kTileB;
        // S^T = K Q^T: lane (query l16, g4) holds keys 16 kb + 4 g4 + r
        f32x4 S[HPW][4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
          for (int j = 0; j < HPW; ++j) S[j][kb] = zero;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kt + kb * 4096 + oF[ks]);
#pragma unroll
            for (int j = 0; j < HPW; ++j) S[j][kb] = mma32(kf, Qf[j][ks], S[j][kb]);
          }
        }
        bf16x8 w01[HPW], w23[HPW];
        float alpha[HPW];
        bool rescale[HPW];  // wave-uniform: some query of the wave moved its reference
        // masks only where a tile is not fully visible (the diagonal tile, a span's last tile, tree tiles)
        const bool masked = cur.kind != 0 || cur.n < kT;
        unsigned vis = 0xffffu;  // bit 4 kb + r: key 16 kb + 4 g4 + r is visible to query qi
        if (masked) {
          unsigned long long ok = cur.kind == 2 ? tmask : cur.kind == 1 ? (2ull << qi) - 1ull : ~0ull;
          if (cur.n < kT) ok &= (1ull << cur.n) - 1ull;
          const unsigned long long sh = ok >> (4 * g4);
          vis = (unsigned)((sh & 0xfull) | ((sh >> 12) & 0xf0ull) | ((sh >> 24) & 0xf00ull) | ((sh >> 36) & 0xf000ull));
        }
#pragma unroll
        for (int j = 0; j < HPW; ++j) {
          if (masked) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (!((vis >> (4 * kb + r)) & 1u)) S[j][kb][r] = -INFINITY;
          }
          // running maxima in the scaled log2 domain (scale > 0): m = c max(s)
          float mt = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) mt = fmaxf(mt, S[j][kb][r]);
          mt = fmaxf(mt, __shfl_xor(mt, 16));
          mt = fmaxf(mt, __shfl_xor(mt, 32));
          // The reference m (scaled log2 domain) moves up only when this tile's
          // maximum exceeds it by more than kLazy, so that the weights stay below
          // 2^kLazy; softmax does not depend on the reference, and most tiles
          // then leave the accumulators alone.
          const float ms = mt * a.c;
          const float mn = ms > m[j] + kLazy ? ms : m[j];
          const float mref = mn == -INFINITY ? 0.f : mn;
          alpha[j] = __builtin_amdgcn_exp2f(m[j] - mref);
          rescale[j] = __builtin_amdgcn_ballot_w64(mn != m[j]) != 0ull;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) S[j][kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[j][kb][r], a.c, -mref));
          m[j] = mn;
          w01[j] = cat8b(to_bf4(S[j][0]), to_bf4(S[j][1]));
          w23[j] = cat8b(to_bf4(S[j][2]), to_bf4(S[j][3]));
        }
        // rescale the accumulators only on the (rare) tiles that moved a
        // reference: a real branch (the empty asm keeps the compiler from
        // turning it into selects on every tile)
#pragma unroll
        for (int j = 0; j < HPW; ++j) {
          if (rescale[j]) {
            asm volatile("" ::: "memory");
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
#pragma unroll
              for (int r = 0; r < 4; ++r) O[j][dt][r] *= alpha[j];
#pragma unroll
            for (int r = 0; r < 4; ++r) L[j][r] *= alpha[j];
          }
        }
        // the weights' row sums: a block of ones times P^T (the same bf16 weights
        // as the numerator's)
#pragma unroll
        for (int j = 0; j < HPW; ++j) {
          const f32x4 t = mma32(kOnes, w01[j], L[j]);
          L[j] = mma32(kOnes, w23[j], t);
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const unsigned char* vp = vt + oT[dt];
          const bf16x8 v01 = cat8(tr_read(vp), tr_read(vp + 4096));
          const bf16x8 v23 = cat8(tr_read(vp + 8192), tr_read(vp + 12288));
#pragma unroll
          for (int j = 0; j < HPW; ++j) {
            const f32x4 o = mma32(v01, w01[j], O[j][dt]);
            O[j][dt] = mma32(v23, w23[j], o);
          }
        }
      }
      }
      if (S == 2) {
#pragma unroll
        for (int i = 0; i < kBuf - 2; ++i) tw[i] = tw[i + 2];
        tw[kBuf - 2] = after(tw[kBuf - 3], sps, nsp, own, q0, tree);
        tw[kBuf - 1] = after(tw[kBuf - 2], sps, nsp, own, q0, tree);
      } else {
#pragma unroll
        for (int i = 0; i < kBuf - 1; ++i) tw[i] = tw[i + 1];
        tw[kBuf - 1] = after(tw[kBuf - 2], sps, nsp, own, q0, tree);
      }
    }
    if (split) {
      // the odd-tile waves' states (references m, row sums L, unnormalised O)
      // to their partners, through the idle tile ring: unit u of lane l of
      // pair (head pair, query block) at ((pair U + u) 64 + l) 16 bytes
      constexpr int U = HPW * 9 + 1;
      f32x4* xb = reinterpret_cast<f32x4*>(smem) + (size_t)(wh * 2 + qb) * U * 64 + lane;
      lds_barrier();  // every wave is done with the ring
      if (par && active) {
#pragma unroll
        for (int j = 0; j < HPW; ++j) {
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) xb[(j * 9 + dt) * 64] = O[j][dt];
          xb[(j * 9 + 8) * 64] = L[j];
        }
        f32x4 mm = zero;
#pragma unroll
        for (int j = 0; j < HPW; ++j) mm[j] = m[j];
        xb[(HPW * 9) * 64] = mm;
      }
      lds_barrier();
      if (!par && active) {
        const f32x4 mm = xb[(HPW * 9) * 64];
#pragma unroll
        for (int j = 0; j < HPW; ++j) {
          // both sides rescaled to the larger reference (a side without keys has m = -inf and weight 0)
          const float mo = mm[j], mx = fmaxf(m[j], mo);
          const float fa = m[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[j] - mx);
          const float fb = mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mo - mx);
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) {
            const f32x4 ob = xb[(j * 9 + dt) * 64];
#pragma unroll
            for (int r = 0; r < 4; ++r) O[j][dt][r] = O[j][dt][r] * fa + ob[r] * fb;
          }
          const f32x4 lb = xb[(j * 9 + 8) * 64];
#pragma unroll
          for (int r = 0; r < 4; ++r) L[j][r] = L[j][r] * fa + lb[r] * fb;
        }
      }
    }
    if (active && !par && qi < nq) {
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        const float inv = 1.f / L[j][0];
        __bf16* orow = a.out + ((size_t)(q0 + qi) * a.Hq + h0 + j) * D;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          f32x4 o = O[j][dt];
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] *= inv;
          *reinterpret_cast<bf16x4*>(orow + 32 * (dt >> 1) + 8 * g4 + 4 * (dt & 1)) = to_bf4(o);
        }
      }
    }
  }
}

// ------------------------------------------------------------- item tables

struct ItemTables {
  int4* item_info;
  int2* spans;
  int* item_off;
  int* n_items;
  int* claim;
};

// Exclusive scan over a 1024-thread block; *total gets the sum.
__device__ inline int block_scan(int v, int* sh, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wv] = x;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < 16; ++i) {
      const int t = sh[i];
      sh[i] = run;
      run += t;
    }
    sh[16] = run;
  }
  __syncthreads();
  const int ex = sh[wv] + x - v;
  *total = sh[16];
  __syncthreads();
  return ex;
}

__device__ inline int seg_containing(const int* seg_start, int n_seg, int t) {
  int lo = 0, hi = n_seg;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (seg_start[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// One workgroup: chunk items of every segment (in stream order) and each
// item's key spans: its own segment's prefix, then the ancestor segments' prefixes.
// cache_start must be a CSR over [0, Tc]: a bad entry raises GDN_DEV_CACHE (the
// attention kernel then computes nothing, so no cached row outside [0, Tc) is read).
__device__ inline void check_cache(const Meta& m, const int* cache_start, int n_seq, long long Tc) {
  if (!cache_start) return;
  for (int s = threadIdx.x; s <= n_seq; s += blockDim.x) {
    const int v = cache_start[s];
    const bool bad = (s == 0 && v != 0) || (s > 0 && (v < cache_start[s - 1] || v > Tc)) || (s == n_seq && v != Tc);
    if (bad) raise_error(m.err, GDN_DEV_CACHE, s);
  }
}

__global__ void __launch_bounds__(1024) k_attn_items(Meta m, ItemTables t, int max_levels, const int* cache_start,
                                                     int n_seq, long long Tc) {
  __shared__ int sh[17];
  const int tid = threadIdx.x;
  check_cache(m, cache_start, n_seq, Tc);
  const int n_seg = (*m.err != kNoError) ? 0 : *m.n_seg;
  int run = 0;
  for (int base = 0; base < n_seg; base += 1024) {
    const int s = base + tid;
    const int nch = s < n_seg ? (m.seg_mode[s] ? 1 : (m.seg_len[s] + kT - 1) / kT) : 0;
    int tot;
    const int ex = block_scan(nch, sh, &tot);
    if (s < n_seg) t.item_off[s] = run + ex;
    run += tot;
  }
  if (tid == 0) {
    *t.n_items = run;
    *t.claim = 0;
  }
  __syncthreads();
  for (int s = tid; s < n_seg; s += 1024) {
    const int st = m.seg_start[s], len = m.seg_len[s], mode = m.seg_mode[s], sq = m.seg_seq[s];
    const int nch = mode ? 1 : (len + kT - 1) / kT;
    const int off = t.item_off[s];
    int nsp = 1;
    int e = m.seg_entry[s];
    while (e >= 0 && nsp < max_levels) {  // the planner bounds the nesting below max_levels
      const int p = seg_containing(m.seg_start, n_seg, e);
      const int2 span = make_int2(m.seg_start[p], e);
      for (int c = 0; c < nch; ++c) t.spans[(size_t)(off + c) * max_levels + nsp] = span;
      ++nsp;
      e = m.seg_entry[p];
    }
    for (int c = 0; c < nch; ++c) {
      const int q0 = st + kT * c, nq = mode ? len : min(kT, len - kT * c);
      t.spans[(size_t)(off + c) * max_levels] = make_int2(st, q0 + nq - 1);
      t.item_info[off + c] = make_int4(q0, nq, mode | (sq << 1), nsp);
    }
  }
}

__global__ void k_attn_replan(Meta m, int* claim, unsigned long long tag, const int* cache_start, int n_seq,
                              long long Tc) {
  if (threadIdx.x == 0) {
    *claim = 0;
    if (*m.plan_tag != tag) raise_error(m.err, GDN_DEV_NOT_PLANNED, 0);
  }
  check_cache(m, cache_start, n_seq, Tc);
}

}  // namespace

bool attn_layout(const gdn_attn_dims& d, AttnLayout* A) {
  gdn_tree_dims pd = {};
  pd.T = d.T;
  pd.H = 1;
  pd.Dk = 0;  // no fork-state slots: the attention reads the segment tables only
  pd.Dv = 0;
  pd.n_seq = d.n_seq;
  pd.dtype = d.dtype;
  pd.max_forks = (int)(d.T > 0x7fffffff ? 0x7fffffff : d.T);
  pd.max_levels = d.max_levels;
  if (!compute_layout(pd, &A->plan)) return false;
  A->pd = pd;
  const size_t T = (size_t)(d.T > 0 ? d.T : 0);
  size_t off = A->plan.pub.total;
  auto take = [&](size_t bytes) { size_t o = off; off = (off + bytes + 255) & ~(size_t)255; return o; };
  A->item_info = take(16 * T);
  A->spans = take(8 * T * (size_t)d.max_levels);
  A->item_off = take(4 * T);
  A->n_items = take(4);
  A->claim = take(4);
  A->total = off;
  return true;
}

hipError_t launch_attention(const gdn_attn_args& aa, const AttnLayout& A, hipStream_t s) {
  char* ws = (char*)aa.workspace;
  Meta m = meta_from(ws, A.plan);
  ItemTables t;
  t.item_info = (int4*)(ws + A.item_info);
  t.spans = (int2*)(ws + A.spans);
  t.item_off = (int*)(ws + A.item_off);
  t.n_items = (int*)(ws + A.n_items);
  t.claim = (int*)(ws + A.claim);
  gdn_tree_fwd_args pa = {};
  pa.dims = A.pd;
  pa.parent_idx = aa.parent_idx;
  pa.seq_start = aa.seq_start;
  pa.workspace = aa.workspace;
  pa.workspace_bytes = aa.workspace_bytes;
  const unsigned long long tag = plan_fingerprint(pa);
  hipError_t e;
  if (aa.flags & GDN_ATTN_PLANNED) {
    hipLaunchKernelGGL(k_attn_replan, dim3(1), dim3(256), 0, s, m, t.claim, tag, aa.cache_start, aa.dims.n_seq,
                       (long long)aa.Tc);
  } else {
    e = launch_plan(pa, m, A.plan, tag, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_attn_items, dim3(1), dim3(1024), 0, s, m, t, aa.dims.max_levels, aa.cache_start,
                       aa.dims.n_seq, (long long)aa.Tc);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (aa.dims.T == 0 || aa.dims.n_seq == 0) return hipSuccess;
  AttnArgs x;
  x.q = reinterpret_cast<const __bf16*>(aa.q);
  x.k = reinterpret_cast<const __bf16*>(aa.k);
  x.v = reinterpret_cast<const __bf16*>(aa.v);
  x.out = reinterpret_cast<__bf16*>(aa.out);
  x.err = m.err;
  x.tree_mask = m.tree_mask;
  x.item_info = t.item_info;
  x.spans = t.spans;
  x.n_items = t.n_items;
  x.claim = t.claim;
  x.k_cache = reinterpret_cast<const __bf16*>(aa.k_cache);
  x.v_cache = reinterpret_cast<const __bf16*>(aa.v_cache);
  x.cache_start = aa.cache_start;
  x.Hq = aa.dims.Hq;
  x.Hkv = aa.dims.Hkv;
  x.max_levels = aa.dims.max_levels;
  x.c = aa.scale * kLog2e;
  // two query heads per wave when a key/value group has an even number of them; cached keys in a variant of their own
  // eight waves and four query heads of a key/value group per item when the
  // group has a multiple of four, else four waves and two heads (or one)
  const int G = aa.dims.Hq / aa.dims.Hkv;
  const bool cache = aa.cache_start != nullptr;
  const bool eight = G % 4 == 0, two = G % 2 == 0;
  void (*kern)(const AttnArgs) = eight ? (cache ? k_fork_attn<2, 8, true> : k_fork_attn<2, 8, false>)
                                 : two ? (cache ? k_fork_attn<2, 4, true> : k_fork_attn<2, 4, false>)
                                       : (cache ? k_fork_attn<1, 4, true> : k_fork_attn<1, 4, false>);
  const int threads = eight ? 512 : 256, lds = attn_lds(eight ? 4 : 2);
  int cus = 0, occ = 1;
  e = ensure_dynamic_lds(reinterpret_cast<const void*>(kern), lds, threads, &occ);
  if (e != hipSuccess) return e;
  e = current_device_cus(&cus);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(cus * occ), dim3(threads), lds, s, x);
  return hipGetLastError();
}

int attn_max_spans() { return kMaxLevels; }

}  // namespace gdn
