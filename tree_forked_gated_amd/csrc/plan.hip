// Tree metadata built on the GPU, before the walk reads it.
//
// Flide ("Accelerating Decision Inference with Exact State Forking", section
// 3.3.1) keeps every quantity that depends on the round's composition in
// compact device buffers that the kernels read, so launch shapes depend only
// on the stream length. Here the launch grids depend only on T, n_seq and the
// capacities; the tree itself is data.
//
// Rules (the chunking is this library's own; the pages fix only that a
// question's chunks start exactly at its fork, Flide section 3.5, and that a
// draft tree is solved as one triangular system, TreeWY "Speculative
// Verification for Gated DeltaNet Hybrids" section 3, Eq. 2):
//  * a sequence of at most 64 tokens is one tree chunk with a 64 x 64
//    ancestor-or-self bit mask;
//  * a longer sequence is cut into segments, each starting at a token whose
//    parent is not the token just before it; each segment into 64-token chunks
//    from its start;
//  * the parent of a segment start is a fork token and owns a fork-state slot
//    (slots numbered in stream order); the segment's level is the level of the
//    segment holding its fork token plus one, 0 from an initial state.
#include "gdn_internal.h"

namespace gdn {

namespace {

__device__ inline int upper_bound_seq(const int* seq_start, int n_seq, int t) {
  // largest s in [0, n_seq) with seq_start[s] <= t (seq_start validated separately; never reads out of range)
  int lo = 0, hi = n_seq;  // answer in [lo, hi)
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (seq_start[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ inline int seg_of(const int* seg_start, int n_seg, int t) {
  int lo = 0, hi = n_seg;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (seg_start[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

constexpr int kBkoLevels = 16;  // levels whose length-bucket offsets are formed in LDS

// Exclusive prefix sum over the 64 lanes of a wave.
__device__ inline int wave_excl_scan(int v) {
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if ((threadIdx.x & 63) >= o) x += y;
  }
  return x - v;
}

// True when seq_start failed validation: later kernels must not index with it.
__device__ inline bool bad_csr(const Meta& m) { return (*m.err >> 32) == (unsigned long long)GDN_DEV_SEQ_START; }

__global__ void k_init(Meta m, int T, int n_seq, int max_levels) {
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < T) {
    m.tok_seq[i] = 0;
    m.out_map[i] = kUnmapped;
    m.state_map[i] = kUnmapped;
    m.is_fork[i] = 0;
    m.is_start[i] = 0;
    m.fork_slot[i] = -1;
    m.depth[i] = 0;
  }
  if (i < (long long)n_seq * kChunk) m.tree_mask[i] = 0ull;
  if (i < max_levels) m.level_count[i] = 0;
  if (i < (long long)max_levels * kLenBuckets) {
    m.level_fill[i] = 0;
    m.level_bkt[i] = 0;
  }
  if (i < (long long)max_levels * kSchedInts) m.walk_ctr[i] = (i % kSchedInts) == kWalkQueues ? 0x7fffffff : 0;
  if (i == 0) {
    *m.err = kNoError;
    *m.n_seg = 0;
    *m.n_fork = 0;
    *m.plan_tag = 0ull;
  }
}

__global__ void k_replan_check(Meta m, int max_levels, unsigned long long tag) {
  for (int i = threadIdx.x; i < max_levels * kWalkQueues; i += blockDim.x)
    m.walk_ctr[(i / kWalkQueues) * kSchedInts + i % kWalkQueues] = 0;
  if (threadIdx.x == 0 && *m.plan_tag != tag) raise_error(m.err, GDN_DEV_NOT_PLANNED, 0);
}

// Per token: sequence, order checks, segment starts and fork flags. The same
// launch checks seq_start (threads 0..n_seq) and maps the requested rows
// (threads beyond T). With a bad seq_start its error (the smallest code) is the
// one reported; the lookups below stay in range whatever seq_start holds.
__device__ inline void map_row(const int* rows, int n, int i, int T, int* map, unsigned long long* err) {
  if (i >= n) return;
  int r = rows[i];
  if (r < 0 || r >= T) raise_error(err, GDN_DEV_ROWS, i);
  else atomicMin(&map[r], i);
}

__device__ inline void check_row(const int* rows, int n, int i, int T, const int* map, unsigned long long* err) {
  if (i >= n) return;
  int r = rows[i];
  if (r >= 0 && r < T && map[r] != i) raise_error(err, GDN_DEV_ROWS, i);
}

__global__ void k_tokens(const int* parent, const int* seq_start, int n_seq, int T, const int* out_rows, int n_out,
                         const int* state_rows, int n_state, Meta m) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid <= n_seq) {
    const int s = (int)gid;
    const int v = seq_start[s];
    // the last entry must be T also when it is the first (n_seq = 0)
    if (s == 0 && v != 0) {
      raise_error(m.err, GDN_DEV_SEQ_START, 0);
    } else if (s > 0 && (v < seq_start[s - 1] || v > T)) {
      raise_error(m.err, GDN_DEV_SEQ_START, s);
    } else if (s == n_seq && v != T) {
      raise_error(m.err, GDN_DEV_SEQ_START, s);
    }
  }
  if (gid >= T) {
    const long long i = gid - T;
    if (out_rows && i < n_out) map_row(out_rows, n_out, (int)i, T, m.out_map, m.err);
    if (state_rows && i < n_state) map_row(state_rows, n_state, (int)i, T, m.state_map, m.err);
    return;
  }
  if (n_seq <= 0) return;
  const int t = (int)gid;
  int s = upper_bound_seq(seq_start, n_seq, t);
  m.tok_seq[t] = s;
  int a = seq_start[s], b = seq_start[s + 1];
  bool tree = (b - a) <= kChunk;
  int p = parent[t];
  bool ok = true;
  if (p < -1 || p >= t) {
    raise_error(m.err, GDN_DEV_PARENT_ORDER, t);
    ok = false;
  } else if (p >= 0 && p < a) {
    raise_error(m.err, GDN_DEV_PARENT_SEQ, t);
    ok = false;
  }
  int start = tree ? (t == a) : (p < 0 || p != t - 1);
  m.is_start[t] = start;
  if (!tree && start && ok && p >= 0) m.is_fork[p] = 1;
}

// ---- exclusive scans of is_start (segment ids) and is_fork (slot ids)

__device__ inline int block_excl_scan(int v, int* sh, int* total) {
  // 256-thread exclusive scan through LDS (Hillis-Steele on the inclusive form)
  int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    int x = (tid >= off) ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += x;
    __syncthreads();
  }
  int incl = sh[tid];
  *total = sh[255];
  __syncthreads();
  return incl - v;
}

// Block totals of the scans; the same launch checks that requested rows are
// distinct (every mapping is in place once the token launch is done).
__global__ void __launch_bounds__(256) k_scan_reduce(int T, const int* out_rows, int n_out, const int* state_rows,
                                                     int n_state, int row_blocks, Meta m) {
  __shared__ int sh[256];
  if ((int)blockIdx.x >= (int)gridDim.x - row_blocks) {
    const int i = ((int)blockIdx.x - ((int)gridDim.x - row_blocks)) * 256 + threadIdx.x;
    if (out_rows) check_row(out_rows, n_out, i, T, m.out_map, m.err);
    if (state_rows) check_row(state_rows, n_state, i, T, m.state_map, m.err);
    return;
  }
  int base = blockIdx.x * kScanTile;
  int a = 0, f = 0;
  for (int i = threadIdx.x; i < kScanTile; i += 256) {
    int t = base + i;
    if (t < T) { a += m.is_start[t]; f += m.is_fork[t]; }
  }
  int ta, tf;
  block_excl_scan(a, sh, &ta);
  block_excl_scan(f, sh, &tf);
  if (threadIdx.x == 0) {
    m.scan_sums[2 * blockIdx.x] = ta;
    m.scan_sums[2 * blockIdx.x + 1] = tf;
  }
}

__global__ void __launch_bounds__(256) k_scan_top(int nb, Meta m) {
  __shared__ int sh[256];
  int* offs = m.scan_sums + 2 * nb;
  int run_a = 0, run_f = 0;
  for (int c = 0; c < nb; c += 256) {
    int i = c + threadIdx.x;
    int a = (i < nb) ? m.scan_sums[2 * i] : 0;
    int f = (i < nb) ? m.scan_sums[2 * i + 1] : 0;
    int ta, tf;
    int ea = block_excl_scan(a, sh, &ta);
    int ef = block_excl_scan(f, sh, &tf);
    if (i < nb) {
      offs[2 * i] = run_a + ea;
      offs[2 * i + 1] = run_f + ef;
    }
    run_a += ta;
    run_f += tf;
  }
  if (threadIdx.x == 0) {
    *m.n_seg = run_a;
    *m.n_fork = run_f;
  }
}

// FOLD: the offsets of the preceding blocks are summed here (few blocks);
// otherwise k_scan_top has written them.
template <bool FOLD>
__global__ void __launch_bounds__(256) k_scan_apply(int T, int nb, int max_forks, Meta m) {
  __shared__ int sh[256];
  constexpr int per = kScanTile / 256;
  int base_a = 0, base_f = 0;
  if (FOLD) {
    int pa = 0, pf = 0, qa = 0, qf = 0;  // preceding blocks, all blocks
    for (int b = threadIdx.x; b < nb; b += 256) {
      const int sa = m.scan_sums[2 * b], sf = m.scan_sums[2 * b + 1];
      qa += sa;
      qf += sf;
      if (b < (int)blockIdx.x) {
        pa += sa;
        pf += sf;
      }
    }
    int t0, t1, t2, t3;
    block_excl_scan(pa, sh, &t0);
    block_excl_scan(pf, sh, &t1);
    block_excl_scan(qa, sh, &t2);
    block_excl_scan(qf, sh, &t3);
    base_a = t0;
    base_f = t1;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      *m.n_seg = t2;
      *m.n_fork = t3;
    }
  } else {
    base_a = m.scan_sums[2 * nb + 2 * blockIdx.x];
    base_f = m.scan_sums[2 * nb + 2 * blockIdx.x + 1];
  }
  static_assert(per == 4, "one int4 of each flag array per thread");
  const int base = blockIdx.x * kScanTile + threadIdx.x * per;
  int st[4] = {0, 0, 0, 0}, fk[4] = {0, 0, 0, 0};
  if (base + 4 <= T) {  // the tables are 16-byte aligned
    const int4 vs = *reinterpret_cast<const int4*>(m.is_start + base);
    const int4 vf = *reinterpret_cast<const int4*>(m.is_fork + base);
    st[0] = vs.x, st[1] = vs.y, st[2] = vs.z, st[3] = vs.w;
    fk[0] = vf.x, fk[1] = vf.y, fk[2] = vf.z, fk[3] = vf.w;
  } else {
#pragma unroll
    for (int i = 0; i < per; ++i)
      if (base + i < T) {
        st[i] = m.is_start[base + i];
        fk[i] = m.is_fork[base + i];
      }
  }
  const int a = st[0] + st[1] + st[2] + st[3], f = fk[0] + fk[1] + fk[2] + fk[3];
  int ta, tf;
  int ea = block_excl_scan(a, sh, &ta) + base_a;
  int ef = block_excl_scan(f, sh, &tf) + base_f;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    const int t = base + i;
    if (st[i]) m.seg_start[ea++] = t;
    if (fk[i]) {
      if (ef == max_forks) raise_error(m.err, GDN_DEV_FORK_CAPACITY, t);
      m.fork_slot[t] = ef++;
    }
  }
}

// Entry token of segment j (the parent of its first token), or -1 when it
// starts from an initial state: a tree chunk always does, and invalid parents
// (already reported) are never followed.
__device__ inline int seg_entry_of(const int* parent, const int* seq_start, const Meta& m, int start, int* seq,
                                   int* mode) {
  const int s = m.tok_seq[start];
  const int md = (seq_start[s + 1] - seq_start[s]) <= kChunk ? 1 : 0;
  int e = md ? -1 : parent[start];
  if (e < 0 || e >= start) e = -1;
  *seq = s;
  *mode = md;
  return e;
}

// Thread i takes segment i: its table row, then its dependency level (the
// number of forks on the way to an initial state, each hop found by a binary
// search of the segment starts) and the level's counts.
__global__ void k_seglev(const int* parent, const int* seq_start, int T, int max_levels, Meta m) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int n_seg = *m.n_seg;
  if (i >= n_seg || bad_csr(m)) return;
  const int start = m.seg_start[i];
  const int end = (i + 1 < n_seg) ? m.seg_start[i + 1] : T;
  int sq, mode;
  const int e0 = seg_entry_of(parent, seq_start, m, start, &sq, &mode);
  m.seg_len[i] = end - start;
  m.seg_seq[i] = sq;
  m.seg_mode[i] = mode;
  m.seg_entry[i] = e0;
  m.seg_slot[i] = (e0 >= 0) ? m.fork_slot[e0] : -1;
  int lv = 0, d = 0, e = e0;
  while (e >= 0) {
    if (lv + 1 >= max_levels) {
      raise_error(m.err, GDN_DEV_LEVEL_CAPACITY, start);
      lv = max_levels;
      break;
    }
    ++lv;
    const int j = seg_of(m.seg_start, n_seg, e);
    const int sj = m.seg_start[j];
    d += e - sj + 1;
    int sq_j, mode_j;
    e = seg_entry_of(parent, seq_start, m, sj, &sq_j, &mode_j);
  }
  m.seg_level[i] = lv;
  m.seg_depth0[i] = d;
  if (lv < max_levels) {
    atomicAdd(&m.level_count[lv], 1);
    const int nch = mode ? 1 : (end - start + kChunk - 1) / kChunk;
    atomicAdd(&m.level_bkt[lv * kLenBuckets + len_bucket(nch)], 1);
    atomicMin(&m.walk_ctr[lv * kSchedInts + kWalkQueues], nch);
    atomicMax(&m.walk_ctr[lv * kSchedInts + kWalkQueues + 1], nch);
  }
}

// Last launch of a plan. Blocks [0, gT) fill the level lists (thread i takes
// segment i; the level offsets are an exclusive scan of the level counts, formed
// by every block) and the depths of chain tokens (thread i takes token i);
// blocks from gT on take four tree sequences each, one per wave, for their
// depths and ancestor-or-self masks by pointer jumping (six rounds cover 64
// levels). Block 0 records the level offsets and the plan's fingerprint.
__global__ void __launch_bounds__(256) k_finish(const int* parent, const int* seq_start, int T, int n_seq,
                                                int max_levels, int gT, unsigned long long tag, Meta m) {
  __shared__ int sh[256];
  if ((int)blockIdx.x < gT) {
    extern __shared__ int lptr[];  // [max_levels + 1]
    int run = 0;
    for (int c = 0; c < max_levels; c += 256) {
      const int l = c + threadIdx.x;
      const int v = l < max_levels ? m.level_count[l] : 0;
      int tot;
      const int ex = block_excl_scan(v, sh, &tot);
      if (l < max_levels) lptr[l] = run + ex;
      run += tot;
    }
    if (threadIdx.x == 0) lptr[max_levels] = run;
    // offsets of the length buckets inside each level (one wave per level, one bucket per lane)
    __shared__ int s_bko[kBkoLevels][kLenBuckets];
    const bool bko = max_levels <= kBkoLevels;
    if (bko)
      for (int lv = threadIdx.x >> 6; lv < max_levels; lv += 4)
        s_bko[lv][threadIdx.x & 63] = wave_excl_scan(m.level_bkt[lv * kLenBuckets + (threadIdx.x & 63)]);
    __syncthreads();
    if (blockIdx.x == 0) {
      for (int l = threadIdx.x; l <= max_levels; l += 256) m.level_ptr[l] = lptr[l];
      if (threadIdx.x == 0) *m.plan_tag = tag;
    }
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < *m.n_seg) {
      const int lv = m.seg_level[i];
      if (lv < max_levels) {
        // longest first: the entries of longer buckets of the level come before
        const int nch = m.seg_mode[i] ? 1 : (m.seg_len[i] + kChunk - 1) / kChunk;
        const int bk = len_bucket(nch);
        int pos = lptr[lv];
        if (bko) {
          pos += s_bko[lv][bk];
        } else {
          const int* cnt = m.level_bkt + lv * kLenBuckets;
          for (int b = 0; b < bk; ++b) pos += cnt[b];
        }
        pos += atomicAdd(&m.level_fill[lv * kLenBuckets + bk], 1);
        m.level_items[pos] = i;
        m.unit_info[pos] = make_int4(m.seg_start[i], m.seg_len[i], m.seg_mode[i] | (m.seg_seq[i] << 1),
                                                m.seg_slot[i]);
      }
    }
    if (i < T && !bad_csr(m)) {
      const int s = m.tok_seq[i];
      if (seq_start[s + 1] - seq_start[s] > kChunk) {  // tree chunks: below
        const int j = seg_of(m.seg_start, *m.n_seg, i);
        m.depth[i] = m.seg_depth0[j] + (i - m.seg_start[j]);
      }
    }
    return;
  }
  const int s = ((int)blockIdx.x - gT) * 4 + (int)(threadIdx.x >> 6);
  if (s >= n_seq || bad_csr(m)) return;
  const int a = seq_start[s], n = seq_start[s + 1] - a;
  if (n <= 0 || n > kChunk) return;
  const int i = threadIdx.x & 63;
  int p = -1;
  if (i < n) {
    const int g = parent[a + i];
    p = (g >= a && g < a + i) ? g - a : -1;
  }
  unsigned long long anc = (i < n) ? (1ull << i) : 0ull;
  int d = (p >= 0) ? 1 : 0;
  for (int r = 0; r < 6; ++r) {
    const int src = p >= 0 ? p : i;
    const unsigned long long panc = __shfl(anc, src);
    const int pd = __shfl(d, src);
    const int pp = __shfl(p, src);
    if (p >= 0) {
      anc |= panc;
      d += pd;
      p = pp;
    }
  }
  if (i < n) {
    m.tree_mask[(size_t)s * kChunk + i] = anc;
    m.depth[a + i] = d;
  }
}

// ---- the whole plan in one workgroup, for short streams
//
// The six launches above each cost a few microseconds even when their work is
// tiny. For a stream of at most kSmallPlanT tokens one workgroup of 1024
// threads runs the same steps in the same order, separated by workgroup
// barriers, and writes the same tables (each step's rules are those of the
// launch it replaces). Measured on an MI355X: 64 draft trees of 64 tokens plan
// in about 7 us less than with six launches; 16384 tokens take longer in one
// workgroup than in six launches, hence the bound.

constexpr int kSmallPlanT = 4096;

__device__ inline int ld_l2(const int* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
constexpr int kPT = 1024;  // threads of the one workgroup

// Exclusive scan over the workgroup (wave scans, then a scan of the 16 wave totals).
__device__ inline int wg_excl_scan(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[w] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int k = 0; k < kPT / 64; ++k) {
      const int t = sh[k];
      sh[k] = run;
      run += t;
    }
    sh[kPT / 64] = run;
  }
  __syncthreads();
  const int r = sh[w] + x - v;
  *total = sh[kPT / 64];
  __syncthreads();
  return r;
}

// Sequence starts and segment starts are kept in LDS when they fit, so the
// binary searches of the token steps do not wait on global memory; token loops
// issue four tokens' loads before using any of them.
constexpr int kSeqLds = 2048;  // sequence starts held in LDS (n_seq + 1 entries)
constexpr int kSegLds = 4096;  // segment starts held in LDS
static_assert(kSegLds <= kSmallPlanT, "segment starts share the short path's buffer");

// ---- streams of short sequences (draft trees)
//
// When every sequence holds at most 64 tokens, each one is a single tree chunk:
// one segment per non-empty sequence, in stream order, all at level 0, no fork
// tokens and no fork slots. The tables then follow from each sequence's bounds
// and parents alone, and only the row maps need two passes (map, then the
// check for repeats). The tables are those the general steps write for such a
// stream, except the planner's own start and fork flags, which only its
// general steps read. Everything is formed from one round of loads; threads
// exchange data through LDS only, so the barriers wait for LDS traffic alone
// and never for the global stores in flight, and the first error is kept in
// LDS and stored at the end. (Stage stamps on an MI355X, 64 trees of 64
// tokens: with ordinary barriers, per-token sequence lookups and a mask pass of
// its own, the barriers waited about 1.5 us for stores, and the lookups and the
// mask pass took 2.2 and 4 us.)
__device__ inline void lds_raise(unsigned long long* e, int code, long long index) {
  atomicMin(e, ((unsigned long long)(unsigned)code << 32) | (unsigned long long)(uint32_t)index);
}

// Workgroup barrier that orders LDS traffic only (global stores stay in flight).
__device__ inline void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Exclusive scan over the workgroup with LDS-only barriers.
__device__ inline int short_scan(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[w] = x;
  lds_sync();
  int base = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < kPT / 64; ++k) {
    const int c = sh[k];
    base += k < w ? c : 0;
    tot += c;
  }
  *total = tot;
  return base + x - v;
}

constexpr int kShortPer = kSmallPlanT / kPT;  // tokens (and rows) per thread

// The short path's loads, issued at the kernel's start right after those of
// seq_start: the parents of tokens tid + u kPT and the rows at those positions.
struct ShortLoads {
  int pv[kShortPer], ro[kShortPer], rs[kShortPer];
};

__device__ inline ShortLoads short_loads(const int* parent, int T, const int* out_rows, int n_out, const int* state_rows,
                                         int n_state) {
  ShortLoads L;
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < kShortPer; ++u) {
    const int i = tid + u * kPT;
    L.pv[u] = i < T ? parent[i] : -1;
    L.ro[u] = (out_rows && i < n_out) ? out_rows[i] : -1;
    L.rs[u] = (state_rows && i < n_state) ? state_rows[i] : -1;
  }
  return L;
}

__device__ void plan_short(const ShortLoads& L, const int* ss, int n_seq, int T, bool no_empty, const int* out_rows,
                           int n_out, const int* state_rows, int n_state, int max_levels, unsigned long long tag,
                           const Meta& m, int* s_out, int* s_st, int* s_par, int* sh, unsigned long long* s_err) {
  const int tid = threadIdx.x, lane = tid & 63;
  constexpr int kPer = kShortPer;
  constexpr int kW = kPT / 64;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int t = tid + u * kPT;
    if (t < T) {
      s_par[t] = L.pv[u];
      s_out[t] = kUnmapped;
      s_st[t] = kUnmapped;
    }
  }
  if (tid == 0) *s_err = kNoError;
  lds_sync();
  // requested rows: the first position asking for a token owns it
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = tid + u * kPT;
    if (out_rows && i < n_out) {
      if (L.ro[u] < 0 || L.ro[u] >= T) lds_raise(s_err, GDN_DEV_ROWS, i);
      else atomicMin(&s_out[L.ro[u]], i);
    }
    if (state_rows && i < n_state) {
      if (L.rs[u] < 0 || L.rs[u] >= T) lds_raise(s_err, GDN_DEV_ROWS, i);
      else atomicMin(&s_st[L.rs[u]], i);
    }
  }
  if (out_rows)
    for (int i = tid + kPer * kPT; i < n_out; i += kPT) {
      const int r = out_rows[i];
      if (r < 0 || r >= T) lds_raise(s_err, GDN_DEV_ROWS, i);
      else atomicMin(&s_out[r], i);
    }
  if (state_rows)
    for (int i = tid + kPer * kPT; i < n_state; i += kPT) {
      const int r = state_rows[i];
      if (r < 0 || r >= T) lds_raise(s_err, GDN_DEV_ROWS, i);
      else atomicMin(&s_st[r], i);
    }
  // one wave per sequence, four sequences of a wave at a time: the token
  // tables, the parent checks, and the ancestor-or-self masks and depths by
  // pointer jumping (the four sequences' shuffles overlap; the jumps stop once
  // every token has reached its root)
  for (int s0 = tid >> 6; s0 < n_seq; s0 += 4 * kW) {
    int a[4], n[4], p[4];
    unsigned long long anc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sq = s0 + u * kW;
      a[u] = 0;
      n[u] = 0;
      if (sq < n_seq) {
        a[u] = ss[sq];
        n[u] = ss[sq + 1] - a[u];
      }
      p[u] = -1;
      if (lane < n[u]) {
        const int t = a[u] + lane;
        const int g = s_par[t];
        if (g < -1 || g >= t) lds_raise(s_err, GDN_DEV_PARENT_ORDER, t);
        else if (g >= 0 && g < a[u]) lds_raise(s_err, GDN_DEV_PARENT_SEQ, t);
        p[u] = (g >= a[u] && g < t) ? g - a[u] : -1;
        m.tok_seq[t] = sq;
        m.fork_slot[t] = -1;
      }
      anc[u] = (lane < n[u]) ? (1ull << lane) : 0ull;
    }
    for (int r = 0; r < 6; ++r) {
      if (!__any(p[0] >= 0 || p[1] >= 0 || p[2] >= 0 || p[3] >= 0)) break;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int src = p[u] >= 0 ? p[u] : lane;
        const unsigned long long panc = __shfl(anc[u], src);
        const int pp = __shfl(p[u], src);
        if (p[u] >= 0) {
          anc[u] |= panc;
          p[u] = pp;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sq = s0 + u * kW;
      if (sq >= n_seq) break;
      m.tree_mask[(size_t)sq * kChunk + lane] = anc[u];
      if (lane < n[u]) m.depth[a[u] + lane] = __popcll(anc[u]) - 1;  // ancestors in the chunk
    }
  }
  // segments: the non-empty sequences in order (two sequences per thread),
  // numbered by a scan unless no sequence is empty; the barrier (the scan's
  // own, or one of its own) orders the row atomics before the checks below
  int ne0 = 0, ne1 = 0;
  const int s0 = 2 * tid;
  if (s0 < n_seq) ne0 = ss[s0 + 1] > ss[s0];
  if (s0 + 1 < n_seq) ne1 = ss[s0 + 2] > ss[s0 + 1];
  int n_seg = n_seq, e = s0;
  if (no_empty) lds_sync();
  else e = short_scan(ne0 + ne1, sh, &n_seg);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int sq = s0 + u;
    if (!(u ? ne1 : ne0)) continue;
    const int i = e + (u ? ne0 : 0);
    const int a = ss[sq], n = ss[sq + 1] - a;
    m.seg_start[i] = a;
    m.seg_len[i] = n;
    m.seg_seq[i] = sq;
    m.seg_mode[i] = 1;
    m.seg_entry[i] = -1;
    m.seg_slot[i] = -1;
    m.seg_level[i] = 0;
    m.seg_depth0[i] = 0;
    m.level_items[i] = i;
    m.unit_info[i] = make_int4(a, n, 1 | (sq << 1), -1);
  }
  // repeats among the requested rows, and the row maps
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = tid + u * kPT;
    if (out_rows && i < n_out && L.ro[u] >= 0 && L.ro[u] < T && s_out[L.ro[u]] != i) lds_raise(s_err, GDN_DEV_ROWS, i);
    if (state_rows && i < n_state && L.rs[u] >= 0 && L.rs[u] < T && s_st[L.rs[u]] != i)
      lds_raise(s_err, GDN_DEV_ROWS, i);
  }
  if (out_rows)
    for (int i = tid + kPer * kPT; i < n_out; i += kPT) {
      const int r = out_rows[i];
      if (r >= 0 && r < T && s_out[r] != i) lds_raise(s_err, GDN_DEV_ROWS, i);
    }
  if (state_rows)
    for (int i = tid + kPer * kPT; i < n_state; i += kPT) {
      const int r = state_rows[i];
      if (r >= 0 && r < T && s_st[r] != i) lds_raise(s_err, GDN_DEV_ROWS, i);
    }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int t = tid + u * kPT;
    if (t < T) {
      m.out_map[t] = s_out[t];
      m.state_map[t] = s_st[t];
    }
  }
  // levels: every segment at level 0 and one chunk long
  const int one = len_bucket(1);
  for (int l = tid; l <= max_levels; l += kPT) {
    m.level_ptr[l] = l == 0 ? 0 : n_seg;
    if (l < max_levels) m.level_count[l] = l == 0 ? n_seg : 0;
  }
  for (int i = tid; i < max_levels * kLenBuckets; i += kPT) {
    const int v = (i == one) ? n_seg : 0;  // level 0, bucket of one chunk
    m.level_bkt[i] = v;
    m.level_fill[i] = v;
  }
  for (int i = tid; i < max_levels * kSchedInts; i += kPT) {
    const int q = i % kSchedInts;
    const bool used = i < kSchedInts && n_seg > 0;
    m.walk_ctr[i] = q < kWalkQueues ? 0 : q == kWalkQueues ? (used ? 1 : 0x7fffffff) : (used ? 1 : 0);
  }
  lds_sync();  // every error raised
  if (tid == 0) {
    *m.err = *s_err;
    *m.n_seg = n_seg;
    *m.n_fork = 0;
    *m.plan_tag = tag;
  }
}

__global__ void __launch_bounds__(kPT) k_plan_small(const int* parent, const int* seq_start, int n_seq, int T,
                                                    const int* out_rows, int n_out, const int* state_rows, int n_state,
                                                    int max_forks, int max_levels, unsigned long long tag, Meta m) {
  __shared__ int sh[kPT / 64 + 1];
  __shared__ int s_ss[kSeqLds + 1];
  __shared__ int s_big[3 * kSmallPlanT];  // segment starts; on the short path the row maps and the parents
  __shared__ unsigned long long s_err;
  __shared__ int s_flag;
  int* s_seg = s_big;
  const int tid = threadIdx.x;
  const bool ss_lds = n_seq <= kSeqLds;
  const int* ss = ss_lds ? s_ss : seq_start;
  if (ss_lds) {
    // seq_start first, then the short path's loads, so that the wait for the
    // former does not include the latter
    int sv[kSeqLds / kPT + 1];
#pragma unroll
    for (int k = 0; k <= kSeqLds / kPT; ++k) {
      const int i = tid + k * kPT;
      sv[k] = i <= n_seq ? seq_start[i] : 0;
    }
    const ShortLoads sl = short_loads(parent, T, out_rows, n_out, state_rows, n_state);
#pragma unroll
    for (int k = 0; k <= kSeqLds / kPT; ++k) {
      const int i = tid + k * kPT;
      if (i <= n_seq) s_ss[i] = sv[k];
    }
    if (tid == 0) s_flag = 3;
    lds_sync();
    // a valid seq_start whose sequences all fit one chunk takes the short path
    // (bit 0 of the flag), noting whether some sequence is empty (bit 1 clear)
    int ok = 1, full = 1;
    for (int s = tid; s <= n_seq; s += kPT) {
      const int v = s_ss[s];
      if (s == 0 ? v != 0 : (v < s_ss[s - 1] || v > T || v - s_ss[s - 1] > kChunk)) ok = 0;
      if (s == n_seq && v != T) ok = 0;
      if (s > 0 && v == s_ss[s - 1]) full = 0;
    }
    if (!ok) atomicAnd(&s_flag, ~1);
    if (!full) atomicAnd(&s_flag, ~2);
    lds_sync();
    const int flag = s_flag;
    if (flag & 1) {
      plan_short(sl, s_ss, n_seq, T, (flag & 2) != 0, out_rows, n_out, state_rows, n_state, max_levels, tag, m, s_big,
                 s_big + kSmallPlanT, s_big + 2 * kSmallPlanT, sh, &s_err);
      return;
    }
  }
  // -- clear (as k_init)
  for (int i = tid; i < T; i += kPT) {
    m.tok_seq[i] = 0;
    m.out_map[i] = kUnmapped;
    m.state_map[i] = kUnmapped;
    m.is_fork[i] = 0;
    m.is_start[i] = 0;
    m.fork_slot[i] = -1;
    m.depth[i] = 0;
  }
  for (int i = tid; i < n_seq * kChunk; i += kPT) m.tree_mask[i] = 0ull;
  for (int i = tid; i < max_levels; i += kPT) m.level_count[i] = 0;
  for (int i = tid; i < max_levels * kLenBuckets; i += kPT) {
    m.level_fill[i] = 0;
    m.level_bkt[i] = 0;
  }
  for (int i = tid; i < max_levels * kSchedInts; i += kPT) m.walk_ctr[i] = (i % kSchedInts) == kWalkQueues ? 0x7fffffff : 0;
  if (tid == 0) {
    *m.err = kNoError;
    *m.n_seg = 0;
    *m.n_fork = 0;
    *m.plan_tag = 0ull;
  }
  __syncthreads();
  // -- sequence checks, row maps, per-token checks, segment starts and fork flags (as k_tokens)
  for (int s = tid; s <= n_seq; s += kPT) {
    const int v = ss[s];
    if (s == 0 && v != 0) {
      raise_error(m.err, GDN_DEV_SEQ_START, 0);
    } else if (s > 0 && (v < ss[s - 1] || v > T)) {
      raise_error(m.err, GDN_DEV_SEQ_START, s);
    } else if (s == n_seq && v != T) {
      raise_error(m.err, GDN_DEV_SEQ_START, s);
    }
  }
  if (out_rows)
    for (int i = tid; i < n_out; i += kPT) map_row(out_rows, n_out, i, T, m.out_map, m.err);
  if (state_rows)
    for (int i = tid; i < n_state; i += kPT) map_row(state_rows, n_state, i, T, m.state_map, m.err);
  for (int t0 = tid; t0 < T; t0 += 4 * kPT) {
    int pv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + u * kPT;
      pv[u] = t < T ? parent[t] : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + u * kPT;
      if (t >= T) break;
      const int s = upper_bound_seq(ss, n_seq, t);
      m.tok_seq[t] = s;
      const int a = ss[s], b = ss[s + 1];
      const bool tree = (b - a) <= kChunk;
      const int p = pv[u];
      bool ok = true;
      if (p < -1 || p >= t) {
        raise_error(m.err, GDN_DEV_PARENT_ORDER, t);
        ok = false;
      } else if (p >= 0 && p < a) {
        raise_error(m.err, GDN_DEV_PARENT_SEQ, t);
        ok = false;
      }
      const int start = tree ? (t == a) : (p < 0 || p != t - 1);
      m.is_start[t] = start;
      if (!tree && start && ok && p >= 0) m.is_fork[p] = 1;
    }
  }
  __syncthreads();
  // -- distinct rows (as k_scan_reduce). Values that atomics formed are read
  //    with atomic loads: atomics complete in L2, and a plain load could hit an
  //    older copy in this CU's L1.
  if (out_rows)
    for (int i = tid; i < n_out; i += kPT) {
      const int r = out_rows[i];
      if (r >= 0 && r < T && ld_l2(m.out_map + r) != i) raise_error(m.err, GDN_DEV_ROWS, i);
    }
  if (state_rows)
    for (int i = tid; i < n_state; i += kPT) {
      const int r = state_rows[i];
      if (r >= 0 && r < T && ld_l2(m.state_map + r) != i) raise_error(m.err, GDN_DEV_ROWS, i);
    }
  // -- segment and fork-slot numbering (as k_scan_apply): thread k takes the
  //    tokens [k c, k c + c), c a multiple of 4 (at most 32), read as 16-byte loads
  {
    constexpr int kMaxPer = kSmallPlanT / kPT;
    const int c = ((T + 4 * kPT - 1) / (4 * kPT)) * 4;
    const int t0 = tid * c;
    int st[kMaxPer], fk[kMaxPer];
#pragma unroll
    for (int q = 0; q < kMaxPer; q += 4) {
      int4 vs = make_int4(0, 0, 0, 0), vf = make_int4(0, 0, 0, 0);
      const int t = t0 + q;
      if (q < c) {
        if (t + 4 <= T) {
          vs = *reinterpret_cast<const int4*>(m.is_start + t);
          vf = *reinterpret_cast<const int4*>(m.is_fork + t);
        } else {
          if (t + 0 < T) vs.x = m.is_start[t + 0], vf.x = m.is_fork[t + 0];
          if (t + 1 < T) vs.y = m.is_start[t + 1], vf.y = m.is_fork[t + 1];
          if (t + 2 < T) vs.z = m.is_start[t + 2], vf.z = m.is_fork[t + 2];
        }
      }
      st[q] = vs.x, st[q + 1] = vs.y, st[q + 2] = vs.z, st[q + 3] = vs.w;
      fk[q] = vf.x, fk[q + 1] = vf.y, fk[q + 2] = vf.z, fk[q + 3] = vf.w;
    }
    int na = 0, nf = 0;
#pragma unroll
    for (int q = 0; q < kMaxPer; ++q) {
      na += st[q];
      nf += fk[q];
    }
    int ta, tf;
    int ea = wg_excl_scan(na, sh, &ta);
    int ef = wg_excl_scan(nf, sh, &tf);
#pragma unroll
    for (int q = 0; q < kMaxPer; ++q) {
      const int t = t0 + q;
      if (st[q]) {
        m.seg_start[ea] = t;
        if (ea < kSegLds) s_seg[ea] = t;
        ++ea;
      }
      if (fk[q]) {
        if (ef == max_forks) raise_error(m.err, GDN_DEV_FORK_CAPACITY, t);
        m.fork_slot[t] = ef++;
      }
    }
    if (tid == 0) {
      *m.n_seg = ta;
      *m.n_fork = tf;
    }
    __syncthreads();
  }
  // -- segment table and dependency levels (as k_seglev)
  const int n_seg = *m.n_seg;
  const int* segs = n_seg <= kSegLds ? s_seg : m.seg_start;
  const bool bad = (__hip_atomic_load(m.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 32) ==
                   (unsigned long long)GDN_DEV_SEQ_START;
  if (!bad) {
    for (int i = tid; i < n_seg; i += kPT) {
      const int start = segs[i];
      const int end = (i + 1 < n_seg) ? segs[i + 1] : T;
      int sq, mode;
      const int e0 = seg_entry_of(parent, ss, m, start, &sq, &mode);
      m.seg_len[i] = end - start;
      m.seg_seq[i] = sq;
      m.seg_mode[i] = mode;
      m.seg_entry[i] = e0;
      m.seg_slot[i] = (e0 >= 0) ? m.fork_slot[e0] : -1;
      int lv = 0, d = 0, e = e0;
      while (e >= 0) {
        if (lv + 1 >= max_levels) {
          raise_error(m.err, GDN_DEV_LEVEL_CAPACITY, start);
          lv = max_levels;
          break;
        }
        ++lv;
        const int j = seg_of(segs, n_seg, e);
        const int sj = segs[j];
        d += e - sj + 1;
        int sq_j, mode_j;
        e = seg_entry_of(parent, ss, m, sj, &sq_j, &mode_j);
      }
      m.seg_level[i] = lv;
      m.seg_depth0[i] = d;
      if (lv < max_levels) {
        atomicAdd(&m.level_count[lv], 1);
        const int nch = mode ? 1 : (end - start + kChunk - 1) / kChunk;
        atomicAdd(&m.level_bkt[lv * kLenBuckets + len_bucket(nch)], 1);
        atomicMin(&m.walk_ctr[lv * kSchedInts + kWalkQueues], nch);
        atomicMax(&m.walk_ctr[lv * kSchedInts + kWalkQueues + 1], nch);
      }
    }
  }
  __syncthreads();
  // -- level offsets, level lists longest first, depths and tree masks (as k_finish)
  if (tid == 0) {
    int run = 0;
    for (int l = 0; l < max_levels; ++l) {
      m.level_ptr[l] = run;
      run += ld_l2(m.level_count + l);
    }
    m.level_ptr[max_levels] = run;
    *m.plan_tag = tag;
  }
  // offsets of the length buckets inside each level (wave w: level w, one bucket per lane)
  __shared__ int s_bko[kBkoLevels][kLenBuckets];
  const bool bko = max_levels <= kBkoLevels;
  if (bko && (tid >> 6) < max_levels) {
    const int lv = tid >> 6, b = tid & 63;
    s_bko[lv][b] = wave_excl_scan(ld_l2(m.level_bkt + lv * kLenBuckets + b));
  }
  __syncthreads();
  if (!bad) {
    for (int i = tid; i < n_seg; i += kPT) {
      const int lv = m.seg_level[i];
      if (lv < max_levels) {
        const int nch = m.seg_mode[i] ? 1 : (m.seg_len[i] + kChunk - 1) / kChunk;
        const int bk = len_bucket(nch);
        int pos = m.level_ptr[lv];
        if (bko) {
          pos += s_bko[lv][bk];
        } else {
          const int* cnt = m.level_bkt + lv * kLenBuckets;
          for (int b = 0; b < bk; ++b) pos += ld_l2(cnt + b);
        }
        pos += atomicAdd(&m.level_fill[lv * kLenBuckets + bk], 1);
        m.level_items[pos] = i;
        m.unit_info[pos] = make_int4(segs[i], m.seg_len[i], m.seg_mode[i] | (m.seg_seq[i] << 1), m.seg_slot[i]);
      }
    }
    for (int t0 = tid; t0 < T; t0 += 4 * kPT) {
      int sv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = t0 + u * kPT;
        sv[u] = t < T ? m.tok_seq[t] : 0;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = t0 + u * kPT;
        if (t < T && ss[sv[u] + 1] - ss[sv[u]] > kChunk) {
          const int j = seg_of(segs, n_seg, t);
          m.depth[t] = m.seg_depth0[j] + (t - segs[j]);
        }
      }
    }
    const int lane = tid & 63;
    // four sequences per wave and round: their parents are loaded before any is used
    for (int s0 = tid >> 6; s0 < n_seq; s0 += 4 * (kPT / 64)) {
      int gp[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int s = s0 + u * (kPT / 64);
        gp[u] = -1;
        if (s < n_seq) {
          const int a = ss[s], n = ss[s + 1] - a;
          if (n > 0 && n <= kChunk && lane < n) gp[u] = parent[a + lane];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
      const int s = s0 + u * (kPT / 64);
      if (s >= n_seq) break;
      const int a = ss[s], n = ss[s + 1] - a;
      if (n <= 0 || n > kChunk) continue;
      int p = -1;
      if (lane < n) {
        const int g = gp[u];
        p = (g >= a && g < a + lane) ? g - a : -1;
      }
      unsigned long long anc = (lane < n) ? (1ull << lane) : 0ull;
      int d = (p >= 0) ? 1 : 0;
      for (int r = 0; r < 6; ++r) {
        const int src = p >= 0 ? p : lane;
        const unsigned long long panc = __shfl(anc, src);
        const int pd = __shfl(d, src);
        const int pp = __shfl(p, src);
        if (p >= 0) {
          anc |= panc;
          d += pd;
          p = pp;
        }
      }
      if (lane < n) {
        m.tree_mask[(size_t)s * kChunk + lane] = anc;
        m.depth[a + lane] = d;
      }
      }
    }
  }
}

inline int blocks_for(long long n, int bs) { return (int)((n + bs - 1) / bs); }

}  // namespace

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool compute_layout(const gdn_tree_dims& d, LayoutFull* L) {
  if (d.T < 0 || d.T > 0x7fffffff || d.n_seq < 0 || d.max_forks < 0 || d.max_levels < 1) return false;
  size_t T = (size_t)d.T;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  gdn_tree_layout& p = L->pub;
  p.err = take(8);
  p.n_seg = take(4);
  p.n_fork = take(4);
  p.tok_seq = take(4 * T);
  p.depth = take(4 * T);
  p.fork_slot = take(4 * T);
  p.seg_start = take(4 * T);
  p.seg_len = take(4 * T);
  p.seg_seq = take(4 * T);
  p.seg_mode = take(4 * T);
  p.seg_entry = take(4 * T);
  p.seg_slot = take(4 * T);
  p.seg_level = take(4 * T);
  p.level_count = take(4 * (size_t)d.max_levels);
  p.level_ptr = take(4 * ((size_t)d.max_levels + 1));
  p.level_items = take(4 * T);
  p.tree_mask = take(8 * (size_t)d.n_seq * kChunk);
  L->is_start = take(4 * T);
  L->is_fork = take(4 * T);
  L->out_map = take(4 * T);
  L->state_map = take(4 * T);
  L->seg_depth0 = take(4 * T);
  L->level_fill = take(4 * (size_t)d.max_levels * kLenBuckets);
  L->level_bkt = take(4 * (size_t)d.max_levels * kLenBuckets);
  L->walk_ctr = take(4 * (size_t)d.max_levels * kSchedInts);
  L->n_scan_blocks = (int)((T + kScanTile - 1) / kScanTile);
  if (L->n_scan_blocks < 1) L->n_scan_blocks = 1;
  L->scan_sums = take(4 * 4 * (size_t)L->n_scan_blocks);
  L->plan_tag = take(8);
  L->unit_info = take(16 * T);
  size_t state_elems = (size_t)d.H * d.Dv * d.Dk;
  p.fork_states = take(4 * state_elems * (size_t)d.max_forks);
  p.total = off;
  return true;
}

Meta meta_from(void* ws, const LayoutFull& L) {
  char* b = (char*)ws;
  const gdn_tree_layout& p = L.pub;
  Meta m;
  m.err = (unsigned long long*)(b + p.err);
  m.n_seg = (int*)(b + p.n_seg);
  m.n_fork = (int*)(b + p.n_fork);
  m.tok_seq = (int*)(b + p.tok_seq);
  m.depth = (int*)(b + p.depth);
  m.fork_slot = (int*)(b + p.fork_slot);
  m.seg_start = (int*)(b + p.seg_start);
  m.seg_len = (int*)(b + p.seg_len);
  m.seg_seq = (int*)(b + p.seg_seq);
  m.seg_mode = (int*)(b + p.seg_mode);
  m.seg_entry = (int*)(b + p.seg_entry);
  m.seg_slot = (int*)(b + p.seg_slot);
  m.seg_level = (int*)(b + p.seg_level);
  m.level_count = (int*)(b + p.level_count);
  m.level_ptr = (int*)(b + p.level_ptr);
  m.level_items = (int*)(b + p.level_items);
  m.tree_mask = (unsigned long long*)(b + p.tree_mask);
  m.fork_states = (float*)(b + p.fork_states);
  m.is_start = (int*)(b + L.is_start);
  m.is_fork = (int*)(b + L.is_fork);
  m.out_map = (int*)(b + L.out_map);
  m.state_map = (int*)(b + L.state_map);
  m.seg_depth0 = (int*)(b + L.seg_depth0);
  m.level_fill = (int*)(b + L.level_fill);
  m.level_bkt = (int*)(b + L.level_bkt);
  m.walk_ctr = (int*)(b + L.walk_ctr);
  m.scan_sums = (int*)(b + L.scan_sums);
  m.plan_tag = (unsigned long long*)(b + L.plan_tag);
  m.unit_info = (int4*)(b + L.unit_info);
  return m;
}

unsigned long long plan_fingerprint(const gdn_tree_fwd_args& a) {
  // FNV-1a over the sizes the tables depend on
  const long long f[] = {a.dims.T, a.dims.H, a.dims.Dk, a.dims.Dv, a.dims.n_seq, a.dims.dtype, a.dims.max_forks,
                         a.dims.max_levels, a.n_out, a.n_state, a.out_rows != nullptr, a.state_rows != nullptr};
  unsigned long long h = 1469598103934665603ull;
  for (long long x : f) {
    for (int b = 0; b < 8; ++b) {
      h ^= (unsigned long long)((x >> (8 * b)) & 0xff);
      h *= 1099511628211ull;
    }
  }
  return h ? h : 1ull;
}

hipError_t launch_replan_check(const Meta& m, int max_levels, unsigned long long tag, hipStream_t s) {
  hipLaunchKernelGGL(k_replan_check, dim3(1), dim3(256), 0, s, m, max_levels, tag);
  return hipGetLastError();
}

hipError_t launch_plan(const gdn_tree_fwd_args& a, const Meta& m, const LayoutFull& L, unsigned long long tag,
                       hipStream_t s) {
  const int T = (int)a.dims.T, n_seq = a.dims.n_seq, ml = a.dims.max_levels;
  const int bs = 256;
  long long init_n = T;
  if ((long long)n_seq * kChunk > init_n) init_n = (long long)n_seq * kChunk;
  if ((long long)ml * kSchedInts > init_n) init_n = (long long)ml * kSchedInts;
  if ((long long)ml * kLenBuckets > init_n) init_n = (long long)ml * kLenBuckets;
  if (init_n < 1) init_n = 1;
  const int gT = blocks_for(T > 0 ? T : 1, bs);
  const int* out_rows = a.n_out > 0 ? a.out_rows : nullptr;
  const int* state_rows = a.n_state > 0 ? a.state_rows : nullptr;
  const long long n_rows = (out_rows ? a.n_out : 0) > (state_rows ? a.n_state : 0) ? (out_rows ? a.n_out : 0)
                                                                                     : (state_rows ? a.n_state : 0);
  if (T > 0 && n_seq > 0 && T <= kSmallPlanT) {
    hipLaunchKernelGGL(k_plan_small, dim3(1), dim3(kPT), 0, s, a.parent_idx, a.seq_start, n_seq, T, out_rows, a.n_out,
                       state_rows, a.n_state, a.dims.max_forks, ml, tag, m);
    return hipGetLastError();
  }
  long long tok_threads = (long long)T + n_rows;
  if (tok_threads < (long long)n_seq + 1) tok_threads = (long long)n_seq + 1;
  hipLaunchKernelGGL(k_init, dim3(blocks_for(init_n, bs)), dim3(bs), 0, s, m, T, n_seq, ml);
  hipLaunchKernelGGL(k_tokens, dim3(blocks_for(tok_threads, bs)), dim3(bs), 0, s, a.parent_idx, a.seq_start, n_seq, T,
                     out_rows, a.n_out, state_rows, a.n_state, m);
  const int nb = L.n_scan_blocks;
  const int row_blocks = blocks_for(n_rows, bs);
  const bool work = T > 0 && n_seq > 0;
  if (work || row_blocks > 0)
    hipLaunchKernelGGL(k_scan_reduce, dim3((work ? nb : 0) + row_blocks), dim3(256), 0, s, T, out_rows, a.n_out,
                       state_rows, a.n_state, row_blocks, m);
  if (work) {
    if (nb <= 1024) {
      hipLaunchKernelGGL(k_scan_apply<true>, dim3(nb), dim3(256), 0, s, T, nb, a.dims.max_forks, m);
    } else {
      hipLaunchKernelGGL(k_scan_top, dim3(1), dim3(256), 0, s, nb, m);
      hipLaunchKernelGGL(k_scan_apply<false>, dim3(nb), dim3(256), 0, s, T, nb, a.dims.max_forks, m);
    }
    hipLaunchKernelGGL(k_seglev, dim3(gT), dim3(bs), 0, s, a.parent_idx, a.seq_start, T, ml, m);
  }
  const int tree_blocks = work ? blocks_for(n_seq, 4) : 0;
  hipLaunchKernelGGL(k_finish, dim3(gT + tree_blocks), dim3(bs), 4 * (ml + 1), s, a.parent_idx, a.seq_start, T, n_seq,
                     ml, gT, tag, m);
  return hipGetLastError();
}

}  // namespace gdn
