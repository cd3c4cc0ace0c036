/*
 * gdn_tree — the gated delta rule over a tree-structured flat token stream,
 * on AMD Instinct MI355X (gfx950).
 *
 * What is computed. Every token t of the stream names its parent p(t): a
 * smaller index in the same sequence, or -1 for the sequence's initial state.
 * With S in R^{Dv x Dk} (TreeWY, "Speculative Verification for Gated DeltaNet
 * Hybrids", section 1 "Hybrid models and GDN layers", Eq. 1):
 *
 *     S_t = alpha_t S_{p(t)} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t,          alpha_t = exp(log_gate_t),
 *
 * so a question branch (Flide, "Accelerating Decision Inference with Exact
 * State Forking", section 3.2.3) or a draft-tree node (TreeWY section 3
 * "Verifying a draft") restarts from the exact state of its trunk inside the
 * same pass. The pseudo-value vt_t = beta_t (v_t - alpha_t S_{p(t)} k_t)
 * (TreeWY section 3 "Key rewrite") can be kept, and gdn_tree_commit rebuilds
 * the state after any node a from it (TreeWY section 3 "Reconstruct on
 * commit", Eq. 3):
 *
 *     S_a = g_a S_0 + sum over i ancestor-or-self of a of (g_a / g_i) vt_i k_i^T,
 *
 * with g_x the product of alpha over the root path of x, x included.
 *
 * Conventions for every call:
 *  - Pointers to tensors are DEVICE pointers; structs and scalars are host
 *    memory. Layouts are row-major and token-major: q, k [T, H, Dk];
 *    v, out, pseudo_v [T, H, Dv] (out: [n_out, H, Dv] when out_rows is given);
 *    log_gate, beta [T, H]; states [.., H, Dv, Dk] fp32.
 *  - `stream` is a hipStream_t (NULL = the null stream). Calls only enqueue
 *    work; they return before it runs and never synchronise, except
 *    gdn_tree_check_error.
 *  - gdn_tree_forward, gdn_tree_plan and gdn_tree_commit enqueue kernel
 *    launches only (no memset, copy or allocation), and their launch shapes
 *    depend on the sizes and capacities in the arguments, never on the tree.
 *    They can therefore be captured once in a HIP graph and replayed for any
 *    tree that fits the same sizes and capacities (Flide section 3.3 replays
 *    one flat graph per capacity bucket this way): the metadata is rebuilt
 *    from parent_idx on every replay.
 *  - The caller owns every buffer, the workspace included, and keeps them
 *    alive until the stream has passed the call. The library allocates no
 *    device memory. Its global state is a thread-local text for the last host
 *    error, per-device caches of the CU count and kernel attributes, and the
 *    static workspace of gdn_tree_forward_static (below). Calls on different
 *    streams with different workspaces may overlap.
 *  - Return value: GDN_OK or a negative gdn_status found synchronously on the
 *    host (nothing is enqueued then). Structural problems of the tree are
 *    found on the device: the kernels record the smallest (code, index) in the
 *    workspace's error word, skip their work, and never fault;
 *    gdn_tree_check_error reads that word.
 */
#ifndef GDN_TREE_H
#define GDN_TREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_TREE_VERSION 1
#define GDN_TREE_CHUNK 64 /* chunk length of the tree-WY walk (fixed: it fixes the bits) */

typedef enum gdn_dtype {
  GDN_F32 = 0,  /* q, k, v, log_gate, beta and out in fp32 */
  GDN_BF16 = 1, /* q, k, v, log_gate, beta and out in bf16 (states stay fp32) */
} gdn_dtype;

/* Forward flags.
 * GDN_FWD_PLANNED: the workspace already holds the metadata that
 *   gdn_tree_plan (or an earlier gdn_tree_forward) built from the same dims,
 *   parent_idx, seq_start, out_rows and state_rows, and nothing has written
 *   the workspace since; the metadata kernels are skipped and only the walk
 *   runs. The tree is the same for every GDN layer of a round (Flide,
 *   "Accelerating Decision Inference with Exact State Forking", section 3.3.1:
 *   metadata is filled once before the round's graph replays), so a model
 *   plans once and walks once per layer. The plan stamps the workspace with
 *   a fingerprint of dims, n_out, n_state and whether out_rows is given; a
 *   walk whose fingerprint differs raises GDN_DEV_NOT_PLANNED and computes
 *   nothing. A workspace planned for another tree of the same sizes gives
 *   that tree's results (never a fault: every table stays within its sizes). */
#define GDN_FWD_PLANNED 1u

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_NULL = -1,      /* a required pointer is NULL */
  GDN_ERR_DIMS = -2,      /* unsupported sizes: see gdn_tree_dims */
  GDN_ERR_DTYPE = -3,     /* unknown dtype */
  GDN_ERR_WORKSPACE = -4, /* workspace_bytes below gdn_tree_workspace_size */
  GDN_ERR_HIP = -5,       /* a HIP launch failed; gdn_tree_last_error() has its text */
  GDN_ERR_ARGS = -6,      /* inconsistent arguments (row counts, dv_tile, ...) */
} gdn_status;

/* Device-side error codes (gdn_tree_check_error). Index meaning per code. */
typedef enum gdn_dev_error {
  GDN_DEV_OK = 0,
  GDN_DEV_SEQ_START = 1,      /* seq_start is not a CSR over [0, T]; index = position in seq_start */
  GDN_DEV_PARENT_ORDER = 2,   /* parent < -1 or parent >= t; index = t */
  GDN_DEV_PARENT_SEQ = 3,     /* parent lies in an earlier sequence; index = t */
  GDN_DEV_FORK_CAPACITY = 4,  /* more fork tokens than max_forks; index = first token without a slot */
  GDN_DEV_LEVEL_CAPACITY = 5, /* fork nesting reaches max_levels; index = first token of the segment */
  GDN_DEV_ROWS = 6,           /* out_rows / state_rows entry outside [0, T) or repeated; index = position */
  GDN_DEV_PATH = 7,           /* commit path is not a root-to-node parent chain; index = path number */
  GDN_DEV_NOT_PLANNED = 8,    /* GDN_FWD_PLANNED on a workspace without a matching plan; index = 0 */
  GDN_DEV_CHAIN = 9,          /* gdn_chain_step: an accepted count outside [0, N] or a history length outside
                                 [0, hist_cap]; index = the first such sequence (it is skipped) */
  GDN_DEV_CACHE = 10,         /* gdn_tree_attention: cache_start is not a CSR over [0, Tc]; index = position */
} gdn_dev_error;

/*
 * Sizes of one forward call.
 *  T          tokens in the flat stream (<= 2^31 - 1)
 *  H          heads (>= 1); every head has its own q, k, v, gate, beta and state;
 *             H * max(Dk, Dv) must stay below 2^24 (GDN_ERR_DIMS otherwise)
 *  Dk, Dv     key and value widths. bf16: Dk in {32, 64, 128}; fp32: Dk in
 *             {16, 32, 64}. Dv: a multiple of 16, at most 128.
 *  n_seq      sequences; seq_start has n_seq + 1 entries
 *  dtype      gdn_dtype of q, k, v, log_gate, beta and out
 *  max_forks  capacity of fork-state slots: tokens that start no segment of
 *             their own but are the parent of a segment start of a sequence
 *             longer than 64 tokens (Flide's fixed capacities, section 3.3.2)
 *  max_levels capacity of fork nesting levels; the walk runs one launch per
 *             level, levels beyond the tree's depth return at once
 */
typedef struct gdn_tree_dims {
  int64_t T;
  int32_t H, Dk, Dv;
  int32_t n_seq;
  int32_t dtype;
  int32_t max_forks;
  int32_t max_levels;
} gdn_tree_dims;

/*
 * Arguments of gdn_tree_forward / gdn_tree_plan.
 *  q, k, v, log_gate, beta   inputs in dims.dtype (layouts above); may be NULL when T = 0
 *  parent_idx [T] int32      global parent index, -1 = the sequence's initial state (NULL when T = 0);
 *                            parents precede children (TreeWY section 3: DFS pre-order
 *                            or any parents-first layout; Flide: trunk before its questions)
 *  seq_start [n_seq+1] int32 CSR of the sequences (seq_start[0] = 0, last = T)
 *  init_state                [n_seq, H, Dv, Dk] fp32, or NULL for zeros
 *  out, out_rows, n_out      outputs in dims.dtype. out_rows NULL: out is [T, H, Dv] and
 *                            n_out must be T. Otherwise out row i holds token out_rows[i]
 *                            (Flide section 3.3.3 selective readout); rows distinct.
 *                            out may be NULL when n_out = 0.
 *  state_out, state_rows,    state after token state_rows[i] into state_out[i] ([n_state, H,
 *  n_state                   Dv, Dk] fp32); rows distinct; n_state may be 0
 *  pseudo_v                  [T, H, Dv] fp32 pseudo-values for a later commit, or NULL
 *  workspace                 device buffer of at least gdn_tree_workspace_size bytes,
 *                            256-byte aligned; holds the tree metadata, fork states and the
 *                            error word; contents need no initialisation
 *  dv_tile                   columns of Dv one workgroup carries: 0 = automatic, else 16, 32
 *                            or 64 dividing Dv. Results are bitwise the same for every choice.
 *  flags                     0 or GDN_FWD_PLANNED
 * Alignment: q, k, v, out, init_state, state_out and pseudo_v must be 16-byte
 * aligned (GDN_ERR_ARGS otherwise); the kernels move them in 8- and 16-byte pieces.
 */
typedef struct gdn_tree_fwd_args {
  gdn_tree_dims dims;
  const void* q;
  const void* k;
  const void* v;
  const void* log_gate;
  const void* beta;
  const int32_t* parent_idx;
  const int32_t* seq_start;
  const float* init_state;
  void* out;
  const int32_t* out_rows;
  int32_t n_out;
  float* state_out;
  const int32_t* state_rows;
  int32_t n_state;
  float* pseudo_v;
  void* workspace;
  size_t workspace_bytes;
  int32_t dv_tile;
  uint32_t flags;
} gdn_tree_fwd_args;

/*
 * Arguments of gdn_tree_commit (TreeWY Eq. 3).
 *  dims                 as for the forward that produced pseudo_v (max_forks, max_levels unused)
 *  k, log_gate          the forward's inputs (dims.dtype)
 *  parent_idx, seq_start, init_state   the forward's structure and initial states
 *  pseudo_v             [T, H, Dv] fp32 written by that forward
 *  n_path, path_ptr [n_path+1], path_nodes   CSR of accepted paths; each lists global token
 *                       indices from a root (parent -1) down to the accepted node, each node
 *                       the parent of the next; an empty path commits the initial state.
 *                       path_nodes is required whenever n_path > 0 (any valid address when
 *                       every path is empty). A node's index is clamped into [0, T) before
 *                       anything indexed by it is read, and every node is checked against its
 *                       sequence's range and parent before any state is written; a bad path
 *                       raises GDN_DEV_PATH (the smallest such path) and its state is not written.
 *  path_seq [n_path]    sequence of each path
 *  out_state            [n_path, H, Dv, Dk] fp32
 *  workspace            device buffer of at least gdn_tree_commit_workspace_size() bytes
 * k, pseudo_v, init_state and out_state must be 16-byte aligned (GDN_ERR_ARGS otherwise).
 */
typedef struct gdn_tree_commit_args {
  gdn_tree_dims dims;
  const void* k;
  const void* log_gate;
  const int32_t* parent_idx;
  const int32_t* seq_start;
  const float* init_state;
  const float* pseudo_v;
  int32_t n_path;
  const int32_t* path_ptr;
  const int32_t* path_nodes;
  const int32_t* path_seq;
  float* out_state;
  void* workspace;
  size_t workspace_bytes;
} gdn_tree_commit_args;

/* Byte offsets of the metadata tables inside a forward workspace, for
 * inspection after gdn_tree_plan (each table is int32 unless noted):
 *  err (uint64: code << 32 | index, all ones = no error), n_seg, n_fork,
 *  tok_seq[T], depth[T], fork_slot[T] (-1 = none),
 *  seg_start/len/seq/mode/entry/slot/level [T] (first n_seg valid; mode 1 = tree chunk),
 *  level_count[max_levels], level_ptr[max_levels + 1], level_items[T] (segment ids grouped
 *  by level; order inside a level unspecified), tree_mask[n_seq][64] (uint64 ancestor-or-self
 *  bits of tree-chunk sequences, zero otherwise), fork_states (fp32 [max_forks, H, Dv, Dk]). */
typedef struct gdn_tree_layout {
  size_t err, n_seg, n_fork;
  size_t tok_seq, depth, fork_slot;
  size_t seg_start, seg_len, seg_seq, seg_mode, seg_entry, seg_slot, seg_level;
  size_t level_count, level_ptr, level_items;
  size_t tree_mask;
  size_t fork_states;
  size_t total;
} gdn_tree_layout;

/* Workspace bytes for a forward with these sizes. Host only. */
int gdn_tree_workspace_size(const gdn_tree_dims* dims, size_t* bytes);

/* Offsets of the metadata tables for these sizes. Host only. */
int gdn_tree_plan_layout(const gdn_tree_dims* dims, gdn_tree_layout* layout);

/* Workspace bytes gdn_tree_commit needs (the error word). Host only. */
size_t gdn_tree_commit_workspace_size(void);

/*
 * Builds the tree metadata only (validation, depth, segments, fork slots,
 * dependency levels, ancestor masks) into a->workspace. It reads dims,
 * parent_idx, seq_start, out_rows/n_out, state_rows/n_state and workspace.
 * gdn_tree_forward runs the same kernels first.
 */
int gdn_tree_plan(const gdn_tree_fwd_args* a, void* stream);

/*
 * The forward pass: metadata, then the chunked tree-WY walk, level by level.
 * Writes out rows, state_out rows and pseudo_v (when given). The output of
 * token t uses its post-update state S_t. The bits of a token's outputs and
 * states depend only on its own sequence: other sequences in the stream, their
 * order, and dv_tile never change them.
 */
int gdn_tree_forward(const gdn_tree_fwd_args* a, void* stream);

/*
 * gdn_tree_forward without a caller workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation. The workspace is a static device array of
 * GDN_TREE_STATIC_WORKSPACE_BYTES bytes inside the library, one per GPU, held
 * from the library's first use on that GPU until the process ends. a->workspace
 * and a->workspace_bytes are ignored; everything else is as for
 * gdn_tree_forward (inputs and outputs are still the caller's).
 *  - Sizes whose workspace (gdn_tree_workspace_size) exceeds the array are
 *    rejected with GDN_ERR_WORKSPACE and a message; nothing is enqueued.
 *  - The call allocates nothing (no hipMalloc, no library allocation). The
 *    device address of the array is looked up once per device, on the first
 *    call with that device current.
 *  - Every call on a GPU shares that GPU's array, which keeps the last call's
 *    metadata and fork states: calls that overlap on one GPU (other streams,
 *    other threads) race and must be serialised by the caller. The metadata
 *    kernels rebuild everything a walk reads, so nothing needs clearing between
 *    calls; GDN_FWD_PLANNED reuses the array's last plan.
 *  - gdn_tree_check_error(NULL, stream, ...) reads the array's error word on the
 *    current device.
 */
#define GDN_TREE_STATIC_WORKSPACE_BYTES (64u << 20)
int gdn_tree_forward_static(const gdn_tree_fwd_args* a, void* stream);

/* Rebuilds the state after each accepted path's last node (TreeWY Eq. 3). */
int gdn_tree_commit(const gdn_tree_commit_args* a, void* stream);

/*
 * ForkAttention: full attention over the same tree-structured flat stream, for
 * the full-attention layers of a hybrid model (Flide, "Accelerating Decision
 * Inference with Exact State Forking", section 3.2.1 "Full-Attention Layers").
 * Token t attends to its ancestors-or-self in its own sequence (the rule under
 * which every question computes its standalone prompt, section 3.2.3; the
 * page's Equation 3 that states it did not survive extraction):
 *
 *     o_t = sum over j ancestor-or-self of t of softmax_j(scale * q_t . k_j) v_j
 *
 * per query head h, with key/value head h / (Hq / Hkv) (grouped heads).
 * The key ranges of every 64-token query chunk (its own segment's prefix and
 * each ancestor segment's prefix up to the fork) are built on the GPU from the
 * recurrence's segment tables (section 3.3.1); fully visible key tiles take no
 * mask. Launch shapes depend only on the sizes.
 *
 * Sizes: T tokens (< 2^31), Hq query heads, Hkv key/value heads (Hq a multiple
 * of Hkv, Hq * D < 2^24), D = 128, dtype GDN_BF16, n_seq sequences, max_levels
 * the fork-nesting capacity in [1, 64] (a deeper tree raises
 * GDN_DEV_LEVEL_CAPACITY and nothing is computed).
 */
typedef struct gdn_attn_dims {
  int64_t T;
  int32_t Hq, Hkv, D;
  int32_t n_seq;
  int32_t dtype;
  int32_t max_levels;
} gdn_attn_dims;

/* GDN_ATTN_PLANNED: the workspace holds the tables an earlier gdn_tree_attention
 * built for the same dims, parent_idx and seq_start; only the attention runs
 * (a model's full-attention layers of one round share them). A workspace
 * planned for other sizes raises GDN_DEV_NOT_PLANNED. */
#define GDN_ATTN_PLANNED 1u

/*
 * Arguments of gdn_tree_attention.
 *  scale                     softmax scale, positive and finite (commonly 1 / sqrt(D))
 *  q [T, Hq, D], k and v [T, Hkv, D]   bf16, token-major, 16-byte aligned
 *  parent_idx [T], seq_start [n_seq + 1]   the stream's structure, as for gdn_tree_forward
 *  out [T, Hq, D]            bf16, 16-byte aligned
 *  workspace                 at least gdn_tree_attention_workspace_size bytes, 256-byte aligned;
 *                            its error word is read with gdn_tree_check_error
 *  flags                     0 or GDN_ATTN_PLANNED
 *  k_cache, v_cache [Tc, Hkv, D], cache_start [n_seq + 1], Tc
 *                            cached keys and values of resumed states (Flide section 3.4: a
 *                            checkpoint keeps the full-attention keys and values before its
 *                            position): every token of sequence s also sees cached rows
 *                            [cache_start[s], cache_start[s + 1]), ahead of its root path.
 *                            cache_start NULL: no cache. bf16, 16-byte aligned. cache_start is
 *                            checked on the device (GDN_DEV_CACHE); it may change between calls
 *                            that reuse one plan.
 */
typedef struct gdn_attn_args {
  gdn_attn_dims dims;
  float scale;
  const void* q;
  const void* k;
  const void* v;
  const int32_t* parent_idx;
  const int32_t* seq_start;
  void* out;
  void* workspace;
  size_t workspace_bytes;
  uint32_t flags;
  const void* k_cache;
  const void* v_cache;
  const int32_t* cache_start;
  int64_t Tc;
} gdn_attn_args;

/* Workspace bytes of gdn_tree_attention for these sizes. Host only. */
int gdn_tree_attention_workspace_size(const gdn_attn_dims* dims, size_t* bytes);

/* ForkAttention over the stream: metadata (unless GDN_ATTN_PLANNED), then the
 * attention kernel. Enqueue only. */
int gdn_tree_attention(const gdn_attn_args* a, void* stream);

/*
 * One speculative round of chain drafts in one kernel (TreeWY, "Speculative
 * Verification for Gated DeltaNet Hybrids", section 4 "Implementation": a chain
 * verifies and commits in one fused, graph-capturable kernel), with the
 * committed state written only at a flush (the deferred write of ReplaySSM, the
 * prior point TreeWY's section 1 and appendix D compare against).
 *
 * Per sequence s the call
 *  1. rebuilds the committed state S from the checkpoint, the history of
 *     accepted tokens since it, and the first accepted[s] tokens of the previous
 *     draft (TreeWY Eq. 3 over that path);
 *  2. flushes (writes S to ckpt and empties the history) when GDN_CHAIN_FLUSH is
 *     set or the history would exceed hist_cap, and otherwise appends those
 *     accepted tokens' pseudo-values, keys and log gates to the history;
 *     writes S to state_out when given;
 *  3. verifies this round's chain draft of N tokens from S (TreeWY Eq. 1 with
 *     the key rewrite, token by token in fp32): outputs and pseudo-values.
 * The next call passes this call's k, log_gate and pseudo_v as prev_k, prev_g
 * and prev_pv, the sampler's accepted counts, and hist_len_out as hist_len_in
 * (callers alternate two draft buffers and two history-length buffers). The
 * first round passes accepted = 0, hist_len_in = 0 and ckpt = the initial state.
 *
 * Layouts (row-major, token-major inside a sequence): ckpt, state_out [n_seq, H,
 * Dv, Dk] fp32; hist_pv [n_seq, hist_cap, H, Dv] fp32; hist_k [n_seq, hist_cap,
 * H, Dk] dtype; hist_g [n_seq, hist_cap, H] fp32; prev_pv, pseudo_v, out
 * [n_seq, N, H, Dv] (pv fp32, out dtype); prev_k, q, k [n_seq, N, H, Dk];
 * v [n_seq, N, H, Dv]; prev_g, log_gate, beta [n_seq, N, H]; accepted,
 * hist_len_in, hist_len_out [n_seq] int32. Sizes: N in [1, 32], Dk in {32, 64,
 * 128}, Dv a multiple of 16 up to 128, hist_cap >= 0 (0: the state is written
 * every round). ckpt, state_out, hist_pv, hist_k, prev_pv, prev_k, q, k and v
 * must be 16-byte aligned (they are moved in 16-byte pieces). workspace: at
 * least gdn_tree_commit_workspace_size() bytes; its error word (GDN_DEV_CHAIN)
 * is read with gdn_tree_check_error.
 */
#define GDN_CHAIN_FLUSH 1u

typedef struct gdn_chain_dims {
  int32_t n_seq;
  int32_t N;
  int32_t H, Dk, Dv;
  int32_t dtype;
  int32_t hist_cap;
} gdn_chain_dims;

typedef struct gdn_chain_args {
  gdn_chain_dims dims;
  float* ckpt;
  float* hist_pv;
  void* hist_k;
  float* hist_g;
  const int32_t* hist_len_in;
  int32_t* hist_len_out;
  const float* prev_pv;
  const void* prev_k;
  const void* prev_g;
  const int32_t* accepted;
  const void* q;
  const void* k;
  const void* v;
  const void* log_gate;
  const void* beta;
  void* out;
  float* pseudo_v;
  float* state_out;
  void* workspace;
  size_t workspace_bytes;
  uint32_t flags;
} gdn_chain_args;

int gdn_chain_step(const gdn_chain_args* a, void* stream);

/* Synchronises `stream`, then reads the workspace's error word. *code gets a
 * gdn_dev_error, *index its index (0 when there is no error). workspace NULL:
 * the static workspace of gdn_tree_forward_static on the current device. */
int gdn_tree_check_error(const void* workspace, void* stream, int32_t* code, int64_t* index);

/* Static text for a gdn_status or, shifted by 100 (100 + code), a gdn_dev_error. */
const char* gdn_tree_strerror(int code);

/* Thread-local text of the last host-side failure of this thread. */
const char* gdn_tree_last_error(void);

int gdn_tree_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_TREE_H */
