// The C ABI of include/gdn_tree.h: argument checks on the host, then kernel
// launches on the caller's stream. No allocation and no synchronisation
// (except gdn_tree_check_error). Between calls the library keeps only
// per-device caches of the CU count and of kernel attributes, and the static
// workspace of gdn_tree_forward_static (whose contents a call rebuilds).
#include <stdio.h>

#include <atomic>
#include <string>

#include "gdn_internal.h"

using namespace gdn;

// Workspace of gdn_tree_forward_static: one copy per GPU, held until the
// process ends. Host code never uses this name as an address: the device
// address of each GPU's copy is looked up once per device (static_workspace).
static __device__ __align__(256) unsigned char scratch[GDN_TREE_STATIC_WORKSPACE_BYTES];

namespace gdn {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];  // 0 = not queried yet
// (kernel, device) pairs whose dynamic-LDS attribute is set, with the
// kernel's occupancy at that size: a small open-addressed table
constexpr int kLdsSlots = 256;
std::atomic<const void*> g_lds_kern[kLdsSlots];
std::atomic<int> g_lds_dev[kLdsSlots];
std::atomic<int> g_lds_bytes[kLdsSlots];
std::atomic<int> g_lds_occ[kLdsSlots];
}  // namespace

hipError_t current_device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int v = (dev >= 0 && dev < kMaxDevices) ? g_cus[dev].load(std::memory_order_relaxed) : 0;
  if (v <= 0) {
    e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) g_cus[dev].store(v, std::memory_order_relaxed);
  }
  *cus = v;
  return hipSuccess;
}

hipError_t ensure_dynamic_lds(const void* kernel, int bytes, int threads, int* occupancy) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  auto query = [&](int* occ) -> hipError_t {
    hipError_t r = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (r != hipSuccess) return r;
    *occ = 1;
    r = hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, kernel, threads, bytes);
    if (r != hipSuccess) return r;
    if (*occ < 1) *occ = 1;
    return hipSuccess;
  };
  const size_t h0 = ((reinterpret_cast<uintptr_t>(kernel) >> 4) * 31u + (unsigned)dev) % kLdsSlots;
  for (size_t i = 0; i < kLdsSlots; ++i) {
    const size_t j = (h0 + i) % kLdsSlots;
    const void* k = g_lds_kern[j].load(std::memory_order_acquire);
    if (k == kernel && g_lds_dev[j].load(std::memory_order_acquire) == dev &&
        g_lds_bytes[j].load(std::memory_order_acquire) == bytes) {
      const int occ = g_lds_occ[j].load(std::memory_order_acquire);
      if (occ > 0) {
        if (occupancy) *occupancy = occ;
        return hipSuccess;
      }
    }
    if (k == nullptr) {
      int occ = 1;
      e = query(&occ);
      if (e != hipSuccess) return e;
      if (occupancy) *occupancy = occ;
      const void* expect = nullptr;
      if (g_lds_kern[j].compare_exchange_strong(expect, kernel, std::memory_order_acq_rel)) {
        g_lds_dev[j].store(dev, std::memory_order_release);
        g_lds_bytes[j].store(bytes, std::memory_order_release);
        g_lds_occ[j].store(occ, std::memory_order_release);
      }
      return hipSuccess;
    }
  }
  int occ = 1;  // table full: query on every call
  e = query(&occ);
  if (occupancy) *occupancy = occ;
  return e;
}

namespace {
std::atomic<void*> g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device
}  // namespace

// Device address of the static workspace on the current device (looked up on
// the first call on each device, with that device current).
hipError_t static_workspace(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace gdn

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* msg) {
  g_last_error = msg;
  return code;
}

int fail_hip(hipError_t e, const char* where) {
  g_last_error = std::string(where) + ": " + hipGetErrorString(e);
  return GDN_ERR_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_dims(const gdn_tree_dims* d) {
  if (!d) return fail(GDN_ERR_NULL, "dims is NULL");
  if (d->dtype != GDN_F32 && d->dtype != GDN_BF16) return fail(GDN_ERR_DTYPE, "dtype must be GDN_F32 or GDN_BF16");
  if (d->T < 0 || d->T > 0x7fffffffLL) return fail(GDN_ERR_DIMS, "T must be in [0, 2^31)");
  if (d->H < 1 || d->n_seq < 0) return fail(GDN_ERR_DIMS, "H must be >= 1 and n_seq >= 0");
  if (d->Dv < 16 || d->Dv > 128 || d->Dv % 16) return fail(GDN_ERR_DIMS, "Dv must be a multiple of 16 in [16, 128]");
  const bool dk_ok = d->dtype == GDN_BF16 ? (d->Dk == 32 || d->Dk == 64 || d->Dk == 128)
                                          : (d->Dk == 16 || d->Dk == 32 || d->Dk == 64);
  if (!dk_ok) return fail(GDN_ERR_DIMS, "Dk must be 32, 64 or 128 (bf16) or 16, 32 or 64 (fp32)");
  if ((long long)d->H * (d->Dk > d->Dv ? d->Dk : d->Dv) >= (1ll << 24))
    return fail(GDN_ERR_DIMS, "H * max(Dk, Dv) must stay below 2^24");
  if (d->max_forks < 0 || d->max_levels < 1 || d->max_levels > 4096)
    return fail(GDN_ERR_DIMS, "max_forks must be >= 0 and max_levels in [1, 4096]");
  return GDN_OK;
}

// Columns of Dv per workgroup: enough items to give every CU one, widest tile otherwise.
int choose_dv_tile(const gdn_tree_dims& d) {
  int cus = 256, v = 0;
  if (current_device_cus(&v) == hipSuccess && v > 0) cus = v;
  const long long units = (long long)(d.n_seq > 0 ? d.n_seq : 1) * d.H;
  const int max_bv = d.dtype == GDN_BF16 ? 64 : 32;
  for (int bv = max_bv; bv >= 16; bv >>= 1) {
    if (d.Dv % bv) continue;
    if (units * (d.Dv / bv) >= cus || bv == 16) return bv;
  }
  return 16;
}

int check_fwd(const gdn_tree_fwd_args* a, bool walk, LayoutFull* L) {
  if (!a) return fail(GDN_ERR_NULL, "args is NULL");
  int rc = check_dims(&a->dims);
  if (rc) return rc;
  const gdn_tree_dims& d = a->dims;
  if (!a->seq_start || !a->workspace || (d.T > 0 && !a->parent_idx))
    return fail(GDN_ERR_NULL, "seq_start, workspace and (T > 0) parent_idx are required");
  if (!compute_layout(d, L)) return fail(GDN_ERR_DIMS, "bad sizes");
  if (a->workspace_bytes < L->pub.total) return fail(GDN_ERR_WORKSPACE, "workspace smaller than gdn_tree_workspace_size");
  if (((uintptr_t)a->workspace & 255u) != 0) return fail(GDN_ERR_ARGS, "workspace must be 256-byte aligned");
  if (a->n_out < 0 || a->n_state < 0) return fail(GDN_ERR_ARGS, "row counts must be >= 0");
  if (a->n_state > 0 && !a->state_rows) return fail(GDN_ERR_NULL, "state_rows is NULL");
  if (a->n_out > 0 && !a->out_rows && a->n_out != d.T) return fail(GDN_ERR_ARGS, "without out_rows, n_out must be T");
  if (a->flags & ~GDN_FWD_PLANNED) return fail(GDN_ERR_ARGS, "unknown flags");
  if (!walk) return GDN_OK;
  if (d.T > 0 && (!a->q || !a->k || !a->v || !a->log_gate || !a->beta))
    return fail(GDN_ERR_NULL, "q, k, v, log_gate and beta are required when T > 0");
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->out) || !aligned16(a->init_state) ||
      !aligned16(a->state_out) || !aligned16(a->pseudo_v))
    return fail(GDN_ERR_ARGS, "q, k, v, out, init_state, state_out and pseudo_v must be 16-byte aligned");
  if (!a->out_rows && a->n_out != d.T) return fail(GDN_ERR_ARGS, "without out_rows, n_out must be T");
  if ((a->n_out > 0 || (!a->out_rows && d.T > 0)) && !a->out) return fail(GDN_ERR_NULL, "out is NULL");
  if (a->n_state > 0 && !a->state_out) return fail(GDN_ERR_NULL, "state_out is NULL");
  if (a->dv_tile != 0) {
    if (!walk_supported(d.dtype, d.Dk, a->dv_tile) || d.Dv % a->dv_tile)
      return fail(GDN_ERR_ARGS, "dv_tile must be 0 or a supported width (16, 32, 64 bf16; 16, 32 fp32) dividing Dv");
  }
  const long long items = d.T * (long long)d.H * (d.Dv / 16);
  if (items >= 0x7fffffffLL) return fail(GDN_ERR_DIMS, "T * H * Dv / 16 must stay below 2^31");
  return GDN_OK;
}

}  // namespace

static int forward_impl(const gdn_tree_fwd_args* a, void* stream);

extern "C" {

int gdn_tree_version(void) { return GDN_TREE_VERSION; }

const char* gdn_tree_last_error(void) { return g_last_error.c_str(); }

const char* gdn_tree_strerror(int code) {
  switch (code) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL: return "a required pointer is NULL";
    case GDN_ERR_DIMS: return "unsupported sizes";
    case GDN_ERR_DTYPE: return "unknown dtype";
    case GDN_ERR_WORKSPACE: return "workspace too small";
    case GDN_ERR_HIP: return "HIP launch failed";
    case GDN_ERR_ARGS: return "inconsistent arguments";
    case 100 + GDN_DEV_OK: return "no device error";
    case 100 + GDN_DEV_SEQ_START: return "seq_start is not a CSR over [0, T]";
    case 100 + GDN_DEV_PARENT_ORDER: return "a parent is < -1 or not before its child";
    case 100 + GDN_DEV_PARENT_SEQ: return "a parent lies in another sequence";
    case 100 + GDN_DEV_FORK_CAPACITY: return "more fork tokens than max_forks";
    case 100 + GDN_DEV_LEVEL_CAPACITY: return "fork nesting reaches max_levels";
    case 100 + GDN_DEV_ROWS: return "an out/state row is out of range or repeated";
    case 100 + GDN_DEV_PATH: return "a commit path is not a root-to-node parent chain";
    case 100 + GDN_DEV_NOT_PLANNED: return "GDN_FWD_PLANNED on a workspace without a matching plan";
    case 100 + GDN_DEV_CHAIN: return "an accepted count or history length is out of range";
    case 100 + GDN_DEV_CACHE: return "cache_start is not a CSR over [0, Tc]";
    default: return "unknown code";
  }
}

int gdn_tree_workspace_size(const gdn_tree_dims* dims, size_t* bytes) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!bytes) return fail(GDN_ERR_NULL, "bytes is NULL");
  LayoutFull L;
  if (!compute_layout(*dims, &L)) return fail(GDN_ERR_DIMS, "bad sizes");
  *bytes = L.pub.total;
  return GDN_OK;
}

int gdn_tree_plan_layout(const gdn_tree_dims* dims, gdn_tree_layout* layout) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (!layout) return fail(GDN_ERR_NULL, "layout is NULL");
  LayoutFull L;
  if (!compute_layout(*dims, &L)) return fail(GDN_ERR_DIMS, "bad sizes");
  *layout = L.pub;
  return GDN_OK;
}

size_t gdn_tree_commit_workspace_size(void) { return 256; }

int gdn_tree_plan(const gdn_tree_fwd_args* a, void* stream) {
  LayoutFull L;
  int rc = check_fwd(a, false, &L);
  if (rc) return rc;
  Meta m = meta_from(a->workspace, L);
  hipError_t e = launch_plan(*a, m, L, plan_fingerprint(*a), (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "gdn_tree_plan");
  return GDN_OK;
}

int gdn_tree_forward(const gdn_tree_fwd_args* a, void* stream) { return forward_impl(a, stream); }

int gdn_tree_forward_static(const gdn_tree_fwd_args* a, void* stream) {
  if (!a) return fail(GDN_ERR_NULL, "args is NULL");
  int rc = check_dims(&a->dims);
  if (rc) return rc;
  LayoutFull L;
  if (!compute_layout(a->dims, &L)) return fail(GDN_ERR_DIMS, "bad sizes");
  if (L.pub.total > (size_t)GDN_TREE_STATIC_WORKSPACE_BYTES) {
    char msg[200];
    snprintf(msg, sizeof msg,
             "these sizes need a %zu-byte workspace, more than the %zu bytes of the static workspace of "
             "gdn_tree_forward_static; use gdn_tree_forward with a workspace of its own",
             L.pub.total, (size_t)GDN_TREE_STATIC_WORKSPACE_BYTES);
    return fail(GDN_ERR_WORKSPACE, msg);
  }
  void* ws = nullptr;
  hipError_t e = static_workspace(&ws);
  if (e != hipSuccess) return fail_hip(e, "gdn_tree_forward_static (static workspace address)");
  gdn_tree_fwd_args b = *a;
  b.workspace = ws;
  b.workspace_bytes = (size_t)GDN_TREE_STATIC_WORKSPACE_BYTES;
  return forward_impl(&b, stream);
}

static int forward_impl(const gdn_tree_fwd_args* a, void* stream) {
  LayoutFull L;
  int rc = check_fwd(a, true, &L);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  Meta m = meta_from(a->workspace, L);
  const unsigned long long tag = plan_fingerprint(*a);
  hipError_t e = (a->flags & GDN_FWD_PLANNED) ? launch_replan_check(m, a->dims.max_levels, tag, s)
                                               : launch_plan(*a, m, L, tag, s);
  if (e != hipSuccess) return fail_hip(e, "gdn_tree_forward (metadata)");
  if (a->dims.T == 0 || a->dims.n_seq == 0) return GDN_OK;
  const int bv = a->dv_tile ? a->dv_tile : choose_dv_tile(a->dims);
  e = launch_walk(*a, m, bv, s);
  if (e != hipSuccess) return fail_hip(e, "gdn_tree_forward (walk)");
  return GDN_OK;
}

int gdn_tree_commit(const gdn_tree_commit_args* a, void* stream) {
  if (!a) return fail(GDN_ERR_NULL, "args is NULL");
  gdn_tree_dims d = a->dims;
  d.max_forks = 0;
  d.max_levels = 1;
  int rc = check_dims(&d);
  if (rc) return rc;
  if (a->n_path < 0) return fail(GDN_ERR_ARGS, "n_path must be >= 0");
  if (!a->workspace) return fail(GDN_ERR_NULL, "workspace is NULL");
  if (a->workspace_bytes < gdn_tree_commit_workspace_size()) return fail(GDN_ERR_WORKSPACE, "commit workspace too small");
  if (a->n_path > 0) {
    if (!a->k || !a->log_gate || !a->parent_idx || !a->seq_start || !a->pseudo_v || !a->path_ptr ||
        !a->path_nodes || !a->path_seq || !a->out_state)
      return fail(GDN_ERR_NULL,
                  "k, log_gate, parent_idx, seq_start, pseudo_v, path_ptr, path_nodes, path_seq and out_state are "
                  "required when n_path > 0");
    if (!aligned16(a->out_state) || (a->init_state && !aligned16(a->init_state)) || !aligned16(a->k) ||
        !aligned16(a->pseudo_v))
      return fail(GDN_ERR_ARGS, "states, k and pseudo_v must be 16-byte aligned");
  }
  hipError_t e = launch_commit(*a, (unsigned long long*)a->workspace, (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "gdn_tree_commit");
  return GDN_OK;
}

static int check_attn_dims(const gdn_attn_dims* d) {
  if (!d) return fail(GDN_ERR_NULL, "dims is NULL");
  if (d->dtype != GDN_BF16) return fail(GDN_ERR_DTYPE, "gdn_tree_attention takes bf16 q, k and v");
  if (d->T < 0 || d->T > 0x7fffffffLL) return fail(GDN_ERR_DIMS, "T must be in [0, 2^31)");
  if (d->Hq < 1 || d->Hkv < 1 || d->Hq % d->Hkv) return fail(GDN_ERR_DIMS, "Hq must be a positive multiple of Hkv");
  if (d->D != 128) return fail(GDN_ERR_DIMS, "D must be 128");
  if ((long long)d->Hq * d->D >= (1ll << 24)) return fail(GDN_ERR_DIMS, "Hq * D must stay below 2^24");
  if (d->n_seq < 0) return fail(GDN_ERR_DIMS, "n_seq must be >= 0");
  if (d->max_levels < 1 || d->max_levels > attn_max_spans())
    return fail(GDN_ERR_DIMS, "max_levels must be in [1, 64] for gdn_tree_attention");
  return GDN_OK;
}

int gdn_tree_attention_workspace_size(const gdn_attn_dims* dims, size_t* bytes) {
  int rc = check_attn_dims(dims);
  if (rc) return rc;
  if (!bytes) return fail(GDN_ERR_NULL, "bytes is NULL");
  AttnLayout A;
  if (!attn_layout(*dims, &A)) return fail(GDN_ERR_DIMS, "bad sizes");
  *bytes = A.total;
  return GDN_OK;
}

int gdn_tree_attention(const gdn_attn_args* a, void* stream) {
  if (!a) return fail(GDN_ERR_NULL, "args is NULL");
  int rc = check_attn_dims(&a->dims);
  if (rc) return rc;
  const gdn_attn_dims& d = a->dims;
  if (!a->seq_start || !a->workspace || (d.T > 0 && (!a->parent_idx || !a->q || !a->k || !a->v || !a->out)))
    return fail(GDN_ERR_NULL, "seq_start, workspace and (T > 0) parent_idx, q, k, v and out are required");
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->out))
    return fail(GDN_ERR_ARGS, "q, k, v and out must be 16-byte aligned");
  if (((uintptr_t)a->workspace & 255u) != 0) return fail(GDN_ERR_ARGS, "workspace must be 256-byte aligned");
  if (a->flags & ~GDN_ATTN_PLANNED) return fail(GDN_ERR_ARGS, "unknown flags");
  if (a->cache_start) {
    if (a->Tc < 0 || a->Tc > 0x7fffffffLL) return fail(GDN_ERR_DIMS, "Tc must be in [0, 2^31)");
    if (a->Tc > 0 && (!a->k_cache || !a->v_cache)) return fail(GDN_ERR_NULL, "k_cache and v_cache are required");
    if (!aligned16(a->k_cache) || !aligned16(a->v_cache))
      return fail(GDN_ERR_ARGS, "k_cache and v_cache must be 16-byte aligned");
  }
  if (!(a->scale > 0.f) || a->scale > 3.0e38f) return fail(GDN_ERR_ARGS, "scale must be positive and finite");
  AttnLayout A;
  if (!attn_layout(d, &A)) return fail(GDN_ERR_DIMS, "bad sizes");
  if (a->workspace_bytes < A.total) return fail(GDN_ERR_WORKSPACE, "workspace smaller than gdn_tree_attention_workspace_size");
  hipError_t e = launch_attention(*a, A, (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "gdn_tree_attention");
  return GDN_OK;
}

int gdn_chain_step(const gdn_chain_args* a, void* stream) {
  if (!a) return fail(GDN_ERR_NULL, "args is NULL");
  const gdn_chain_dims& d = a->dims;
  if (d.dtype != GDN_F32 && d.dtype != GDN_BF16) return fail(GDN_ERR_DTYPE, "dtype must be GDN_F32 or GDN_BF16");
  if (d.n_seq < 0 || d.H < 1 || d.N < 1 || d.N > 32 || d.hist_cap < 0)
    return fail(GDN_ERR_DIMS, "n_seq >= 0, H >= 1, N in [1, 32] and hist_cap >= 0 are required");
  if (!(d.Dk == 32 || d.Dk == 64 || d.Dk == 128) || d.Dv < 16 || d.Dv > 128 || d.Dv % 16)
    return fail(GDN_ERR_DIMS, "Dk must be 32, 64 or 128 and Dv a multiple of 16 up to 128");
  if ((long long)d.H * (d.Dk > d.Dv ? d.Dk : d.Dv) >= (1ll << 24))
    return fail(GDN_ERR_DIMS, "H * max(Dk, Dv) must stay below 2^24");
  if (d.n_seq > 0) {
    if (!a->ckpt || !a->hist_len_in || !a->hist_len_out || !a->prev_pv || !a->prev_k || !a->prev_g || !a->accepted ||
        !a->q || !a->k || !a->v || !a->log_gate || !a->beta || !a->out || !a->pseudo_v || !a->workspace)
      return fail(GDN_ERR_NULL, "a required pointer of gdn_chain_step is NULL");
    if (d.hist_cap > 0 && (!a->hist_pv || !a->hist_k || !a->hist_g))
      return fail(GDN_ERR_NULL, "hist_pv, hist_k and hist_g are required when hist_cap > 0");
    if ((const void*)a->hist_len_in == (const void*)a->hist_len_out || (const void*)a->prev_pv == (const void*)a->pseudo_v)
      return fail(GDN_ERR_ARGS, "hist_len_out and pseudo_v must be other buffers than hist_len_in and prev_pv");
    if (!aligned16(a->ckpt) || !aligned16(a->state_out) || !aligned16(a->hist_pv) || !aligned16(a->hist_k) ||
        !aligned16(a->prev_pv) || !aligned16(a->prev_k) || !aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v))
      return fail(GDN_ERR_ARGS, "ckpt, state_out, hist_pv, hist_k, prev_pv, prev_k, q, k and v must be 16-byte aligned");
    if (a->workspace_bytes < 8) return fail(GDN_ERR_WORKSPACE, "the chain workspace holds an 8-byte error word");
  }
  if (a->flags & ~GDN_CHAIN_FLUSH) return fail(GDN_ERR_ARGS, "unknown flags");
  hipError_t e = launch_chain(*a, (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "gdn_chain_step");
  return GDN_OK;
}

int gdn_tree_check_error(const void* workspace, void* stream, int32_t* code, int64_t* index) {
  if (!code || !index) return fail(GDN_ERR_NULL, "code and index are required");
  if (!workspace) {  // the static workspace of gdn_tree_forward_static on the current device
    void* ws = nullptr;
    hipError_t e = static_workspace(&ws);
    if (e != hipSuccess) return fail_hip(e, "gdn_tree_check_error (static workspace address)");
    workspace = ws;
  }
  unsigned long long word = 0;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(&word, workspace, sizeof(word), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return fail_hip(e, "gdn_tree_check_error (copy)");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail_hip(e, "gdn_tree_check_error (sync)");
  if (word == kNoError) {
    *code = GDN_DEV_OK;
    *index = 0;
  } else {
    *code = (int32_t)(word >> 32);
    *index = (int64_t)(uint32_t)(word & 0xffffffffu);
  }
  return GDN_OK;
}

}  // extern "C"
