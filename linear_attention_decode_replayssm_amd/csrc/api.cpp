// api.cpp -- the C ABI of librssm.so (declared in include/rssm.h): argument
// validation, kernel dispatch on the caller's stream, error codes.
//
// Every entry point validates everything it can on the host before launching
// anything; a non-zero return means nothing was enqueued.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "rssm.h"
#include "common.hpp"
#include "launch.hpp"

// Arrival counters of rssm_mamba2_step_noalloc: one 128-byte line per
// sequence, as in a caller's `arrive` buffer, for up to
// RSSM_NOALLOC_MAX_BATCH sequences (512 KiB on each device, held until the
// process ends).  Host code never passes this name to a kernel: on the host
// it is a stand-in, not a device address; the address comes from
// hipGetSymbolAddress, once per device (scratch_address below).
static __device__ __align__(256) uint32_t scratch[RSSM_NOALLOC_MAX_BATCH * RSSM_ARRIVE_STRIDE];

namespace {

constexpr int kMaxDevices = 64;

// Zero the counter word of sequences 0..batch-1 (a kernel, not a memset, so
// that the call stays a launch-only sequence under graph capture).
__global__ __launch_bounds__(256) void clear_counters_kernel(uint32_t* counters, int batch) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch) counters[(long)b * rssm::kArriveStride] = 0u;
}

// Device address of `scratch` on the current device, looked up once per
// device with that device current; NULL if the lookup fails.
uint32_t* scratch_address() {
  static std::mutex mu;
  static uint32_t* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    addr[dev] = static_cast<uint32_t*>(p);
  }
  return addr[dev];
}

inline bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// max_cap: the largest ring capacity the call serves (16; 32 for the
// Mamba-2 fp32 step, commit and rollback).
int check_layer_dims(const rssm_layer* L, int max_cap = rssm::kMaxCap) {
  if (!L) return RSSM_EINVAL;
  if (L->kind != RSSM_MAMBA2 && L->kind != RSSM_GDN) return RSSM_EINVAL;
  if (L->scheme < RSSM_F32 || L->scheme > RSSM_SHARED) return RSSM_EINVAL;
  if (L->batch < 0 || L->nheads < 1 || L->ngroups < 1 || L->dim_v < 1 || L->dim_k < 1 ||
      L->capacity < 1)
    return RSSM_EINVAL;
  // launch grids hold up to two workgroups per head (half-head GDN kernels)
  if ((int64_t)L->batch * L->nheads > (int64_t)INT32_MAX / 2) return RSSM_EUNSUPPORTED;
  if (L->capacity > max_cap) return RSSM_EUNSUPPORTED;
  if (L->kind == RSSM_MAMBA2) {
    if (L->nheads % L->ngroups != 0) return RSSM_EINVAL;
    if (L->dim_v != 64 || L->dim_k != 128) return RSSM_EUNSUPPORTED;
  } else {
    if (L->ngroups != 1) return RSSM_EINVAL;
    if (L->dim_v != 128 || L->dim_k != 128) return RSSM_EUNSUPPORTED;
  }
  if (L->scheme != RSSM_F32 && L->lp_dtype != RSSM_BF16 && L->lp_dtype != RSSM_E4M3)
    return RSSM_EINVAL;
  if (L->flags & ~RSSM_LAYER_INDEX_READONLY) return RSSM_EINVAL;
  return RSSM_OK;
}

// The capacity a call may serve on this layer: 32 for the fp32 Mamba-2 step,
// commit and rollback (long_ring), else 16.
int max_cap_for(const rssm_layer* L, bool long_ring) {
  return long_ring && L && L->kind == RSSM_MAMBA2 && L->scheme == RSSM_F32 ? rssm::kMaxCapM2
                                                                         : rssm::kMaxCap;
}

// Pointer checks of the descriptor.  Skipped at batch == 0, where every
// per-sequence array holds no elements and may be NULL.
int check_layer_ptrs(const rssm_layer* L) {
  // checkpoints
  if (L->scheme != RSSM_SHARED) {
    if (!L->ckpt) return RSSM_EINVAL;
    if (!a16(L->ckpt)) return RSSM_EALIGN;
  }
  if (L->scheme != RSSM_F32) {
    if (!L->ckpt_lp) return RSSM_EINVAL;
    if (!a16(L->ckpt_lp)) return RSSM_EALIGN;
    if (L->lp_dtype == RSSM_E4M3 && !L->lp_scale) return RSSM_EINVAL;
  }
  if (L->kind == RSSM_MAMBA2 && (!L->A || !L->D)) return RSSM_EINVAL;
  return RSSM_OK;
}

// Rings and indices are needed by every call except the eager step (the
// arrival counters too, unless the call brings its own: need_arrive false).
int check_state(const rssm_layer* L, bool need_arrive = true) {
  const int nring = L->kind == RSSM_MAMBA2 ? 3 : 4;
  for (int i = 0; i < nring; ++i)
    if (!L->ring[i]) return RSSM_EINVAL;
  if (!a16(L->ring[0]) || !a16(L->ring[1])) return RSSM_EALIGN;
  if (!L->ckpt_pos || !L->len || !L->status) return RSSM_EINVAL;
  if (need_arrive && !(L->flags & RSSM_LAYER_INDEX_READONLY) && !L->arrive) return RSSM_EINVAL;
  return RSSM_OK;
}

int hip_rc(hipError_t e) { return e == hipSuccess ? RSSM_OK : RSSM_EHIP; }

rssm::M2Args m2_args(const rssm_layer* L) {
  rssm::M2Args a{};
  a.ckpt = L->ckpt;
  a.ckpt_lp = L->ckpt_lp;
  a.lp_scale = L->lp_scale;
  a.scheme = L->scheme;
  a.lp = L->lp_dtype;
  a.A = L->A;
  a.D = L->D;
  a.ring_x = L->ring[0];
  a.ring_B = L->ring[1];
  a.ring_dt = L->ring[2];
  a.pos = L->ckpt_pos;
  a.len = L->len;
  a.arrive = L->arrive;
  a.status = L->status;
  a.idx_ro = (L->flags & RSSM_LAYER_INDEX_READONLY) != 0;
  a.batch = L->batch;
  a.H = L->nheads;
  a.G = L->ngroups;
  a.cap = L->capacity;
  a.n_pos = 1;
  return a;
}

rssm::GdnArgs gdn_args(const rssm_layer* L) {
  rssm::GdnArgs a{};
  a.ckpt = L->ckpt;
  a.ckpt_lp = L->ckpt_lp;
  a.lp_scale = L->lp_scale;
  a.ring_k = L->ring[0];
  a.ring_v = L->ring[1];
  a.ring_a = L->ring[2];
  a.ring_b = L->ring[3];
  a.pos = L->ckpt_pos;
  a.len = L->len;
  a.arrive = L->arrive;
  a.status = L->status;
  a.idx_ro = (L->flags & RSSM_LAYER_INDEX_READONLY) != 0;
  a.batch = L->batch;
  a.H = L->nheads;
  a.cap = L->capacity;
  a.n_pos = 1;
  a.scheme = L->scheme;
  a.lp = L->lp_dtype;
  return a;
}

inline hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Shared by rssm_verify (a chain: anc[j] = drafts 0..j, appended) and
// rssm_verify_tree (ancestor masks from the parent array, nothing appended).
// commit_min_len > 0: rssm_verify_commit (F32 checkpoints only).
int verify_common(const rssm_layer* L, int n_pos, const uint32_t* anc, int append,
                  const rssm_inputs* in, float* out, void* stream, int commit_min_len = 0,
                  const int32_t* n_reject = nullptr) {
  int rc = check_layer_dims(L);
  if (rc) return rc;
  if (!in) return RSSM_EINVAL;
  if (n_pos < 1 || n_pos > L->capacity || n_pos > rssm::kMaxPos) return RSSM_ERANGE;
  if (commit_min_len > 0 && L->scheme != RSSM_F32) return RSSM_EUNSUPPORTED;
  if (L->batch == 0) return RSSM_OK;
  if ((rc = check_layer_ptrs(L)) || (rc = check_state(L))) return rc;
  if (!out) return RSSM_EINVAL;
  if (!a16(out)) return RSSM_EALIGN;
  if (L->kind == RSSM_MAMBA2) {
    if (!in->x || !in->B || !in->C || !in->dt) return RSSM_EINVAL;
    if (!a16(in->x) || !a16(in->B) || !a16(in->C)) return RSSM_EALIGN;
    rssm::M2Args a = m2_args(L);
    a.x = in->x;
    a.B = in->B;
    a.C = in->C;
    a.dt = in->dt;
    a.y = out;
    a.n_pos = n_pos;
    for (int j = 0; j < n_pos; ++j) a.anc[j] = anc[j];
    a.append = append;
    a.min_len = commit_min_len;
    a.n_reject = n_reject;
    return hip_rc(rssm::launch_m2_verify(a, S(stream)));
  }
  if (!in->q || !in->k || !in->v || !in->alpha || !in->beta) return RSSM_EINVAL;
  if (!a16(in->q) || !a16(in->k) || !a16(in->v)) return RSSM_EALIGN;
  rssm::GdnArgs a = gdn_args(L);
  a.q = in->q;
  a.k = in->k;
  a.v = in->v;
  a.alpha = in->alpha;
  a.beta = in->beta;
  a.o = out;
  a.n_pos = n_pos;
  for (int j = 0; j < n_pos; ++j) a.anc[j] = anc[j];
  a.append = append;
  a.min_len = commit_min_len;
  a.n_reject = n_reject;
  return hip_rc(rssm::launch_gdn_verify(a, S(stream)));
}

}  // namespace

extern "C" {

int rssm_abi_version(void) { return RSSM_ABI_VERSION; }

const char* rssm_strerror(int code) {
  switch (code) {
    case RSSM_OK: return "ok";
    case RSSM_EINVAL: return "invalid argument (null pointer, bad enum or inconsistent dims)";
    case RSSM_EUNSUPPORTED: return "shape or scheme not supported by this library";
    case RSSM_EALIGN: return "pointer not 16-byte aligned";
    case RSSM_ERANGE: return "count out of range";
    case RSSM_EHIP: return "HIP runtime error";
    default: return "unknown error code";
  }
}

int rssm_mamba2_step(const rssm_layer* L, const float* x, const float* B, const float* C,
                     const float* dt, float* y, int commit_after, void* stream) {
  int rc = check_layer_dims(L, max_cap_for(L, true));
  if (rc) return rc;
  if (L->kind != RSSM_MAMBA2) return RSSM_EINVAL;
  if (commit_after && L->scheme == RSSM_SHARED) return RSSM_EUNSUPPORTED;
  if (L->batch == 0) return RSSM_OK;
  if ((rc = check_layer_ptrs(L)) || (rc = check_state(L))) return rc;
  if (!x || !B || !C || !dt || !y) return RSSM_EINVAL;
  if (!a16(x) || !a16(B) || !a16(C) || !a16(y)) return RSSM_EALIGN;
  rssm::M2Args a = m2_args(L);
  a.x = x;
  a.B = B;
  a.C = C;
  a.dt = dt;
  a.y = y;
  return hip_rc(rssm::launch_m2_step(a, commit_after != 0, S(stream)));
}

int rssm_mamba2_step_noalloc(const rssm_layer* L, const float* x, const float* B,
                             const float* C, const float* dt, float* y, int commit_after,
                             void* stream) {
  int rc = check_layer_dims(L, max_cap_for(L, true));
  if (rc) return rc;
  if (L->kind != RSSM_MAMBA2) return RSSM_EINVAL;
  if (commit_after && L->scheme == RSSM_SHARED) return RSSM_EUNSUPPORTED;
  if (L->batch > RSSM_NOALLOC_MAX_BATCH) return RSSM_ERANGE;
  if (L->batch == 0) return RSSM_OK;
  if ((rc = check_layer_ptrs(L)) || (rc = check_state(L, false))) return rc;
  if (!x || !B || !C || !dt || !y) return RSSM_EINVAL;
  if (!a16(x) || !a16(B) || !a16(C) || !a16(y)) return RSSM_EALIGN;
  uint32_t* counters = scratch_address();
  if (!counters) return RSSM_EHIP;
  hipLaunchKernelGGL(clear_counters_kernel, dim3((unsigned)((L->batch + 255) / 256)), dim3(256),
                     0, S(stream), counters, L->batch);
  if ((rc = hip_rc(hipGetLastError()))) return rc;
  rssm::M2Args a = m2_args(L);
  a.arrive = counters;
  a.x = x;
  a.B = B;
  a.C = C;
  a.dt = dt;
  a.y = y;
  return hip_rc(rssm::launch_m2_step(a, commit_after != 0, S(stream)));
}

int rssm_gdn_step(const rssm_layer* L, const float* q, const float* k, const float* v,
                  const float* alpha, const float* beta, float* o, int commit_after,
                  void* stream) {
  int rc = check_layer_dims(L);
  if (rc) return rc;
  if (L->kind != RSSM_GDN) return RSSM_EINVAL;
  if (commit_after && L->scheme == RSSM_SHARED) return RSSM_EUNSUPPORTED;
  if (L->batch == 0) return RSSM_OK;
  if ((rc = check_layer_ptrs(L)) || (rc = check_state(L))) return rc;
  if (!q || !k || !v || !alpha || !beta || !o) return RSSM_EINVAL;
  if (!a16(q) || !a16(k) || !a16(v) || !a16(o)) return RSSM_EALIGN;
  rssm::GdnArgs a = gdn_args(L);
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.beta = beta;
  a.o = o;
  return hip_rc(rssm::launch_gdn_step(a, commit_after != 0, S(stream)));
}

int rssm_commit(const rssm_layer* L, const uint8_t* mask, int min_len, void* stream) {
  int rc = check_layer_dims(L, max_cap_for(L, true));
  if (rc) return rc;
  if (min_len < 0) return RSSM_ERANGE;
  if (L->batch == 0) return RSSM_OK;
  if ((rc = check_layer_ptrs(L)) || (rc = check_state(L))) return rc;
  if (L->kind == RSSM_MAMBA2) {
    rssm::M2Args a = m2_args(L);
    a.mask = mask;
    a.min_len = min_len;
    return hip_rc(rssm::launch_m2_commit(a, S(stream)));
  }
  rssm::GdnArgs a = gdn_args(L);
  a.mask = mask;
  a.min_len = min_len;
  return hip_rc(rssm::launch_gdn_commit(a, S(stream)));
}

int rssm_verify(const rssm_layer* L, int n_pos, const rssm_inputs* in, float* out,
                void* stream) {
  uint32_t anc[rssm::kMaxPos] = {};
  for (int j = 0; j < rssm::kMaxPos; ++j) anc[j] = (2u << j) - 1u;   // drafts 0..j
  return verify_common(L, n_pos, anc, 1, in, out, stream);
}

int rssm_verify_commit(const rssm_layer* L, int n_pos, const rssm_inputs* in, float* out,
                       int min_len, void* stream) {
  if (min_len < 1) return RSSM_ERANGE;
  uint32_t anc[rssm::kMaxPos] = {};
  for (int j = 0; j < rssm::kMaxPos; ++j) anc[j] = (2u << j) - 1u;
  return verify_common(L, n_pos, anc, 1, in, out, stream, min_len);
}

int rssm_rollback_verify_commit(const rssm_layer* L, const int32_t* n_reject, int n_pos,
                                const rssm_inputs* in, float* out, int min_len, void* stream) {
  if (min_len < 1) return RSSM_ERANGE;
  if (!n_reject) return RSSM_EINVAL;
  uint32_t anc[rssm::kMaxPos] = {};
  for (int j = 0; j < rssm::kMaxPos; ++j) anc[j] = (2u << j) - 1u;
  return verify_common(L, n_pos, anc, 1, in, out, stream, min_len, n_reject);
}

namespace {
int verify_tree_common(const rssm_layer* L, int n_nodes, const int32_t* parent,
                       const rssm_inputs* in, float* out, void* stream, int min_len) {
  if (!parent) return RSSM_EINVAL;
  if (n_nodes < 1 || n_nodes > rssm::kMaxPos) return RSSM_ERANGE;
  uint32_t anc[rssm::kMaxPos] = {};
  for (int j = 0; j < n_nodes; ++j) {
    if (parent[j] < -1 || parent[j] >= j) return RSSM_EINVAL;   // parents come first
    anc[j] = (1u << j) | (parent[j] >= 0 ? anc[parent[j]] : 0u);
  }
  return verify_common(L, n_nodes, anc, 0, in, out, stream, min_len);
}
}  // namespace

int rssm_verify_tree(const rssm_layer* L, int n_nodes, const int32_t* parent,
                     const rssm_inputs* in, float* out, void* stream) {
  return verify_tree_common(L, n_nodes, parent, in, out, stream, 0);
}

int rssm_verify_tree_commit(const rssm_layer* L, int n_nodes, const int32_t* parent,
                            const rssm_inputs* in, float* out, int min_len, void* stream) {
  if (min_len < 1) return RSSM_ERANGE;
  return verify_tree_common(L, n_nodes, parent, in, out, stream, min_len);
}

int rssm_prefill(const rssm_layer* L, int n_tok, const rssm_inputs* in, float* out,
                 const uint8_t* mask, void* stream) {
  int rc = check_layer_dims(L);
  if (rc) return rc;
  if (!in) return RSSM_EINVAL;
  if (n_tok < 1) return RSSM_ERANGE;
  if (L->batch == 0) return RSSM_OK;
  if ((rc = check_layer_ptrs(L)) || (rc = check_state(L))) return rc;
  if (out && !a16(out)) return RSSM_EALIGN;
  if (L->kind == RSSM_MAMBA2) {
    if (!in->x || !in->B || !in->dt || (out && !in->C)) return RSSM_EINVAL;
    if (!a16(in->x) || !a16(in->B) || (out && !a16(in->C))) return RSSM_EALIGN;
    rssm::M2Args a = m2_args(L);
    a.x = in->x;
    a.B = in->B;
    a.C = out ? in->C : nullptr;
    a.dt = in->dt;
    a.y = out;
    a.mask = mask;
    a.n_pos = n_tok;
    return hip_rc(rssm::launch_m2_prefill(a, S(stream)));
  }
  if (!in->k || !in->v || !in->alpha || !in->beta || (out && !in->q)) return RSSM_EINVAL;
  if (!a16(in->k) || !a16(in->v) || (out && !a16(in->q))) return RSSM_EALIGN;
  rssm::GdnArgs a = gdn_args(L);
  a.q = out ? in->q : nullptr;
  a.k = in->k;
  a.v = in->v;
  a.alpha = in->alpha;
  a.beta = in->beta;
  a.o = out;
  a.mask = mask;
  a.n_pos = n_tok;
  return hip_rc(rssm::launch_gdn_prefill(a, S(stream)));
}

int rssm_append_path(const rssm_layer* L, int n_nodes, const int32_t* path,
                     const int32_t* path_len, int depth, const rssm_inputs* in, void* stream) {
  int rc = check_layer_dims(L);
  if (rc) return rc;
  if (!in) return RSSM_EINVAL;
  if (n_nodes < 1 || n_nodes > rssm::kMaxPos || depth < 1 || depth > n_nodes) return RSSM_ERANGE;
  if (L->batch == 0) return RSSM_OK;
  if ((rc = check_layer_ptrs(L)) || (rc = check_state(L))) return rc;
  if (!path || !path_len) return RSSM_EINVAL;
  if (L->kind == RSSM_MAMBA2) {
    if (!in->x || !in->B || !in->dt) return RSSM_EINVAL;
    if (!a16(in->x) || !a16(in->B)) return RSSM_EALIGN;
    rssm::M2Args a = m2_args(L);
    a.x = in->x;
    a.B = in->B;
    a.dt = in->dt;
    a.n_pos = n_nodes;
    a.path = path;
    a.path_len = path_len;
    a.depth = depth;
    return hip_rc(rssm::launch_m2_append_path(a, S(stream)));
  }
  if (!in->k || !in->v || !in->alpha || !in->beta) return RSSM_EINVAL;
  if (!a16(in->k) || !a16(in->v)) return RSSM_EALIGN;
  rssm::GdnArgs a = gdn_args(L);
  a.k = in->k;
  a.v = in->v;
  a.alpha = in->alpha;
  a.beta = in->beta;
  a.n_pos = n_nodes;
  a.path = path;
  a.path_len = path_len;
  a.depth = depth;
  return hip_rc(rssm::launch_gdn_append_path(a, S(stream)));
}

int rssm_rollback(const rssm_layer* L, const int32_t* n_reject, void* stream) {
  int rc = check_layer_dims(L, max_cap_for(L, true));
  if (rc) return rc;
  if (L->batch == 0) return RSSM_OK;
  if ((rc = check_layer_ptrs(L)) || (rc = check_state(L))) return rc;
  if (!n_reject) return RSSM_EINVAL;
  if (L->flags & RSSM_LAYER_INDEX_READONLY) return RSSM_OK;   // the updating layer rolls back
  return hip_rc(rssm::launch_rollback(L->ckpt_pos, L->len, L->status, n_reject, L->batch,
                                      L->capacity, S(stream)));
}

int rssm_eager_step(const rssm_layer* L, const rssm_inputs* in, float* out, void* stream) {
  int rc = check_layer_dims(L);
  if (rc) return rc;
  if (!in) return RSSM_EINVAL;
  if (L->batch == 0) return RSSM_OK;
  if ((rc = check_layer_ptrs(L))) return rc;
  if (!out) return RSSM_EINVAL;
  if (!a16(out)) return RSSM_EALIGN;
  if (L->kind == RSSM_MAMBA2) {
    if (!in->x || !in->B || !in->C || !in->dt) return RSSM_EINVAL;
    if (!a16(in->x) || !a16(in->B) || !a16(in->C)) return RSSM_EALIGN;
    rssm::M2Args a = m2_args(L);
    a.x = in->x;
    a.B = in->B;
    a.C = in->C;
    a.dt = in->dt;
    a.y = out;
    return hip_rc(rssm::launch_m2_eager(a, S(stream)));
  }
  if (!in->q || !in->k || !in->v || !in->alpha || !in->beta) return RSSM_EINVAL;
  if (!a16(in->q) || !a16(in->k) || !a16(in->v)) return RSSM_EALIGN;
  rssm::GdnArgs a = gdn_args(L);
  a.q = in->q;
  a.k = in->k;
  a.v = in->v;
  a.alpha = in->alpha;
  a.beta = in->beta;
  a.o = out;
  return hip_rc(rssm::launch_gdn_eager(a, S(stream)));
}

int rssm_eager_spec_round(const rssm_layer* L, int n_pos, const rssm_inputs* in, float* out,
                          float* slots, const int32_t* cur, void* stream) {
  int rc = check_layer_dims(L);
  if (rc) return rc;
  if (!in) return RSSM_EINVAL;
  if (L->scheme != RSSM_F32) return RSSM_EUNSUPPORTED;
  if (n_pos < 1 || n_pos > rssm::kMaxPos) return RSSM_ERANGE;
  if (L->batch == 0) return RSSM_OK;
  if ((rc = check_layer_ptrs(L))) return rc;
  if (!out || !slots || !cur || !L->status) return RSSM_EINVAL;
  if (!a16(out) || !a16(slots)) return RSSM_EALIGN;
  if (L->kind == RSSM_MAMBA2) {
    if (!in->x || !in->B || !in->C || !in->dt) return RSSM_EINVAL;
    if (!a16(in->x) || !a16(in->B) || !a16(in->C)) return RSSM_EALIGN;
    rssm::M2Args a = m2_args(L);
    a.x = in->x;
    a.B = in->B;
    a.C = in->C;
    a.dt = in->dt;
    a.y = out;
    a.n_pos = n_pos;
    return hip_rc(rssm::launch_m2_eager_spec(a, slots, cur, S(stream)));
  }
  if (!in->q || !in->k || !in->v || !in->alpha || !in->beta) return RSSM_EINVAL;
  if (!a16(in->q) || !a16(in->k) || !a16(in->v)) return RSSM_EALIGN;
  rssm::GdnArgs a = gdn_args(L);
  a.q = in->q;
  a.k = in->k;
  a.v = in->v;
  a.alpha = in->alpha;
  a.beta = in->beta;
  a.o = out;
  a.n_pos = n_pos;
  return hip_rc(rssm::launch_gdn_eager_spec(a, slots, cur, S(stream)));
}

int rssm_eager_spec_accept(const rssm_layer* L, int n_pos, int32_t* cur, const int32_t* n_accept,
                           void* stream) {
  int rc = check_layer_dims(L);
  if (rc) return rc;
  if (n_pos < 1 || n_pos > rssm::kMaxPos) return RSSM_ERANGE;
  if (L->batch == 0) return RSSM_OK;
  if (!cur || !n_accept || !L->status) return RSSM_EINVAL;
  return hip_rc(rssm::launch_eager_spec_accept(cur, L->status, n_accept, n_pos, L->batch,
                                                S(stream)));
}

namespace {
int probe(const void* src, void* dst, float* sink, int64_t bytes, int32_t tile_bytes, int check,
          void* stream) {
  if (!src || (!dst && !sink)) return RSSM_EINVAL;
  if (tile_bytes != 32768 && tile_bytes != 4096) return RSSM_EUNSUPPORTED;
  if (!a16(src) || (dst && !a16(dst))) return RSSM_EALIGN;
  if (bytes <= 0 || bytes % tile_bytes != 0 || bytes / tile_bytes > (int64_t)INT32_MAX)
    return RSSM_ERANGE;
  return hip_rc(rssm::launch_probe(src, dst, sink, (long)(bytes / tile_bytes), tile_bytes,
                                   check, S(stream)));
}
}  // namespace

int rssm_probe_stream_tiles(const void* src, void* dst, float* sink, int64_t bytes,
                           int32_t tile_bytes, int32_t check, void* stream) {
  return probe(src, dst, sink, bytes, tile_bytes, check, stream);
}

int rssm_probe_stream(const void* src, void* dst, float* sink, int64_t bytes, void* stream) {
  return probe(src, dst, sink, bytes, 32768, 1, stream);
}

int rssm_status(const rssm_layer* L, uint32_t* bits, void* stream) {
  if (!L || !L->status || !bits) return RSSM_EINVAL;
  uint32_t h = 0;
  hipError_t e = hipMemcpyAsync(&h, L->status, sizeof(uint32_t), hipMemcpyDeviceToHost, S(stream));
  if (e == hipSuccess) e = hipStreamSynchronize(S(stream));
  if (e != hipSuccess) return RSSM_EHIP;
  *bits = h;
  return hip_rc(rssm::launch_clear_status(L->status, S(stream)));
}

}  // extern "C"
