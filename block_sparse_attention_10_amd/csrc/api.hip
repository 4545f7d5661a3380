// C ABI of libmsa: argument validation, workspace layout, dispatch records
// and the entry points declared in include/msa.h.
#include "msa.h"
#include "msa_internal.h"

#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>

// The workspace of msa_decode_noalloc, for callers that cannot allocate
// device memory.  Each device the library runs on holds its own copy until
// the process ends.  In host code the array's name is only a stand-in for
// the symbol, never a device address: the address comes from
// hipGetSymbolAddress, taken once per device with that device current and
// kept per device (scratch_of_stream_device: the device that runs the
// call's stream), and only that address is handed to kernels.  The kernels write every workspace byte before they
// read it, so the array needs no clearing between calls; calls that overlap
// on one device share it and race.
static __device__ __align__(256) uint8_t scratch[MSA_NOALLOC_SCRATCH_BYTES];

namespace msa {

static thread_local int g_last_hip_error = 0;
static thread_local std::string g_last_dispatch;
static thread_local std::string g_last_check_failure;

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Workspace workspace_layout(const Dims& d) {
  const SplitPlan sp = plan_splits(d);
  const size_t rh = (size_t)d.R() * d.Hq;
  Workspace w;
  size_t off = 0;
  w.part_o = off;
  off = align256(off + rh * sp.splits * 128 * sizeof(float));
  w.part_ml = off;
  off = align256(off + rh * sp.splits * 2 * sizeof(float));
  w.scores = off;
  off = align256(off + (size_t)d.R() * d.MAXB * sizeof(float));
  w.n_selected = off;
  off = align256(off + (size_t)d.R() * sizeof(int32_t));
  w.selected = off;
  off = align256(off + (size_t)d.R() * d.topk * sizeof(int32_t));
  w.page_table = off;
  off = align256(off + (size_t)d.R() * d.PT() * sizeof(int32_t));
  w.total = off;
  return w;
}

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Validates the descriptor; fills `d`.
int check_problem(const msa_problem* p, Dims* d) {
  if (!p || p->struct_size != sizeof(msa_problem)) return MSA_ERR_INVALID_ARG;
  if (p->batch < 1 || p->decode_query_len < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1 ||
      p->num_idx_heads < 1 || p->max_blocks_per_seq < 1 || p->num_phys_blocks < 1 ||
      p->topk < 1 || p->local_blocks < 0)
    return MSA_ERR_INVALID_ARG;
  if (p->num_q_heads % p->num_kv_heads != 0) return MSA_ERR_INVALID_ARG;
  if (!(p->sm_scale >= 0.f) || !isfinite(p->sm_scale)) return MSA_ERR_INVALID_ARG;
  if ((p->flags & ~(uint32_t)MSA_FLAG_DEBUG_CHECKS) != 0) return MSA_ERR_INVALID_ARG;
  if (p->head_dim != 128 || p->idx_dim != 64 || p->block_size != 128 || p->page_size != 16 ||
      p->local_blocks != 1 || p->topk > 16 || p->decode_query_len > 16 ||
      p->num_idx_heads > 16 || p->num_q_heads / p->num_kv_heads > 16)
    return MSA_ERR_UNSUPPORTED;
  if (p->kv_dtype < MSA_DTYPE_BF16 || p->kv_dtype > MSA_DTYPE_NVFP4) return MSA_ERR_UNSUPPORTED;
  if (p->idx_k_dtype < MSA_DTYPE_BF16 || p->idx_k_dtype > MSA_DTYPE_NVFP4)
    return MSA_ERR_UNSUPPORTED;
  // An int32 context spans at most 2^24 blocks (block offsets c * 128 stay
  // in int32), and page ids phys * 8 + j must fit int32.
  if (p->max_blocks_per_seq > (1 << 24) || p->num_phys_blocks > (1 << 28))
    return MSA_ERR_UNSUPPORTED;
  // Grid limits (a launch holds fewer than 2^32 work-items): the scan runs
  // one 64-lane wave per (request, block); attention, merge and the write
  // path (one wave per row and K, V or index head) stay below 2^31
  // work-items with at most 2^22 (row, query head) and (row, index head)
  // pairs.
  const long rows = (long)p->batch * p->decode_query_len;
  if ((long)p->batch * p->max_blocks_per_seq > (1L << 25) ||
      rows * p->num_q_heads > (1L << 22) || rows * p->num_idx_heads > (1L << 22))
    return MSA_ERR_UNSUPPORTED;
  d->B = p->batch;
  d->T = p->decode_query_len;
  d->Hq = p->num_q_heads;
  d->Hkv = p->num_kv_heads;
  d->Hidx = p->num_idx_heads;
  d->MAXB = p->max_blocks_per_seq;
  d->NB = p->num_phys_blocks;
  d->topk = p->topk;
  d->kv_dtype = p->kv_dtype;
  d->idx_dtype = p->idx_k_dtype;
  const float scale = p->sm_scale > 0.f ? p->sm_scale : 1.0f / sqrtf((float)p->head_dim);
  d->scale_log2 = scale * 1.4426950408889634f;
  d->debug = (p->flags & MSA_FLAG_DEBUG_CHECKS) != 0;
  return MSA_OK;
}

int check_ptr(const void* p) {
  if (!p) return MSA_ERR_INVALID_ARG;
  return aligned16(p) ? MSA_OK : MSA_ERR_INVALID_ARG;
}

int check_index_inputs(const Dims& d, const msa_tensors* t) {
  if (!t) return MSA_ERR_INVALID_ARG;
  int e;
  if ((e = check_ptr(t->idx_q)) || (e = check_ptr(t->idx_k_pool)) ||
      (e = check_ptr(t->block_table)) || (e = check_ptr(t->ctx_lens)))
    return e;
  if (d.idx_dtype == MSA_DTYPE_NVFP4 && (e = check_ptr(t->idx_k_scale))) return e;
  return MSA_OK;
}

int check_kv_inputs(const Dims& d, const msa_tensors* t) {
  if (!t) return MSA_ERR_INVALID_ARG;
  int e;
  if ((e = check_ptr(t->q)) || (e = check_ptr(t->k_pool)) || (e = check_ptr(t->v_pool)) ||
      (e = check_ptr(t->ctx_lens)))
    return e;
  if (d.kv_dtype != MSA_DTYPE_BF16) {
    if ((e = check_ptr(t->k_scale)) || (e = check_ptr(t->v_scale))) return e;
  }
  return MSA_OK;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MSA_OK;
  g_last_hip_error = (int)e;
  return MSA_ERR_HIP;
}

// With MSA_FLAG_DEBUG_CHECKS: checks the data-dependent inputs of a call
// (synchronising `s`) and returns MSA_ERR_BAD_DATA, before any other launch,
// when one is invalid.  Without the flag: nothing.
int debug_checks(const Dims& d, const int32_t* ctx_lens, const int32_t* block_table,
                 const int32_t* selected, const int32_t* page_table, bool new_tokens_only,
                 hipStream_t s, std::string* note) {
  if (!d.debug) return MSA_OK;
  const CheckInputs a = {ctx_lens, block_table, selected, page_table, d.B, d.T, d.MAXB, d.NB,
                         d.topk, new_tokens_only};
  std::string failure;
  const int e = hip_status(run_input_checks(a, s, &failure));
  if (e) return e;
  if (!failure.empty()) {
    g_last_check_failure = failure;
    return MSA_ERR_BAD_DATA;
  }
  *note += "input_checks[1x1024] ";
  return MSA_OK;
}

// msa_decode on a workspace already validated for presence: the index scan,
// the selection (its own launch, or inside the attention launch for
// single-row requests), the attention and its merge.
int decode_with_workspace(const Dims& d, const msa_tensors* t, int32_t* selected,
                          int32_t* page_table, float* out, void* workspace,
                          size_t workspace_bytes, hipStream_t s) {
  int e;
  if ((e = check_index_inputs(d, t)) || (e = check_kv_inputs(d, t)) || (e = check_ptr(out)))
    return e;
  if ((selected && !aligned16(selected)) || (page_table && !aligned16(page_table)))
    return MSA_ERR_INVALID_ARG;
  const Workspace w = workspace_layout(d);
  if (workspace_bytes < w.total) return MSA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  float* scores = reinterpret_cast<float*>(ws + w.scores);
  int32_t* nsel = reinterpret_cast<int32_t*>(ws + w.n_selected);
  int32_t* sel = selected ? selected : reinterpret_cast<int32_t*>(ws + w.selected);
  int32_t* pt = page_table ? page_table : reinterpret_cast<int32_t*>(ws + w.page_table);
  std::string note;
  if ((e = debug_checks(d, t->ctx_lens, t->block_table, nullptr, nullptr, false, s, &note)))
    return e;
  if ((e = hip_status(launch_index_scan(d, t->idx_q, t->idx_k_pool, t->idx_k_scale,
                                        t->block_table, t->ctx_lens, scores, s, &note))))
    return e;
  note += " ";
  // Single-row requests, and multi-row requests that walk their union,
  // select inside the attention launch (one launch fewer on the dependent
  // chain); the rest select in a launch of their own.
  const bool fuse = fused_select_eligible(d);
  const SelectArgs fused{scores, t->block_table, selected, nullptr, page_table};
  if (!fuse) {
    if ((e = hip_status(launch_select(d, scores, t->ctx_lens, t->block_table, sel, nsel, pt, s,
                                      &note))))
      return e;
    note += " ";
  }
  if ((e = hip_status(launch_sparse_attention(d, t->q, t->k_pool, t->v_pool, t->k_scale,
                                              t->v_scale, pt, t->ctx_lens,
                                              reinterpret_cast<float*>(ws + w.part_o),
                                              reinterpret_cast<float*>(ws + w.part_ml), out, s,
                                              &note, fuse ? &fused : nullptr))))
    return e;
  g_last_dispatch = note;
  return MSA_OK;
}

// ---- the workspace of msa_decode_noalloc (the array `scratch` above)
constexpr size_t kScratchBytes = MSA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

// The array's address on the device that runs `stream` (the current device
// for the null stream), taken once per device with that device current.
hipError_t scratch_of_stream_device(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      int cur = 0;
      if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
      if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(::scratch));
      if (cur != dev) {
        const hipError_t back = hipSetDevice(cur);
        if (e == hipSuccess) e = back;
      }
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace
}  // namespace msa

using namespace msa;

extern "C" {

int msa_index_score(const msa_problem* p, const msa_tensors* t, float* block_scores,
                    void* stream) {
  Dims d;
  int e;
  if ((e = check_problem(p, &d))) return e;
  if ((e = check_index_inputs(d, t)) || (e = check_ptr(block_scores))) return e;
  std::string note;
  if ((e = debug_checks(d, t->ctx_lens, t->block_table, nullptr, nullptr, false,
                        (hipStream_t)stream, &note)))
    return e;
  e = hip_status(launch_index_scan(d, t->idx_q, t->idx_k_pool, t->idx_k_scale, t->block_table,
                                   t->ctx_lens, block_scores, (hipStream_t)stream, &note));
  if (e == MSA_OK) g_last_dispatch = note;
  return e;
}

int msa_select_blocks(const msa_problem* p, const float* block_scores, const int32_t* ctx_lens,
                      int32_t* selected, int32_t* n_selected, void* stream) {
  Dims d;
  int e;
  if ((e = check_problem(p, &d))) return e;
  if ((e = check_ptr(block_scores)) || (e = check_ptr(ctx_lens)) || (e = check_ptr(selected)) ||
      (e = check_ptr(n_selected)))
    return e;
  std::string note;
  if ((e = debug_checks(d, ctx_lens, nullptr, nullptr, nullptr, false, (hipStream_t)stream,
                        &note)))
    return e;
  e = hip_status(launch_select(d, block_scores, ctx_lens, nullptr, selected, n_selected, nullptr,
                               (hipStream_t)stream, &note));
  if (e == MSA_OK) g_last_dispatch = note;
  return e;
}

int msa_build_page_table(const msa_problem* p, const int32_t* selected,
                         const int32_t* block_table, int32_t* page_table, void* stream) {
  Dims d;
  int e;
  if ((e = check_problem(p, &d))) return e;
  if ((e = check_ptr(selected)) || (e = check_ptr(block_table)) || (e = check_ptr(page_table)))
    return e;
  std::string note;
  if ((e = debug_checks(d, nullptr, block_table, selected, nullptr, false, (hipStream_t)stream,
                        &note)))
    return e;
  e = hip_status(launch_page_table(d, selected, block_table, page_table, (hipStream_t)stream,
                                   &note));
  if (e == MSA_OK) g_last_dispatch = note;
  return e;
}

size_t msa_workspace_bytes(const msa_problem* p) {
  Dims d;
  if (check_problem(p, &d)) return 0;
  return workspace_layout(d).total;
}

int msa_sparse_decode(const msa_problem* p, const msa_tensors* t, const int32_t* page_table,
                      float* out, void* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  int e;
  if ((e = check_problem(p, &d))) return e;
  if ((e = check_kv_inputs(d, t)) || (e = check_ptr(page_table)) || (e = check_ptr(out)) ||
      (e = check_ptr(workspace)))
    return e;
  const Workspace w = workspace_layout(d);
  if (workspace_bytes < w.total) return MSA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  std::string note;
  if ((e = debug_checks(d, t->ctx_lens, nullptr, nullptr, page_table, false, (hipStream_t)stream,
                        &note)))
    return e;
  e = hip_status(launch_sparse_attention(d, t->q, t->k_pool, t->v_pool, t->k_scale, t->v_scale,
                                         page_table, t->ctx_lens,
                                         reinterpret_cast<float*>(ws + w.part_o),
                                         reinterpret_cast<float*>(ws + w.part_ml), out,
                                         (hipStream_t)stream, &note));
  if (e == MSA_OK) g_last_dispatch = note;
  return e;
}

int msa_decode(const msa_problem* p, const msa_tensors* t, int32_t* selected,
               int32_t* page_table, float* out, void* workspace, size_t workspace_bytes,
               void* stream) {
  Dims d;
  int e;
  if ((e = check_problem(p, &d))) return e;
  if ((e = check_ptr(workspace))) return e;
  return decode_with_workspace(d, t, selected, page_table, out, workspace, workspace_bytes,
                               (hipStream_t)stream);
}

int msa_decode_noalloc(const msa_problem* p, const msa_tensors* t, int32_t* selected,
                       int32_t* page_table, float* out, void* stream) {
  Dims d;
  int e;
  if ((e = check_problem(p, &d))) return e;
  if (workspace_layout(d).total > kScratchBytes) return MSA_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((e = hip_status(scratch_of_stream_device((hipStream_t)stream, &ws)))) return e;
  return decode_with_workspace(d, t, selected, page_table, out, ws, kScratchBytes,
                               (hipStream_t)stream);
}

int msa_insert_kv(const msa_problem* p, const msa_pools* pools, const int32_t* block_table,
                  const int32_t* ctx_lens, const void* k_new, const void* v_new,
                  const void* idx_k_new, void* stream) {
  Dims d;
  int e;
  if ((e = check_problem(p, &d))) return e;
  if (!pools) return MSA_ERR_INVALID_ARG;
  if ((e = check_ptr(pools->k_pool)) || (e = check_ptr(pools->v_pool)) ||
      (e = check_ptr(pools->idx_k_pool)) || (e = check_ptr(block_table)) ||
      (e = check_ptr(ctx_lens)) || (e = check_ptr(k_new)) || (e = check_ptr(v_new)) ||
      (e = check_ptr(idx_k_new)))
    return e;
  if (d.kv_dtype != MSA_DTYPE_BF16 &&
      ((e = check_ptr(pools->k_scale)) || (e = check_ptr(pools->v_scale))))
    return e;
  if (d.idx_dtype == MSA_DTYPE_NVFP4 && (e = check_ptr(pools->idx_k_scale))) return e;
  const InsertPools pl = {pools->k_pool, pools->v_pool, pools->k_scale, pools->v_scale,
                          pools->idx_k_pool, pools->idx_k_scale};
  std::string note;
  if ((e = debug_checks(d, ctx_lens, block_table, nullptr, nullptr, true, (hipStream_t)stream,
                        &note)))
    return e;
  e = hip_status(launch_insert(d, k_new, v_new, idx_k_new, block_table, ctx_lens, pl,
                               (hipStream_t)stream, &note));
  if (e == MSA_OK) g_last_dispatch = note;
  return e;
}

const char* msa_status_string(int status) {
  switch (status) {
    case MSA_OK: return "ok";
    case MSA_ERR_INVALID_ARG: return "invalid argument";
    case MSA_ERR_UNSUPPORTED: return "unsupported dtype or shape";
    case MSA_ERR_WORKSPACE:
      return "workspace too small (msa_decode_noalloc: the problem needs more than "
             "MSA_NOALLOC_SCRATCH_BYTES)";
    case MSA_ERR_HIP: return "HIP launch failed";
    case MSA_ERR_BAD_DATA: return "input data failed a debug check";
    default: return "unknown status";
  }
}

int msa_last_hip_error(void) { return g_last_hip_error; }

int msa_last_check_failure(char* buf, size_t n) {
  const std::string& s = g_last_check_failure;
  if (buf && n > 0) {
    const size_t k = s.size() < n - 1 ? s.size() : n - 1;
    memcpy(buf, s.data(), k);
    buf[k] = '\0';
  }
  return (int)s.size();
}

int msa_last_dispatch(char* buf, size_t n) {
  const std::string& s = g_last_dispatch;
  if (buf && n > 0) {
    const size_t k = s.size() < n - 1 ? s.size() : n - 1;
    memcpy(buf, s.data(), k);
    buf[k] = '\0';
  }
  return (int)s.size();
}

int msa_selftest_decoders(float* out, void* stream) {
  if (check_ptr(out)) return MSA_ERR_INVALID_ARG;
  return hip_status(launch_selftest_decoders(out, (hipStream_t)stream));
}

}  // extern "C"
