// Host-side launchers shared by the translation units of libmsa.  Each
// kernel file owns its kernels and exposes one launcher; api.hip validates
// arguments, lays out the workspace and calls them.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>

namespace msa {

// Dimensions of one call, already validated.
struct Dims {
  int B, T, Hq, Hkv, Hidx, MAXB, NB, topk;
  int kv_dtype, idx_dtype;
  float scale_log2;  // softmax scale * log2(e)
  bool debug;        // MSA_FLAG_DEBUG_CHECKS
  int R() const { return B * T; }
  int G() const { return Hq / Hkv; }
  int PT() const { return topk * 8; }  // page-table row length
};

// Attention plan: one workgroup of `waves` waves per (row, KV head, split);
// the `splits` workgroups of a (row, KV head) share its chunks of 32 keys.
struct SplitPlan {
  int waves;   // waves per workgroup: 4 or 8
  int splits;  // workgroups per (row, KV head), or per (request, KV head) with rows_union
  // multi-row requests: one workgroup walks the union of the request's rows'
  // blocks for all of them (rows x query heads of the KV head as columns)
  bool rows_union;
  int tiles;   // 16-column MFMA tiles of a rows_union workgroup (1 or 2)
};
SplitPlan plan_splits(const Dims& d);

// Workspace carve-up (byte offsets, 256-aligned).
struct Workspace {
  size_t part_o, part_ml, scores, n_selected, selected, page_table, total;
};
Workspace workspace_layout(const Dims& d);

hipError_t launch_index_scan(const Dims& d, const void* idx_q, const void* idx_k,
                             const void* idx_k_scale, const int32_t* block_table,
                             const int32_t* ctx_lens, float* scores, hipStream_t s,
                             std::string* note);

hipError_t launch_select(const Dims& d, const float* scores, const int32_t* ctx_lens,
                         const int32_t* block_table, int32_t* selected, int32_t* n_selected,
                         int32_t* page_table, hipStream_t s, std::string* note);

hipError_t launch_page_table(const Dims& d, const int32_t* selected, const int32_t* block_table,
                             int32_t* page_table, hipStream_t s, std::string* note);

// Inputs of the selection an attention workgroup runs itself when the
// selection is fused into the attention launch (single-row requests, and
// multi-row requests that walk their union).  The (KV head 0, split 0)
// workgroup of each row (request) exports its selection and page ids to
// selected / n_selected / page_table when those are not null.
struct SelectArgs {
  const float* scores;
  const int32_t* block_table;
  int32_t* selected;
  int32_t* n_selected;
  int32_t* page_table;
};

// True when msa_decode selects inside the attention launch for `d`.
bool fused_select_eligible(const Dims& d);

// One launch when a workgroup covers a whole (row, KV head); otherwise the
// split partials land in part_o / part_ml and a merge launch follows.  With
// `sel` (fused_select_eligible(d) must hold) the workgroups select their
// row's blocks from the block scores first and page_table is not read.
hipError_t launch_sparse_attention(const Dims& d, const void* q, const void* k_pool,
                                   const void* v_pool, const void* k_scale,
                                   const void* v_scale, const int32_t* page_table,
                                   const int32_t* ctx_lens, float* part_o, float* part_ml,
                                   float* out, hipStream_t s, std::string* note,
                                   const SelectArgs* sel = nullptr);

// Pools the write path fills (layouts as the attention reads them).
struct InsertPools {
  void* k_pool;
  void* v_pool;
  void* k_scale;
  void* v_scale;
  void* idx_k_pool;
  void* idx_k_scale;
};

hipError_t launch_insert(const Dims& d, const void* k_new, const void* v_new,
                         const void* idx_new, const int32_t* block_table,
                         const int32_t* ctx_lens, const InsertPools& pools, hipStream_t s,
                         std::string* note);

hipError_t launch_selftest_decoders(float* out, hipStream_t s);

// Data-dependent inputs one call reads (NULL: not read by that call).
struct CheckInputs {
  const int32_t* ctx_lens;
  const int32_t* block_table;
  const int32_t* selected;
  const int32_t* page_table;
  int B, T, MAXB, NB, topk;
  bool new_tokens_only;  // table entries of the T newest tokens' blocks only
};

// Runs the input checks on `s`, waits for them, and leaves in `failure` a
// description of the first violation ("" when the inputs are valid).
hipError_t run_input_checks(const CheckInputs& a, hipStream_t s, std::string* failure);

}  // namespace msa
