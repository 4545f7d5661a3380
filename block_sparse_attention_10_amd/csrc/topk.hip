// Steps 2 and 3 of MSA decode: top-k block selection and the page table.
//
// aisoku.org MiniMax-M3.1-Flash article, section "MSAの仕組み", and the
// agentlenshq page, section "MSA 実行プロセス" step 2 (local_blocks = 1): each
// row keeps its local block (the one holding the query token) plus the best
// of the other causal blocks, topk blocks in all.  Ties go to the lower block
// id; the kept ids are emitted ascending.  news.ainew.jp MI355X article,
// section 2: one workgroup per request covers all draft positions.
// news.ainew.jp article, section 3 and Figure 5: each kept block is resolved
// to its physical block and expanded to 8 page ids of 16 tokens; KV stays in
// place, only this table is rebuilt.
//
// Design: one 256-thread workgroup per request; the selection itself (a
// threshold that leaves a few dozen candidates per row, ranked by counting
// in LDS, with a per-lane sorted-list path as the fallback) is described in
// select_device.h.
#include "msa_device.h"
#include "msa_internal.h"
#include "select_device.h"

namespace msa {
namespace {

template <int NW>
__global__ __launch_bounds__(64 * NW) void select_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ ctx_lens,
    const int32_t* __restrict__ block_table, int32_t* __restrict__ selected,
    int32_t* __restrict__ n_selected, int32_t* __restrict__ page_table, int T, int MAXB,
    int topk) {
  __shared__ SelectLds<NW> sh;
  select_request<NW>(blockIdx.x, scores, ctx_lens, block_table, selected, n_selected,
                     page_table, T, MAXB, topk, sh);
}

__global__ __launch_bounds__(256) void page_table_kernel(const int32_t* __restrict__ selected,
                                                         const int32_t* __restrict__ block_table,
                                                         int32_t* __restrict__ page_table,
                                                         int R, int T, int MAXB, int topk) {
  const int pt = topk * 8;
  const long e = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (long)R * pt) return;
  const int r = (int)(e / pt);
  const int slot = (int)(e - (long)r * pt);
  const int c = selected[(size_t)r * topk + (slot >> 3)];
  int v = -1;
  // a selected id past the table row reads the row's last entry
  if (c >= 0) v = block_table[(size_t)(r / T) * MAXB + min(c, MAXB - 1)] * 8 + (slot & 7);
  page_table[e] = v;
}

}  // namespace

// Rows of at least this many blocks (single-row requests) select with 8
// waves per request.
constexpr int kLongRowBlocks = 2048;

hipError_t launch_select(const Dims& d, const float* scores, const int32_t* ctx_lens,
                         const int32_t* block_table, int32_t* selected, int32_t* n_selected,
                         int32_t* page_table, hipStream_t s, std::string* note) {
  // single-row requests with long rows: 8 waves, so that each lane holds
  // half as many candidates
  const int nw = d.T == 1 && d.MAXB >= kLongRowBlocks ? 8 : 4;
  if (nw == 8)
    hipLaunchKernelGGL((select_kernel<8>), dim3(d.B), dim3(512), 0, s, scores, ctx_lens,
                       block_table, selected, n_selected, page_table, d.T, d.MAXB, d.topk);
  else
    hipLaunchKernelGGL((select_kernel<4>), dim3(d.B), dim3(256), 0, s, scores, ctx_lens,
                       block_table, selected, n_selected, page_table, d.T, d.MAXB, d.topk);
  if (note)
    *note += std::string("select_topk[grid=") + std::to_string(d.B) + "x" +
             std::to_string(64 * nw) + (page_table ? ",+pages]" : "]");
  return hipGetLastError();
}

hipError_t launch_page_table(const Dims& d, const int32_t* selected, const int32_t* block_table,
                             int32_t* page_table, hipStream_t s, std::string* note) {
  const long n = (long)d.R() * d.PT();
  const unsigned grid = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(page_table_kernel, dim3(grid), dim3(256), 0, s, selected, block_table,
                     page_table, d.R(), d.T, d.MAXB, d.topk);
  if (note) *note += "page_table[grid=" + std::to_string(grid) + "x256]";
  return hipGetLastError();
}

}  // namespace msa
