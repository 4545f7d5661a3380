/*
 * msa.h -- C ABI of libmsa: MiniMax Sparse Attention (MSA) decode on AMD
 * Instinct MI355X (gfx950).
 *
 * The path, per query token (row), follows the three-step process of the
 * agentlenshq page "MiniMax M3 vLLM サポート: 1M トークンマルチモーダル推論の
 * Day-0 サービング", section "MSA 実行プロセス":
 *   1. msa_index_score      small index heads score every 128-token KV block;
 *   2. msa_select_blocks    top-k blocks (16), the block holding the query
 *                           token always among them (local_blocks = 1), which
 *                           caps a query at 2,048 keys (aisoku.org
 *                           MiniMax-M3.1-Flash article, section "MSAの仕組み");
 *   3. msa_build_page_table each selected block is resolved to its physical
 *                           block and expanded to 8 page ids of 16 tokens, KV
 *                           left in place (news.ainew.jp MI355X article,
 *                           section 3 "どのバイトが移動するのか", Figure 5);
 *   4. msa_sparse_decode    exact split-K online-softmax GQA attention over
 *                           the pages of that table, partials merged by
 *                           log-sum-exp (agentlenshq page, section "EAGLE3 を
 *                           用いた投機的デコード": a decode split-K path that
 *                           takes a unified decode_query_len);
 *   msa_decode runs 1-4 in one call.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers to row-major, contiguous data,
 *    owned by the caller.  The library allocates nothing on any call, keeps
 *    no pointer after it returns, and launches work asynchronously on
 *    `stream` (a hipStream_t passed as void*; NULL = the null stream).
 *    Outputs are valid once the stream has reached the end of the call.
 *  - Row r = b * T + t is query position t (0 <= t < T = decode_query_len)
 *    of request b.  Its position in the sequence is p = ctx_lens[b] - T + t
 *    and it attends causally up to and including p (draft positions of a
 *    speculative-verify step each see only their own prefix: news.ainew.jp
 *    article, section "EAGLE3 が第 2 のデコードループを追加").  ctx_lens[b]
 *    must be >= T and <= max_blocks_per_seq * block_size.
 *  - Layouts (NB = num_phys_blocks, MAXB = max_blocks_per_seq, R = B * T):
 *      q           [R][Hq][head_dim]                bf16
 *      idx_q       [R][Hidx][idx_dim]               bf16
 *      idx_k_pool  [NB][Hidx][block_size][idx_dim]  bf16 or fp8 e4m3 codes, or
 *                  [NB][Hidx][block_size][idx_dim/2] bytes of two e2m1 codes
 *                  (MSA_DTYPE_NVFP4, element 2j in the low nibble) with
 *      idx_k_scale [NB][Hidx][block_size][idx_dim/16] e4m3 codes, one per 16
 *                  consecutive elements (NULL for the other index dtypes)
 *      k_pool, v_pool
 *        MSA_DTYPE_BF16     [NB][Hkv][block_size][head_dim] bf16
 *        MSA_DTYPE_FP8_E4M3 [NB][Hkv][block_size][head_dim] e4m3 codes, and
 *                           k_scale, v_scale [NB][Hkv][block_size] fp32, one
 *                           dequantisation factor per token and KV head
 *        MSA_DTYPE_NVFP4    [NB][Hkv][block_size][head_dim/2] bytes, two e2m1
 *                           codes each (element 2j in the low nibble), and
 *                           k_scale, v_scale [NB][Hkv][block_size][head_dim/16]
 *                           e4m3 codes, one per 16 consecutive elements
 *      block_table [B][MAXB] int32 physical block of logical block c
 *      ctx_lens    [B]       int32
 *      block_scores[R][MAXB] fp32
 *      selected    [R][topk] int32 logical block ids, ascending, -1 padded
 *      n_selected  [R]       int32
 *      page_table  [R][topk * block_size / page_size] int32, -1 padded;
 *                  page id = physical block * 8 + j
 *      out         [R][Hq][head_dim] fp32
 *    Every pointer must be 16-byte aligned.  GQA: query head h reads KV head
 *    h / (Hq / Hkv).  fp8 is OCP E4M3FN; the 4-bit format is OCP E2M1.
 *  - Supported shape: head_dim 128, idx_dim 64, block_size 128, page_size 16,
 *    local_blocks 1, 1 <= topk <= 16, 1 <= Hq/Hkv <= 16, 1 <= T <= 16,
 *    1 <= Hidx <= 16; MAXB <= 2^24 (the blocks of the longest int32
 *    context), NB <= 2^28 (page ids fit int32), B * MAXB <= 2^25,
 *    B * T * Hq <= 2^22 and B * T * Hidx <= 2^22 (every launch below 2^32
 *    work-items).  Anything else returns MSA_ERR_UNSUPPORTED.
 *  - Return codes: MSA_OK when every launch was enqueued; MSA_ERR_INVALID_ARG
 *    for a NULL pointer, a misaligned pointer or an inconsistent dimension;
 *    MSA_ERR_UNSUPPORTED for a dtype or shape outside the list above;
 *    MSA_ERR_WORKSPACE for a workspace smaller than msa_workspace_bytes();
 *    MSA_ERR_HIP when a launch failed (msa_last_hip_error() gives the HIP
 *    code); MSA_ERR_BAD_DATA when a debug check failed (below).  No
 *    exception crosses this boundary.
 *  - Data-dependent inputs (ctx_lens outside the bounds above, block_table
 *    entries outside [0, NB), selections or page tables not of the form
 *    described) are not checked by default and give undefined results.
 *    The kernels clamp every physical block id they dereference to [0, NB)
 *    and every logical block to the table row, so such inputs read or write
 *    wrong entries of the caller's pools but no memory outside them.
 *    With flags = MSA_FLAG_DEBUG_CHECKS every call first checks, on the
 *    device, the ctx_lens, block_table entries, selected ids and page-table
 *    rows it reads (for the write path: the table entries of the new
 *    tokens' blocks; elsewhere every block of the context), waits for that
 *    check (the call synchronises `stream`, so it cannot be captured into a
 *    graph), and returns MSA_ERR_BAD_DATA without launching anything else
 *    when an input is invalid; msa_last_check_failure() names the first
 *    offending entry.  Checks of calls on one device are serialised.
 *  - Calls on different streams must use distinct workspaces and outputs.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = -1,
  MSA_ERR_UNSUPPORTED = -2,
  MSA_ERR_WORKSPACE = -3,
  MSA_ERR_HIP = -4,
  MSA_ERR_BAD_DATA = -5
};

/* msa_problem.flags */
enum { MSA_FLAG_DEBUG_CHECKS = 1 };

enum { MSA_DTYPE_BF16 = 0, MSA_DTYPE_FP8_E4M3 = 1, MSA_DTYPE_NVFP4 = 2 };

typedef struct msa_problem {
  uint32_t struct_size;       /* sizeof(msa_problem)                          */
  int32_t batch;              /* B requests                                   */
  int32_t decode_query_len;   /* T: 1 + number of draft positions             */
  int32_t num_q_heads;        /* Hq                                           */
  int32_t num_kv_heads;       /* Hkv (Hq % Hkv == 0)                          */
  int32_t num_idx_heads;      /* Hidx                                         */
  int32_t head_dim;           /* 128                                          */
  int32_t idx_dim;            /* 64                                           */
  int32_t block_size;         /* 128 tokens per KV block                      */
  int32_t page_size;          /* 16 tokens per page                           */
  int32_t topk;               /* blocks kept per row, local block included    */
  int32_t local_blocks;       /* 1                                            */
  int32_t max_blocks_per_seq; /* MAXB: row length of block_table              */
  int32_t num_phys_blocks;    /* NB: blocks in each pool                      */
  int32_t kv_dtype;           /* MSA_DTYPE_BF16 / _FP8_E4M3 / _NVFP4          */
  int32_t idx_k_dtype;        /* MSA_DTYPE_BF16 / _FP8_E4M3 / _NVFP4          */
  float sm_scale;             /* softmax scale; 0 means 1/sqrt(head_dim)      */
  uint32_t flags;             /* 0 or MSA_FLAG_DEBUG_CHECKS                   */
} msa_problem;

typedef struct msa_tensors {
  const void* q;              /* bf16                                         */
  const void* idx_q;          /* bf16                                         */
  const void* k_pool;
  const void* v_pool;
  const void* k_scale;        /* NULL for bf16 KV                             */
  const void* v_scale;        /* NULL for bf16 KV                             */
  const void* idx_k_pool;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  const void* idx_k_scale;    /* 4-bit index keys only, else NULL             */
} msa_tensors;

/* Step 1, block scoring (agentlenshq page, section "MSA 実行プロセス", step 1).
 * block_scores[r][c] = max over tokens i of logical block c with i <= p of
 * sum over index heads h and dims d of idx_q[r][h][d] * k_idx[i][h][d]
 * (no scale, no activation), accumulated in fp32; -inf for c > p / 128.
 * 4-bit keys are e2m1 code x e4m3 scale; the dot product is summed per
 * group of 16 dims and each group sum scaled (exact whenever products and
 * partial sums fit fp32, as for integer queries and power-of-two scales).
 * Reads t->idx_q, t->idx_k_pool, t->idx_k_scale (4-bit keys),
 * t->block_table, t->ctx_lens.  One launch. */
int msa_index_score(const msa_problem* p, const msa_tensors* t, float* block_scores,
                    void* stream);

/* Step 2, top-k selection (aisoku.org article, section "MSAの仕組み";
 * agentlenshq page, section "MSA 実行プロセス", step 2; news.ainew.jp article,
 * section 2 on one indexer workgroup per request).  With l = p / 128, rows
 * with l + 1 <= topk keep blocks 0..l; otherwise block l plus the topk - 1
 * best of blocks 0..l-1 ordered by score (descending), equal scores to the
 * lower id, NaN as -inf, -0 equal to +0.  selected is written ascending and
 * -1 padded; n_selected receives the count.  One workgroup per request
 * handles all T rows.  One launch. */
int msa_select_blocks(const msa_problem* p, const float* block_scores, const int32_t* ctx_lens,
                      int32_t* selected, int32_t* n_selected, void* stream);

/* Step 3, page table (news.ainew.jp article, section 3 and Figure 5):
 * page_table[r][8k + j] = block_table[b][selected[r][k]] * 8 + j for each
 * selected block k, -1 elsewhere.  One launch. */
int msa_build_page_table(const msa_problem* p, const int32_t* selected,
                         const int32_t* block_table, int32_t* page_table, void* stream);

/* Step 4, sparse GQA attention (aisoku.org article, section "MSAの仕組み";
 * agentlenshq page, "MSA 実行プロセス" step 3 and "EAGLE3 を用いた投機的デコード").
 * page_table rows must be as msa_build_page_table writes them: the pages of
 * the row's blocks in ascending logical order, the local block last.  Key n
 * of the row (n-th token of the concatenated pages) is attended iff
 * n < 128 * (blocks - 1) + (p mod 128) + 1.  out = softmax(q K^T * scale) V
 * per query head, computed split-K with fp32 partials in `workspace` and
 * merged by log-sum-exp.  Reads t->q, t->k_pool, t->v_pool, t->k_scale,
 * t->v_scale, t->ctx_lens.  Page ids are clamped to the pools.  One launch,
 * plus a merge launch when a row is split over several workgroups.
 * Cross-layer reuse (news.ainew.jp article, section 3, on index sharing:
 * adjacent sparse layers pick nearly the same blocks, so one layer selects
 * and later layers reuse its top-k): call this with a later layer's q and
 * pools and the page table an earlier layer's msa_decode exported; layers
 * share the block table, so the page ids hold in every layer's pool. */
int msa_sparse_decode(const msa_problem* p, const msa_tensors* t, const int32_t* page_table,
                      float* out, void* workspace, size_t workspace_bytes, void* stream);

/* Pools the write path fills: the same buffers and layouts as in
 * msa_tensors, writable.  Scale pools are NULL for bf16 data. */
typedef struct msa_pools {
  void* k_pool;
  void* v_pool;
  void* k_scale;
  void* v_scale;
  void* idx_k_pool;
  void* idx_k_scale;
} msa_pools;

/* The write path that fills the pools this path reads (news.ainew.jp
 * article, section 3: the fused projection writes each new token's index
 * key into the index cache; aisoku.org article, section "何が新しいか": KV
 * kept as fp8 / NVFP4).  Row r = b * T + t is the token at position
 * p = ctx_lens[b] - T + t (ctx_lens already counts it); its K and V
 * (k_new, v_new [R][Hkv][head_dim] bf16) and index key (idx_k_new
 * [R][Hidx][idx_dim] bf16) are written to slot p mod 128 of physical block
 * block_table[b][p / 128], quantised to the pools' dtypes:
 *   fp8 K / V      scale = amax / 448 per (token, head) (1 if amax is 0),
 *                  codes = E4M3 round-to-nearest-even of x / scale;
 *   4-bit K / V / index keys
 *                  per 16 elements scale code = E4M3(amax / 6), codes =
 *                  E2M1 round-to-nearest-even of x / scale (saturating at
 *                  6), all 0 when the scale is 0, negative zero as +0;
 *   fp8 index keys E4M3 code of the value (no scale).
 * Decisions are taken in fp32.  Rows must target distinct slots (a request's
 * T rows do).  Nothing else in the pools changes.  One launch. */
int msa_insert_kv(const msa_problem* p, const msa_pools* pools, const int32_t* block_table,
                  const int32_t* ctx_lens, const void* k_new, const void* v_new,
                  const void* idx_k_new, void* stream);

/* Steps 1-4 in one call: the index scan, the selection with the page table
 * built in the same launch, then the attention (and its merge launch when
 * rows are split).  For single-row requests (decode_query_len 1), and for
 * requests of 2-4 rows whose rows' query heads per KV head number at most
 * 32, with at most 16384 blocks per row, every attention workgroup selects
 * its rows' blocks at its start instead, and the selection launch is
 * skipped.
 * selected / page_table may be NULL; when given they receive the step 2 /
 * step 3 results.  Block scores, counts and any table not supplied live in
 * `workspace`. */
int msa_decode(const msa_problem* p, const msa_tensors* t, int32_t* selected,
               int32_t* page_table, float* out, void* workspace, size_t workspace_bytes,
               void* stream);

/* Size of the per-device array msa_decode_noalloc takes its workspace from. */
#define MSA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* msa_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments, launches and results as msa_decode, without the
 * workspace argument.  The workspace is a MSA_NOALLOC_SCRATCH_BYTES (16 MiB)
 * array the library holds on each device it runs on, from the first call
 * on that device until the process ends; problems whose
 * msa_workspace_bytes() exceed it return MSA_ERR_WORKSPACE (the batch must
 * be split).  The call allocates nothing.  All calls on one device share
 * that device's array, so calls that overlap on one device (on different
 * streams or from different host threads) race and must be serialised by
 * the caller; the array needs no clearing between calls (every byte the
 * kernels read was written earlier in the same call).  Runs on the device
 * of `stream` (the current device for the null stream) and uses that
 * device's array. */
int msa_decode_noalloc(const msa_problem* p, const msa_tensors* t, int32_t* selected,
                       int32_t* page_table, float* out, void* stream);

/* Bytes of device workspace msa_sparse_decode and msa_decode need for this
 * problem (a multiple of 256; 0 for an invalid problem).  The workspace is
 * scratch owned by the caller; its contents need no initialisation. */
size_t msa_workspace_bytes(const msa_problem* p);

/* Static text for a return code. */
const char* msa_status_string(int status);

/* HIP error code of the last MSA_ERR_HIP on the calling thread (0 if none). */
int msa_last_hip_error(void);

/* Describes the first invalid input found by the debug checks of the
 * calling thread's last call that returned MSA_ERR_BAD_DATA (which entry,
 * its value and the rule it breaks).  Copies at most n - 1 bytes plus a
 * terminating NUL into buf; returns the full length (0 if none). */
int msa_last_check_failure(char* buf, size_t n);

/* Names the kernels and launch shapes the calling thread's last successful
 * call enqueued (what was executed, not just configured).  Copies at most
 * n - 1 bytes plus a terminating NUL into buf; returns the full length. */
int msa_last_dispatch(char* buf, size_t n);

/* Diagnostics: decode every OCP E4M3 and E2M1 code with the device decoders
 * the kernels use, into out[832] fp32 (device pointer, 16-byte aligned):
 *   out[c]            E4M3 code c (0..255) via the bf16 path (K/V, index keys)
 *   out[256 + c]      E2M1 code c (0..15) in the low nibble of a byte (fp32)
 *   out[272 + c]      E2M1 code c (0..15) in the high nibble of a byte (fp32)
 *   out[288 + c]      E4M3 code c (0..255) via the fp32 path (4-bit scales)
 *   out[544 + c]      E2M1 code c in the low nibble, bf16 path (index keys)
 *   out[560 + c]      E2M1 code c in the high nibble, bf16 path
 *   out[576 + c]      E4M3 code c (0..255) as the second code of an fp32 pair
 * One launch. */
int msa_selftest_decoders(float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H_ */
