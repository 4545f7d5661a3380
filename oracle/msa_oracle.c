/*
 * msa_oracle.c -- plain CPU oracle for MiniMax Sparse Attention (MSA) decode.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke entry and the benchmark's CPU-baseline leg load it; the product
 * path never does.  It shares no code, header, table or helper with the GPU
 * library: every format decoder below is written from the format definition.
 *
 * Sources (web pages; cited by title and section):
 *  [P1] aisoku.org, "MiniMax-M3.1-Flash Day-0 support in vLLM", section
 *       "MSAの仕組み" (how MSA works): KV cache cut into 128-token blocks, a
 *       light indexer picks the top 16 blocks together with the most recent
 *       block, exact attention runs only there, at most 2,048 keys per query.
 *  [P2] agentlenshq, "MiniMax M3 vLLM サポート: 1M トークンマルチモーダル推論の
 *       Day-0 サービング", section "MSA 実行プロセス" (three steps: block
 *       scoring by small index heads, top-k block selection with
 *       local_blocks=1, online-softmax sparse GQA over the chosen blocks) and
 *       section "EAGLE3 を用いた投機的デコード" (unified decode_query_len).
 *  [P3] news.ainew.jp, "vLLM、AMD Instinct MI355X上でMiniMax M3のボトルネック
 *       最適化手法を公開", section 2 "何が繰り返されるコストなのか" (one indexer
 *       workgroup per request for all draft positions; a positive score scale
 *       does not change the top-k order), section 3 "どのバイトが移動するのか"
 *       with Figure 5 (each selected 128-token block resolved to its physical
 *       block and expanded to 8 page ids of 16 tokens; KV stays in place) and
 *       section "EAGLE3 が第 2 のデコードループを追加" (flattened verify rows
 *       mapped to (request, speculative position)).
 *
 * Readings taken where the pages are silent (each listed in the design notes):
 *  - block score = max over the block's causal tokens of the index dot
 *    product summed over index heads; no scale, no activation;
 *  - the local block counts within the 16 (16 x 128 = 2,048-key cap);
 *  - ties go to the lower logical block id; selection output is ascending;
 *  - query row r = b * T + t sits at position p = ctx_len[b] - T + t and is
 *    causal to itself (draft rows of a verify step);
 *  - page id = physical block * 8 + j, j = 0..7;
 *  - softmax scale 1/sqrt(head_dim) unless the caller passes another;
 *  - GQA: query head h reads KV head h / (Hq / Hkv);
 *  - fp8 = OCP E4M3FN; 4-bit KV = E2M1 with one E4M3 scale per 16
 *    consecutive elements along the head dimension, element 2j in the low
 *    nibble of byte j.
 *
 * Everything is computed in double.  Index keys and queries of the synthetic
 * workloads hold small integers, so the double dot products are exact.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- storage formats, decoded from their definitions ------------------ */

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double msa_oracle_bf16_to_double(uint16_t bits) {
  int sign = (bits >> 15) & 1;
  int expo = (bits >> 7) & 0xFF;
  int frac = bits & 0x7F;
  double mag;
  if (expo == 0xFF) {
    mag = frac ? NAN : INFINITY;
  } else if (expo == 0) {
    mag = ldexp((double)frac / 128.0, -126);
  } else {
    mag = ldexp(1.0 + (double)frac / 128.0, expo - 127);
  }
  return sign ? -mag : mag;
}

/* OCP FP8 E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits,
 * subnormals when the exponent field is 0, no infinities, and the all-ones
 * exponent+fraction pattern (0x7F / 0xFF) is NaN.  Largest finite = 448. */
double msa_oracle_e4m3_to_double(uint8_t code) {
  int sign = (code >> 7) & 1;
  int expo = (code >> 3) & 0xF;
  int frac = code & 0x7;
  double mag;
  if (expo == 0xF && frac == 0x7) {
    mag = NAN;
  } else if (expo == 0) {
    mag = ldexp((double)frac / 8.0, -6);
  } else {
    mag = ldexp(1.0 + (double)frac / 8.0, expo - 7);
  }
  return sign ? -mag : mag;
}

/* OCP FP4 E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 fraction bit,
 * subnormal when the exponent field is 0; magnitudes 0,0.5,1,1.5,2,3,4,6. */
double msa_oracle_e2m1_to_double(uint8_t nibble) {
  int sign = (nibble >> 3) & 1;
  int expo = (nibble >> 1) & 0x3;
  int frac = nibble & 0x1;
  double mag;
  if (expo == 0) {
    mag = (double)frac * 0.5;
  } else {
    mag = ldexp(1.0 + (double)frac / 2.0, expo - 1);
  }
  return sign ? -mag : mag;
}

/* ---- problem description ---------------------------------------------- */

enum { ORACLE_BF16 = 0, ORACLE_FP8 = 1, ORACLE_NVFP4 = 2 };

typedef struct {
  int32_t batch;        /* B requests                                   */
  int32_t query_len;    /* T = decode_query_len (1 + draft positions)   */
  int32_t num_q_heads;  /* Hq                                           */
  int32_t num_kv_heads; /* Hkv                                          */
  int32_t num_idx_heads;/* Hidx                                         */
  int32_t head_dim;     /* D (128)                                      */
  int32_t idx_dim;      /* index head dim (64)                          */
  int32_t block_size;   /* tokens per KV block (128)                    */
  int32_t page_size;    /* tokens per page (16)                         */
  int32_t topk;         /* blocks kept per query row (16)               */
  int32_t max_blocks;   /* block_table row length                       */
  int32_t kv_dtype;     /* ORACLE_BF16 / ORACLE_FP8 / ORACLE_NVFP4      */
  int32_t idx_dtype;    /* ORACLE_BF16 / ORACLE_FP8 / ORACLE_NVFP4      */
  double sm_scale;      /* 0 means 1/sqrt(head_dim)                     */
} oracle_problem;

/* Position of query row t of a request with `ctx_len` tokens and T rows. */
static int64_t row_position(int32_t ctx_len, int32_t T, int32_t t) {
  return (int64_t)ctx_len - T + t;
}

/* Index key element (token tok of physical block phys, index head h, dim
 * d): bf16 as is, fp8 e4m3 code as is (no scale), or 4-bit: the E2M1 code
 * times the E4M3 scale of its group of 16 dims (idx_k_scale), the key
 * format the pages name next for the index cache (aisoku.org article,
 * section "何が新しいか": NVFP4 storage). */
static double idx_key_value(const oracle_problem* p, const void* idx_k_pool,
                            const void* idx_k_scale, int64_t phys, int h, int tok, int d) {
  int64_t row = (phys * p->num_idx_heads + h) * p->block_size + tok;
  int E = p->idx_dim;
  if (p->idx_dtype == ORACLE_BF16)
    return msa_oracle_bf16_to_double(((const uint16_t*)idx_k_pool)[row * E + d]);
  if (p->idx_dtype == ORACLE_FP8)
    return msa_oracle_e4m3_to_double(((const uint8_t*)idx_k_pool)[row * E + d]);
  /* 4-bit: byte j of the row holds elements 2j (low nibble), 2j+1 (high). */
  uint8_t byte = ((const uint8_t*)idx_k_pool)[row * (E / 2) + d / 2];
  uint8_t nib = (d & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF);
  uint8_t sc = ((const uint8_t*)idx_k_scale)[row * (E / 16) + d / 16];
  return msa_oracle_e2m1_to_double(nib) * msa_oracle_e4m3_to_double(sc);
}

/* One K or V element, dequantised: bf16 as is; fp8 code times the token's
 * fp32 scale; 4-bit code times the E4M3 scale of its 16-element group. */
static double kv_value(const oracle_problem* p, const void* pool, const void* scale,
                       int64_t phys, int g, int tok, int d) {
  int64_t row = ((phys * p->num_kv_heads + g) * p->block_size) + tok;
  int D = p->head_dim;
  if (p->kv_dtype == ORACLE_BF16)
    return msa_oracle_bf16_to_double(((const uint16_t*)pool)[row * D + d]);
  if (p->kv_dtype == ORACLE_FP8) {
    double code = msa_oracle_e4m3_to_double(((const uint8_t*)pool)[row * D + d]);
    return code * (double)((const float*)scale)[row];
  }
  /* 4-bit: byte j of the row holds elements 2j (low nibble), 2j+1 (high). */
  uint8_t byte = ((const uint8_t*)pool)[row * (D / 2) + d / 2];
  uint8_t nib = (d & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF);
  uint8_t sc = ((const uint8_t*)scale)[row * (D / 16) + d / 16];
  return msa_oracle_e2m1_to_double(nib) * msa_oracle_e4m3_to_double(sc);
}

/* ---- step 1: block scoring -------------------------------------------- */
/* [P2] "MSA 実行プロセス", step 1: small index heads score every candidate
 * 128-token block.  Reading: token score = sum over index heads and dims of
 * q_idx * k_idx; block score = max over the block's tokens that are causal
 * to the row (token position <= row position).  Blocks past the row's local
 * block score -inf.  `rows` lists the query rows to compute (NULL = all);
 * scores is [nrows][max_blocks]. */
int msa_oracle_index_scores(const oracle_problem* p, const uint16_t* idx_q,
                            const void* idx_k_pool, const void* idx_k_scale,
                            const int32_t* block_table,
                            const int32_t* ctx_lens, const int32_t* rows, int32_t nrows,
                            double* scores) {
  int T = p->query_len, H = p->num_idx_heads, E = p->idx_dim, BS = p->block_size;
  int64_t n;
#pragma omp parallel for schedule(dynamic, 1)
  for (n = 0; n < nrows; n++) {
    int32_t r = rows ? rows[n] : (int32_t)n;
    int32_t b = r / T, t = r % T;
    int64_t pos = row_position(ctx_lens[b], T, t);
    int64_t local = pos / BS;
    double* out = scores + n * (int64_t)p->max_blocks;
    for (int64_t c = 0; c < p->max_blocks; c++) {
      if (c > local) { out[c] = -INFINITY; continue; }
      int64_t phys = block_table[(int64_t)b * p->max_blocks + c];
      double best = -INFINITY;
      for (int tok = 0; tok < BS; tok++) {
        if (c * BS + tok > pos) break;
        double s = 0.0;
        for (int h = 0; h < H; h++)
          for (int d = 0; d < E; d++)
            s += msa_oracle_bf16_to_double(idx_q[((int64_t)r * H + h) * E + d]) *
                 idx_key_value(p, idx_k_pool, idx_k_scale, phys, h, tok, d);
        if (s > best) best = s;
      }
      out[c] = best;
    }
  }
  return 0;
}

/* ---- step 2: top-k selection with the forced local block --------------- */
/* [P1] "MSAの仕組み" and [P2] "MSA 実行プロセス", step 2 (local_blocks=1):
 * keep the block holding the query token plus the best-scoring others, 16
 * blocks in all (16 x 128 = 2,048 keys).  If the row has at most 16 causal
 * blocks, all of them are kept.  Order among the others: higher score first,
 * equal scores to the lower block id; NaN counts as -inf.  Output ascending,
 * padded with -1.  scores is [nrows][max_blocks] as produced above, in the
 * same row order. */
static int better(double sa, int32_t ca, double sb, int32_t cb) {
  if (isnan(sa)) sa = -INFINITY;
  if (isnan(sb)) sb = -INFINITY;
  if (sa != sb) return sa > sb;
  return ca < cb;
}

int msa_oracle_select(const oracle_problem* p, const double* scores, const int32_t* ctx_lens,
                      const int32_t* rows, int32_t nrows, int32_t* selected,
                      int32_t* n_selected) {
  int T = p->query_len, K = p->topk, BS = p->block_size;
  for (int64_t n = 0; n < nrows; n++) {
    int32_t r = rows ? rows[n] : (int32_t)n;
    int32_t b = r / T, t = r % T;
    int64_t pos = row_position(ctx_lens[b], T, t);
    int32_t local = (int32_t)(pos / BS);
    const double* s = scores + n * (int64_t)p->max_blocks;
    int32_t* sel = selected + n * (int64_t)K;
    for (int k = 0; k < K; k++) sel[k] = -1;
    int cnt = 0;
    if (local + 1 <= K) {
      for (int32_t c = 0; c <= local; c++) sel[cnt++] = c;
    } else {
      /* repeated best-of-the-rest scan over the non-local candidates */
      char* taken = (char*)calloc((size_t)local, 1);
      for (int k = 0; k < K - 1; k++) {
        int32_t arg = -1;
        for (int32_t c = 0; c < local; c++) {
          if (taken[c]) continue;
          if (arg < 0 || better(s[c], c, s[arg], arg)) arg = c;
        }
        taken[arg] = 1;
      }
      for (int32_t c = 0; c < local; c++)
        if (taken[c]) sel[cnt++] = c; /* ascending by construction */
      sel[cnt++] = local;
      free(taken);
    }
    n_selected[n] = cnt;
  }
  return 0;
}

/* ---- step 3: block -> 16-token page table ------------------------------ */
/* [P3] section 3 and Figure 5: each selected logical block is resolved to
 * its physical block and expanded to 8 page ids of 16 tokens; the KV data is
 * never moved.  Reading: page id = physical block * 8 + j.  Row length is
 * topk * 8, padded with -1. */
int msa_oracle_page_table(const oracle_problem* p, const int32_t* selected,
                          const int32_t* block_table, const int32_t* rows, int32_t nrows,
                          int32_t* page_table) {
  int T = p->query_len, K = p->topk;
  int ppb = p->block_size / p->page_size;
  for (int64_t n = 0; n < nrows; n++) {
    int32_t r = rows ? rows[n] : (int32_t)n;
    int32_t b = r / T;
    int32_t* pt = page_table + n * (int64_t)K * ppb;
    for (int i = 0; i < K * ppb; i++) pt[i] = -1;
    for (int k = 0; k < K; k++) {
      int32_t c = selected[n * (int64_t)K + k];
      if (c < 0) break;
      int32_t phys = block_table[(int64_t)b * p->max_blocks + c];
      for (int j = 0; j < ppb; j++) pt[k * ppb + j] = phys * ppb + j;
    }
  }
  return 0;
}

/* ---- step 4: exact sparse GQA attention -------------------------------- */
/* [P1] "MSAの仕組み" (exact attention only inside the chosen blocks) and
 * [P2] "MSA 実行プロセス", step 3 (softmax attention over the selected KV
 * blocks only).  The key set of row r is every token i of a selected block
 * with i <= position of r.  For query head h on KV head g = h / (Hq/Hkv):
 *   z_i = scale * q_h . K_{i,g},  out_h = sum_i softmax(z)_i V_{i,g}.
 * Plain two-pass softmax with max subtraction, in double.  out is
 * [nrows][Hq][D]. */
int msa_oracle_attention(const oracle_problem* p, const uint16_t* q, const void* k_pool,
                         const void* v_pool, const void* k_scale, const void* v_scale,
                         const int32_t* block_table, const int32_t* ctx_lens,
                         const int32_t* selected, const int32_t* rows, int32_t nrows,
                         double* out) {
  int T = p->query_len, K = p->topk, BS = p->block_size, D = p->head_dim;
  int Hq = p->num_q_heads, Hkv = p->num_kv_heads;
  int group = Hq / Hkv;
  double scale = p->sm_scale > 0 ? p->sm_scale : 1.0 / sqrt((double)D);
  int64_t n;
#pragma omp parallel for schedule(dynamic, 1)
  for (n = 0; n < nrows; n++) {
    int32_t r = rows ? rows[n] : (int32_t)n;
    int32_t b = r / T, t = r % T;
    int64_t pos = row_position(ctx_lens[b], T, t);
    const int32_t* sel = selected + n * (int64_t)K;
    int64_t maxkeys = (int64_t)K * BS;
    double* z = (double*)malloc(sizeof(double) * (size_t)maxkeys);
    int64_t* kphys = (int64_t*)malloc(sizeof(int64_t) * (size_t)maxkeys);
    int* ktok = (int*)malloc(sizeof(int) * (size_t)maxkeys);
    /* the key set, in ascending position order */
    int64_t nk = 0;
    for (int k = 0; k < K; k++) {
      int32_t c = sel[k];
      if (c < 0) continue;
      int64_t phys = block_table[(int64_t)b * p->max_blocks + c];
      for (int tok = 0; tok < BS; tok++) {
        if ((int64_t)c * BS + tok > pos) break;
        kphys[nk] = phys;
        ktok[nk] = tok;
        nk++;
      }
    }
    for (int h = 0; h < Hq; h++) {
      int g = h / group;
      const uint16_t* qh = q + ((int64_t)r * Hq + h) * D;
      double zmax = -INFINITY;
      for (int64_t i = 0; i < nk; i++) {
        double dot = 0.0;
        for (int d = 0; d < D; d++)
          dot += msa_oracle_bf16_to_double(qh[d]) *
                 kv_value(p, k_pool, k_scale, kphys[i], g, ktok[i], d);
        z[i] = dot * scale;
        if (z[i] > zmax) zmax = z[i];
      }
      double denom = 0.0;
      for (int64_t i = 0; i < nk; i++) {
        z[i] = exp(z[i] - zmax);
        denom += z[i];
      }
      double* o = out + ((n * Hq) + h) * (int64_t)D;
      for (int d = 0; d < D; d++) o[d] = 0.0;
      for (int64_t i = 0; i < nk; i++) {
        double w = z[i] / denom;
        for (int d = 0; d < D; d++)
          o[d] += w * kv_value(p, v_pool, v_scale, kphys[i], g, ktok[i], d);
      }
    }
    free(z);
    free(kphys);
    free(ktok);
  }
  return 0;
}

/* ---- the write path: quantising new tokens into the pools ------------- */
/* The step before the hot path (news.ainew.jp MI355X article, section 3:
 * the fused projection writes the index cache; aisoku.org article, section
 * "何が新しいか": KV stored as fp8 or NVFP4).  The pages give no recipe, so
 * these follow the plainest reading, the one the synthetic inputs use:
 *  - fp8 K / V: per (token, head) scale = amax / 448 (1 when amax is 0),
 *    code = E4M3 round-to-nearest-even of x / scale clamped to +-448;
 *  - 4-bit K / V / index keys: per 16 elements s = E4M3 RNE of amax / 6,
 *    code = E2M1 RNE of x / s saturating at 6, all codes 0 when s is 0;
 *  - fp8 index keys: the E4M3 RNE code of the value itself (no scale).
 * Every step that decides a code runs in fp32 (IEEE single: division and
 * round-to-nearest-even), the precision the GPU kernel decides it in. */

/* fp32 -> OCP E4M3 code, round-to-nearest-even, magnitudes saturating at
 * 448; the sign is kept (negative values that round to 0 give 0x80). */
uint8_t msa_oracle_f32_to_e4m3(float x) {
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  float a = fabsf(x);
  if (isnan(a)) return (uint8_t)(sign | 0x7F);
  if (a >= 448.0f) return (uint8_t)(sign | 0x7E);
  if (a < 0.015625f) {                       /* below 2^-6: steps of 2^-9 */
    float m = nearbyintf(a * 512.0f);        /* 0..8; 8 is the first normal */
    return (uint8_t)(sign | (uint8_t)m);
  }
  int e2;
  float f = frexpf(a, &e2);                  /* a = f * 2^e2, f in [0.5, 1) */
  int e = e2 - 1;                            /* a = (2f) * 2^e, 2f in [1, 2) */
  float m = nearbyintf((2.0f * f - 1.0f) * 8.0f);  /* 3 mantissa bits */
  if (m == 8.0f) { m = 0.0f; e += 1; }
  int code = ((e + 7) << 3) | (int)m;
  if (code > 0x7E) code = 0x7E;
  return (uint8_t)(sign | code);
}

/* fp32 -> OCP E2M1 code: round-to-nearest-even onto {0, .5, 1, 1.5, 2, 3,
 * 4, 6}, saturating at 6; the sign bit only on a nonzero magnitude. */
uint8_t msa_oracle_f32_to_e2m1(float x) {
  float a = fabsf(x);
  int m;
  if (!(a < 6.0f)) m = 7;                               /* 6 (and NaN)      */
  else if (a < 2.0f) m = (int)nearbyintf(a * 2.0f);     /* 0 .. 2 by 0.5   */
  else if (a < 4.0f) m = 2 + (int)nearbyintf(a);        /* 2, 3, 4 -> 4..6 */
  else m = 4 + (int)nearbyintf(a * 0.5f);               /* 4, 6 -> 6, 7    */
  return (uint8_t)((x < 0.0f && m > 0) ? (m | 8) : m);
}

/* fp8 one row of n values: codes and the row's fp32 scale. */
static void quantize_fp8_row(const float* x, int n, uint8_t* codes, float* scale) {
  float amax = 0.0f;
  for (int i = 0; i < n; i++) amax = fmaxf(amax, fabsf(x[i]));
  float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  for (int i = 0; i < n; i++) {
    float y = x[i] / s;
    if (y > 448.0f) y = 448.0f;
    if (y < -448.0f) y = -448.0f;
    codes[i] = msa_oracle_f32_to_e4m3(y);
  }
  *scale = s;
}

/* 4-bit one row of n values (n a multiple of 16): packed codes (element 2j
 * in the low nibble of byte j) and one E4M3 scale code per 16 elements. */
static void quantize_fp4_row(const float* x, int n, uint8_t* packed, uint8_t* scales) {
  for (int g = 0; g < n / 16; g++) {
    const float* v = x + 16 * g;
    float amax = 0.0f;
    for (int i = 0; i < 16; i++) amax = fmaxf(amax, fabsf(v[i]));
    uint8_t sc = msa_oracle_f32_to_e4m3(amax / 6.0f);
    float s = (float)msa_oracle_e4m3_to_double(sc);
    scales[g] = sc;
    for (int i = 0; i < 16; i += 2) {
      uint8_t lo = s > 0.0f ? msa_oracle_f32_to_e2m1(v[i] / s) : 0;
      uint8_t hi = s > 0.0f ? msa_oracle_f32_to_e2m1(v[i + 1] / s) : 0;
      packed[(16 * g + i) / 2] = (uint8_t)(lo | (hi << 4));
    }
  }
}

/* Writes the T new tokens of every request: row r = b T + t is the token at
 * position p = ctx_lens[b] - T + t, stored at slot p mod 128 of physical
 * block block_table[b][p / 128].  k_new, v_new [R][Hkv][head_dim] and
 * idx_new [R][Hidx][idx_dim] are bf16 bit patterns; each row of each head is
 * quantised to the pool's format.  Pools as the attention reads them. */
int msa_oracle_insert(const oracle_problem* p, const uint16_t* k_new, const uint16_t* v_new,
                      const uint16_t* idx_new, const int32_t* block_table,
                      const int32_t* ctx_lens, void* k_pool, void* v_pool, void* k_scale,
                      void* v_scale, void* idx_k_pool, void* idx_k_scale) {
  int T = p->query_len, D = p->head_dim, E = p->idx_dim, BS = p->block_size;
  int R = p->batch * T;
  float buf[256];
  for (int r = 0; r < R; r++) {
    int b = r / T, t = r % T;
    int64_t pos = row_position(ctx_lens[b], T, t);
    int64_t phys = block_table[(int64_t)b * p->max_blocks + pos / BS];
    int64_t slot = pos % BS;
    for (int kv = 0; kv < 2; kv++) {
      const uint16_t* src = kv ? v_new : k_new;
      void* pool = kv ? v_pool : k_pool;
      void* scale = kv ? v_scale : k_scale;
      for (int g = 0; g < p->num_kv_heads; g++) {
        const uint16_t* x = src + ((int64_t)r * p->num_kv_heads + g) * D;
        int64_t row = (phys * p->num_kv_heads + g) * BS + slot;
        for (int i = 0; i < D; i++) buf[i] = (float)msa_oracle_bf16_to_double(x[i]);
        if (p->kv_dtype == ORACLE_BF16)
          memcpy((uint16_t*)pool + row * D, x, (size_t)D * 2);
        else if (p->kv_dtype == ORACLE_FP8)
          quantize_fp8_row(buf, D, (uint8_t*)pool + row * D, (float*)scale + row);
        else
          quantize_fp4_row(buf, D, (uint8_t*)pool + row * (D / 2),
                           (uint8_t*)scale + row * (D / 16));
      }
    }
    for (int h = 0; h < p->num_idx_heads; h++) {
      const uint16_t* x = idx_new + ((int64_t)r * p->num_idx_heads + h) * E;
      int64_t row = (phys * p->num_idx_heads + h) * BS + slot;
      for (int i = 0; i < E; i++) buf[i] = (float)msa_oracle_bf16_to_double(x[i]);
      if (p->idx_dtype == ORACLE_BF16)
        memcpy((uint16_t*)idx_k_pool + row * E, x, (size_t)E * 2);
      else if (p->idx_dtype == ORACLE_FP8)
        for (int i = 0; i < E; i++) {
          float y = buf[i] > 448.0f ? 448.0f : (buf[i] < -448.0f ? -448.0f : buf[i]);
          ((uint8_t*)idx_k_pool)[row * E + i] = msa_oracle_f32_to_e4m3(y);
        }
      else
        quantize_fp4_row(buf, E, (uint8_t*)idx_k_pool + row * (E / 2),
                         (uint8_t*)idx_k_scale + row * (E / 16));
    }
  }
  return 0;
}

/* Number of worker threads the parallel loops above use. */
int msa_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Sets the number of worker threads of the parallel loops above (the
 * benchmark's single-core baseline uses 1); n < 1 leaves it unchanged. */
void msa_oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
