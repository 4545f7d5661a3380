// Step 1 of MSA decode: block scoring by the index heads.
//
// agentlenshq page "MiniMax M3 vLLM サポート", section "MSA 実行プロセス",
// step 1: small index heads score every candidate 128-token KV block.  The
// block score is the maximum, over the block's tokens that are causal to the
// row, of the index dot product summed over index heads.  news.ainew.jp
// MI355X article, section 2: one indexer pass per request covers every draft
// position, so each key load is reused by all T rows.
//
// Design (gfx950): for a single row this is a matrix-vector stream, not a
// dense contraction, so it runs on the VALU.  One wave scores one logical
// block for all rows of its request: every load instruction moves 1 KB of
// contiguous keys (64 lanes x 16 B); bf16 keys feed v_dot2_f32_bf16 directly, fp8 keys are
// widened to bf16 pairs in registers first.  4-bit keys (E2M1 codes, one
// E4M3 scale per 16 dims, the NVFP4 layout of the aisoku.org article,
// section "何が新しいか") are widened to unscaled bf16 pairs, dotted with the
// query per group of 16 dims, and each group sum is multiplied by its
// scale.  With the synthetic keys (small integers, or E2M1 codes under
// power-of-two scales) every fp32 partial sum is exact in any order.  The
// lanes that share a token are folded by a transpose-reduce (each butterfly
// stage halves the partials a lane carries), then the wave takes the causal
// max.  Single rows with several index heads (bf16 or fp8 keys) instead
// give each block a workgroup of four waves, each a quarter of every head's
// tokens (index_scan_q4_kernel): the read pattern the memory system serves
// fastest for blocks scattered over the pool.  Requests with several rows
// (speculative verification) multiply the VALU work per byte; from a few
// rows on, the dot products move to the matrix cores with the rows as the
// M dimension (scan_block_mfma).
#include "msa_device.h"
#include "msa_internal.h"

#include <math.h>

namespace msa {
namespace {

constexpr int kBlock = 128;  // tokens per KV block
constexpr int kIdxDim = 64;  // index head dimension

// One butterfly stage of the transpose-reduce: lanes with `MASK` set keep
// the upper half of their partials, the others the lower half, and each adds
// its partner's copy of the half it keeps.  DPP: partner values by DPP lane
// moves, else by LDS-pipe shuffles.
template <int HALF, int MASK, bool DPP>
__device__ __forceinline__ void fold_stage(float* v, int lane) {
  const bool up = (lane & MASK) != 0;
#pragma unroll
  for (int j = 0; j < HALF; ++j) {
    const float send = up ? v[j] : v[j + HALF];
    const float keep = up ? v[j + HALF] : v[j];
    v[j] = keep + (DPP ? dpp_xor<MASK>(send) : __shfl_xor(send, MASK));
  }
}

// Wave-wide max by LDS-pipe shuffles (the DPP form is wave_max).
__device__ __forceinline__ float wave_max_shfl(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

// Key formats of the index cache.
enum KeyKind { kBf16 = 0, kFp8 = 1, kFp4 = 2 };

// Scores of logical block c (a real block: c * 128 < L, stored in physical
// block phys_block) for every row of request b, written by lane 0.  TR: rows
// scored per pass (1, 2 or 4); more rows loop.  idx_ks: the 4-bit keys'
// scale pool (unused otherwise).
template <int KIND, int TR>
__device__ __forceinline__ void scan_block(const uint16_t* __restrict__ idx_q,
                                           const uint8_t* __restrict__ idx_k,
                                           const uint8_t* __restrict__ idx_ks, int phys_block,
                                           float* __restrict__ scores, int b, int c, int L, int T,
                                           int Hidx, int MAXB, int lane) {
  constexpr int DPL = KIND == kBf16 ? 8 : (KIND == kFp8 ? 16 : 32);  // dims per lane per load
  // Cross-lane steps: DPP for bf16 and fp8 keys; the 4-bit scan, which does
  // more VALU work per byte, measured about 10% slower with them (the
  // compiler keeps fewer key loads in flight) and uses shuffles.
  constexpr bool kDpp = KIND != kFp4;
  constexpr int LPT = kIdxDim / DPL; // lanes per token (8 / 4 / 2)
  constexpr int TPL = kWave / LPT;   // tokens per load instruction (8 / 16 / 32)
  constexpr int NLD = kBlock / TPL;  // loads per (block, head) (16 / 8 / 4)
  constexpr int QW = DPL / 2;        // query dwords per lane per row (4 / 8 / 16)
  static_assert(NLD == 2 * LPT, "transpose-reduce leaves two tokens per lane");

  float* srow = scores + (size_t)b * T * MAXB + c;
  // bytes of one (block, head): LPT lane slices of 16 B per token
  const size_t head_bytes = (size_t)kBlock * LPT * 16;
  const size_t phys = (size_t)phys_block;
  const uint8_t* kblk = idx_k + phys * Hidx * head_bytes + lane * 16;
  // 4-bit scales [block][head][token][4]: this lane's two codes (its 32
  // dims) of token 32 i + lane / 2 sit at sblk + i * 128
  const uint8_t* sblk = nullptr;
  if constexpr (KIND == kFp4)
    sblk = idx_ks + phys * Hidx * (kBlock * 4) + (lane >> 1) * 4 + (lane & 1) * 2;
  const int dim0 = (lane % LPT) * DPL;

  // one index head's loads: keys (and 4-bit scales) of the block, queries
  struct Head {
    u32x4 kv[NLD];
    uint32_t ks[NLD];
    uint32_t qv[TR][QW];
  };
  auto load_head = [&](Head& hd, int h, int t0) {
    const uint8_t* kh = kblk + (size_t)h * head_bytes;
#pragma unroll
    for (int i = 0; i < NLD; ++i) hd.kv[i] = ldg128_stream(kh + i * 1024);
    if constexpr (KIND == kFp4) {
      const uint8_t* sh = sblk + (size_t)h * (kBlock * 4);
#pragma unroll
      for (int i = 0; i < NLD; ++i)
        hd.ks[i] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(sh + i * 128));
    }
#pragma unroll
    for (int t = 0; t < TR; ++t) {
      const int row = b * T + min(t0 + t, T - 1);
      const uint16_t* qp = idx_q + ((size_t)row * Hidx + h) * kIdxDim + dim0;
#pragma unroll
      for (int w = 0; w < QW; w += 4) {
        u32x4 v = ldg128(qp + 2 * w);
        hd.qv[t][w] = v.x; hd.qv[t][w + 1] = v.y; hd.qv[t][w + 2] = v.z; hd.qv[t][w + 3] = v.w;
      }
    }
  };
  auto score_head = [&](const Head& hd, float (&part)[TR][NLD]) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      uint32_t kw[QW];
      const uint32_t src[4] = {hd.kv[i].x, hd.kv[i].y, hd.kv[i].z, hd.kv[i].w};
      if constexpr (KIND == kBf16) {
#pragma unroll
        for (int w = 0; w < 4; ++w) kw[w] = src[w];
      } else if constexpr (KIND == kFp8) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          kw[2 * w] = e4m3x2_to_bf16x2<false>(src[w]);
          kw[2 * w + 1] = e4m3x2_to_bf16x2<true>(src[w]);
        }
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          kw[4 * w] = e2m1x2_to_bf16x2<0>(src[w]);
          kw[4 * w + 1] = e2m1x2_to_bf16x2<1>(src[w]);
          kw[4 * w + 2] = e2m1x2_to_bf16x2<2>(src[w]);
          kw[4 * w + 3] = e2m1x2_to_bf16x2<3>(src[w]);
        }
      }
      if constexpr (KIND == kFp4) {
        // dims 0..15 of the lane under scale 0, 16..31 under scale 1
        const f32x2 sc = e4m3x2_to_f32x2(hd.ks[i]);
#pragma unroll
        for (int t = 0; t < TR; ++t) {
          float g0 = 0.f, g1 = 0.f;
#pragma unroll
          for (int w = 0; w < QW / 2; ++w) g0 = dot2_bf16(kw[w], hd.qv[t][w], g0);
#pragma unroll
          for (int w = QW / 2; w < QW; ++w) g1 = dot2_bf16(kw[w], hd.qv[t][w], g1);
          part[t][i] = fmaf(sc.y, g1, fmaf(sc.x, g0, part[t][i]));
        }
      } else {
#pragma unroll
        for (int t = 0; t < TR; ++t) {
          float acc = part[t][i];
#pragma unroll
          for (int w = 0; w < QW; ++w) acc = dot2_bf16(kw[w], hd.qv[t][w], acc);
          part[t][i] = acc;
        }
      }
    }
  };

  for (int t0 = 0; t0 < T; t0 += TR) {
    float part[TR][NLD];
#pragma unroll
    for (int t = 0; t < TR; ++t)
#pragma unroll
      for (int i = 0; i < NLD; ++i) part[t][i] = 0.f;

    // (keeping the next head's loads in flight was measured no faster for
    // 4-bit keys: it costs the occupancy that the 4-bit scan relies on)
    for (int h = 0; h < Hidx; ++h) {
      Head hd;
      load_head(hd, h, t0);
      score_head(hd, part);
    }

#pragma unroll
    for (int t = 0; t < TR; ++t) {
      if (t0 + t >= T) break;
      float* v = part[t];
      if constexpr (LPT == 8) {
        fold_stage<8, 4, kDpp>(v, lane);
        fold_stage<4, 2, kDpp>(v, lane);
        fold_stage<2, 1, kDpp>(v, lane);
      } else if constexpr (LPT == 4) {
        fold_stage<4, 2, kDpp>(v, lane);
        fold_stage<2, 1, kDpp>(v, lane);
      } else {
        fold_stage<2, 1, kDpp>(v, lane);
      }
      // lane now holds the full scores of loads i = 2 * (lane % LPT) + e
      const int pos = L - T + t0 + t;
      float best = -INFINITY;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int tok = (2 * (lane % LPT) + e) * TPL + lane / LPT;
        if (c * kBlock + tok <= pos) best = fmaxf(best, v[e]);
      }
      best = kDpp ? wave_max(best) : wave_max_shfl(best);
      if (lane == 0) srow[(size_t)(t0 + t) * MAXB] = best;
    }
  }
}

// Max over the 16 lanes of each DPP row (lanes 16 r .. 16 r + 15), returned
// to all of them: quad swaps, then half-row and row mirrors.
__device__ __forceinline__ float row16_max(float v) {
  v = dpp_max_step<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_max_step<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_max_step<0x141, 0xF>(v);  // row_half_mirror
  return dpp_max_step<0x140, 0xF>(v);  // row_mirror
}

// The same scores on the matrix cores, for requests with several rows
// (speculative verification): per index head, S = Q K^T with the request's
// rows as the M dimension (T <= 16, zero rows beyond T) and the block's
// tokens as N, 16 tokens per tile, on v_mfma_f32_16x16x32_bf16.  Lane l
// supplies row / token l % 16 and the dims of k-group l / 16 (bf16 keys:
// dims 32 s + 8 g .. + 7 of step s; fp8 keys: one 16-byte load of dims
// 16 g .. 16 g + 15, split over the two steps and widened to bf16 exactly);
// it receives rows 4 g .. 4 g + 3 of token l % 16.  Summing over heads in
// the accumulators and taking the causal max per row over the tiles and the
// 16 lanes of a DPP row gives the block score.  Products of bf16 values are
// exact in fp32 and the synthetic sums stay below 2^24, so the scores equal
// the VALU path's bit for bit.
template <int KIND, bool ONE_HEAD>
__device__ __forceinline__ void scan_block_mfma(const uint16_t* __restrict__ idx_q,
                                                const uint8_t* __restrict__ idx_k,
                                                int phys_block, float* __restrict__ scores,
                                                int b, int c, int L, int T, int Hidx, int MAXB,
                                                int lane) {
  static_assert(KIND == kBf16 || KIND == kFp8, "matrix-core scan: bf16 or fp8 keys");
  constexpr int TB = KIND == kBf16 ? 128 : 64;  // bytes per token and head
  constexpr int NL = KIND == kBf16 ? 2 : 1;     // 16-byte loads per token and lane
  const int n = lane & 15, g = lane >> 4;
  const size_t head_bytes = (size_t)kBlock * TB;
  const uint8_t* kblk = idx_k + (size_t)phys_block * Hidx * head_bytes;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  float* srow = scores + (size_t)b * T * MAXB + c;
  const int tok0 = c * kBlock + n;

  // one head's key loads (tile i: token 16 i + n, this lane's dims) and
  // query operands (row n of the request, zeros past T)
  auto load_keys = [&](u32x4 (&kv)[8][NL], int h) {
    const uint8_t* kh = kblk + (size_t)h * head_bytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint8_t* kt = kh + (size_t)(16 * i + n) * TB;
      if constexpr (KIND == kBf16) {
        kv[i][0] = ldg128_stream(kt + 16 * g);
        kv[i][1] = ldg128_stream(kt + 64 + 16 * g);
      } else {
        kv[i][0] = ldg128_stream(kt + 16 * g);
      }
    }
  };
  auto load_query = [&](u32x4 (&qa)[2], int h) {
    qa[0] = zero;
    qa[1] = zero;
    if (n < T) {
      const uint16_t* qp = idx_q + ((size_t)(b * T + n) * Hidx + h) * kIdxDim;
      if constexpr (KIND == kBf16) {
        qa[0] = ldg128(qp + 8 * g);
        qa[1] = ldg128(qp + 32 + 8 * g);
      } else {
        qa[0] = ldg128(qp + 16 * g);
        qa[1] = ldg128(qp + 16 * g + 8);
      }
    }
  };
  // tile i of one head added to `a`
  auto tile = [&](f32x4 a, const u32x4 (&kv)[8][NL], const u32x4 (&qa)[2], int i) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      u32x4 kb;
      if constexpr (KIND == kBf16) {
        kb = kv[i][st];
      } else {
        const uint32_t lo = st ? kv[i][0].z : kv[i][0].x;
        const uint32_t hi = st ? kv[i][0].w : kv[i][0].y;
        kb.x = e4m3x2_to_bf16x2<false>(lo);
        kb.y = e4m3x2_to_bf16x2<true>(lo);
        kb.z = e4m3x2_to_bf16x2<false>(hi);
        kb.w = e4m3x2_to_bf16x2<true>(hi);
      }
      a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa[st]),
                                                  __builtin_bit_cast(bf16x8, kb), a, 0, 0, 0);
    }
    return a;
  };
  // rows 4 g + j: the max over this lane's causal tokens, then over the 16
  // lanes of the DPP row
  float best[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  auto fold = [&](const f32x4& a, int i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (tok0 + 16 * i <= L - T + 4 * g + j) best[j] = fmaxf(best[j], a[j]);
  };

  if constexpr (ONE_HEAD) {
    // one index head: each tile is final as soon as it is computed, so only
    // one accumulator is live (fewer registers, more waves in flight)
    u32x4 kv[8][NL], qa[2];
    load_keys(kv, 0);
    load_query(qa, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) fold(tile(f32x4{0.f, 0.f, 0.f, 0.f}, kv, qa, i), i);
  } else {
    // the head sum comes before the max: all 8 tiles stay live over heads
    f32x4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int h = 0; h < Hidx; ++h) {
      u32x4 kv[8][NL], qa[2];
      load_keys(kv, h);
      load_query(qa, h);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = tile(acc[i], kv, qa, i);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) fold(acc[i], i);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float m = row16_max(best[j]);
    if (n == 0 && 4 * g + j < T) srow[(size_t)(4 * g + j) * MAXB] = m;
  }
}

// msa_index_score: one wave per (request, logical block); blocks past the
// context score -inf for every row.  TR 0: the matrix-core path; TR -1:
// the matrix-core path for one index head.
//
// The single-row 4-bit scan holds only 4.5 KB per wave in flight (one
// head's codes and scales), so it needs many waves: built for 6 waves per
// SIMD (at most 80 registers; 76 used, no spills) it scanned the 128K layer
// with 4-bit keys in 88.6 us against 93.3 us at the 112 registers the
// compiler picks on its own (4 waves per SIMD); 5 waves per SIMD took 95.8
// and 7 spill.
constexpr int kFp4SingleRowWavesPerSimd = 6;

template <int KIND, int TR>
__global__ __launch_bounds__(256, KIND == kFp4 && TR == 1 ? kFp4SingleRowWavesPerSimd : 1)
void index_scan_kernel(
    const uint16_t* __restrict__ idx_q, const uint8_t* __restrict__ idx_k,
    const uint8_t* __restrict__ idx_ks, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ ctx_lens, float* __restrict__ scores, int B, int T, int Hidx,
    int MAXB, int max_block) {
  const int lane = lane_id();
  const int item = blockIdx.x * 4 + wave_id();
  if (item >= B * MAXB) return;
  const int b = item / MAXB;
  const int c = item - b * MAXB;
  // the table entry is in bounds for every c < MAXB: read it together with
  // the context length instead of after it
  int phys = block_table[(size_t)b * MAXB + c];
  const int L = ctx_lens[b];
  asm volatile("" : "+s"(phys));  // keeps the table load ahead of the branch
  phys = min(max(phys, 0), max_block);  // a bad table entry cannot leave the pool
  if (c * kBlock > L - 1) {
    float* srow = scores + (size_t)b * T * MAXB + c;
    for (int t = lane; t < T; t += kWave) srow[(size_t)t * MAXB] = -INFINITY;
    return;
  }
  if constexpr (TR == 0)
    scan_block_mfma<KIND, false>(idx_q, idx_k, phys, scores, b, c, L, T, Hidx, MAXB, lane);
  else if constexpr (TR < 0)
    scan_block_mfma<KIND, true>(idx_q, idx_k, phys, scores, b, c, L, T, Hidx, MAXB, lane);
  else
    scan_block<KIND, TR>(idx_q, idx_k, idx_ks, phys, scores, b, c, L, T, Hidx, MAXB, lane);
}

// Single rows with several index heads (bf16 or fp8 keys): one 4-wave
// workgroup per (request, logical block), wave q scoring tokens 32 q ..
// 32 q + 31 of every index head with all of its key loads in flight at
// once; the block's causal max goes through LDS.  The four waves stream one
// 64 KB block together, which the memory system serves faster than the
// waves of single-wave blocks spread over four blocks (see the launcher).
// `lds`: dynamic LDS of at least 4 floats (the launch sizes it to cap
// residency).
template <int KIND>
__global__ __launch_bounds__(256) void index_scan_q4_kernel(
    const uint16_t* __restrict__ idx_q, const uint8_t* __restrict__ idx_k,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ ctx_lens,
    float* __restrict__ scores, int B, int Hidx, int MAXB, int max_block) {
  static_assert(KIND != kFp4, "bf16 or fp8 keys");
  constexpr int DPL = KIND == kBf16 ? 8 : 16;  // dims per lane per load
  constexpr int LPT = kIdxDim / DPL;           // lanes per token (8 / 4)
  constexpr int TPL = kWave / LPT;             // tokens per load (8 / 16)
  constexpr int NLD = 32 / TPL;                // loads per head and wave (4 / 2)
  constexpr int QW = DPL / 2;                  // query dwords per lane (4 / 8)
  constexpr int kHeads = 4;                    // heads whose loads are in flight together
  extern __shared__ float wmax[];              // [4]
  const int lane = lane_id();
  const int q4 = wave_id();
  const int item = blockIdx.x;
  if (item >= B * MAXB) return;
  const int b = item / MAXB;
  const int c = item - b * MAXB;
  // the table entry is in bounds for every c < MAXB: read it together with
  // the context length
  int phys = block_table[(size_t)b * MAXB + c];
  const int L = ctx_lens[b];
  asm volatile("" : "+s"(phys));  // keeps the table load ahead of the branch
  phys = min(max(phys, 0), max_block);  // a bad table entry cannot leave the pool
  float* sp = scores + (size_t)b * MAXB + c;
  if (c * kBlock > L - 1) {  // uniform over the workgroup
    if (threadIdx.x == 0) *sp = -INFINITY;
    return;
  }
  const size_t head_bytes = (size_t)kBlock * LPT * 16;
  const uint8_t* kbase =
      idx_k + (size_t)phys * Hidx * head_bytes + (size_t)(32 * q4) * LPT * 16 + lane * 16;
  const int dim0 = (lane % LPT) * DPL;
  float part[NLD];  // partial dot products of token 32 q + TPL i + lane / LPT
#pragma unroll
  for (int i = 0; i < NLD; ++i) part[i] = 0.f;
  for (int h0 = 0; h0 < Hidx; h0 += kHeads) {
    u32x4 kv[kHeads][NLD];
    uint32_t qv[kHeads][QW];
#pragma unroll
    for (int hh = 0; hh < kHeads; ++hh) {
      if (h0 + hh >= Hidx) break;
      const uint8_t* kh = kbase + (size_t)(h0 + hh) * head_bytes;
#pragma unroll
      for (int i = 0; i < NLD; ++i) kv[hh][i] = ldg128_stream(kh + i * 1024);
      const uint16_t* qp = idx_q + ((size_t)b * Hidx + h0 + hh) * kIdxDim + dim0;
#pragma unroll
      for (int w = 0; w < QW; w += 4) {
        const u32x4 v = ldg128(qp + 2 * w);
        qv[hh][w] = v.x;
        qv[hh][w + 1] = v.y;
        qv[hh][w + 2] = v.z;
        qv[hh][w + 3] = v.w;
      }
    }
#pragma unroll
    for (int hh = 0; hh < kHeads; ++hh) {
      if (h0 + hh >= Hidx) break;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        uint32_t kw[QW];
        const uint32_t src[4] = {kv[hh][i].x, kv[hh][i].y, kv[hh][i].z, kv[hh][i].w};
        if constexpr (KIND == kBf16) {
#pragma unroll
          for (int w = 0; w < 4; ++w) kw[w] = src[w];
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            kw[2 * w] = e4m3x2_to_bf16x2<false>(src[w]);
            kw[2 * w + 1] = e4m3x2_to_bf16x2<true>(src[w]);
          }
        }
        float acc = part[i];
#pragma unroll
        for (int w = 0; w < QW; ++w) acc = dot2_bf16(kw[w], qv[hh][w], acc);
        part[i] = acc;
      }
    }
  }
  // sum over the LPT lanes of each token (DPP), then the causal max
  float best = -INFINITY;
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    float v = part[i];
    v += dpp_xor<1>(v);
    v += dpp_xor<2>(v);
    if constexpr (LPT == 8) v += dpp_xor<4>(v);
    const int tok = 32 * q4 + TPL * i + lane / LPT;
    if (c * kBlock + tok <= L - 1) best = fmaxf(best, v);
  }
  best = wave_max(best);
  if (lane == 0) wmax[q4] = best;
  __syncthreads();
  if (threadIdx.x == 0) *sp = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
}

// Workgroups per CU that a scan launch lets run at once.  The kernel uses
// no LDS, so a dynamic LDS request of a share of the CU's 160 KiB caps
// residency.  Measured on MI355X: with bf16 or fp8 keys the stream runs
// faster with fewer waves in flight than the register limit allows -- 3
// workgroups per CU on grids of 8192 workgroups or more (1.5-3% on the 128K
// and 1M-context layers), 4 on smaller grids, where 3 leaves a short last
// round; 4-bit keys spend more ALU work per byte and run best uncapped.
constexpr size_t kLdsPerCu = 160 * 1024;

size_t scan_lds_bytes(int kind, unsigned workgroups) {
  if (kind == kFp4) return 0;
  return kLdsPerCu / (workgroups >= 8192 ? 3 : 4);
}

// Requests with at least this many rows score on the matrix cores.
// Measured on MI355X (scan of a 128-request fp8 layer, 8-16K contexts):
// fp8 keys 17.5 vs 26.5 us at 3 rows, 17.8 vs 27.4 at 4, on par at 2; bf16
// keys (32 requests, 32K) lose at 2 and 4 rows (26.0 vs 21.5, 26.4 vs 24.6:
// a 128-byte key row spans two of the operand's load instructions) and win
// from 8 (26.8 vs 42.2), where the row passes of the VALU path multiply.
// The matrix-core launches run best uncapped (fp8, 4 rows: 17.8 us, 27.6
// with 3 workgroups per CU).
constexpr int kMfmaMinRowsBf16 = 5;
constexpr int kMfmaMinRowsFp8 = 2;

// Single rows with at least this many index heads (bf16 / fp8 keys) score
// each block with four waves (index_scan_q4_kernel), 4 workgroups per CU.
// Measured on MI355X, same box, against one wave per block: the 128K layer
// (4 bf16 heads) scan 325.8 vs 326.8 us; the 1M context (4 fp8 heads)
// 153.4-153.7 vs 157.0-157.1 us.  Small blocks lose: on 32 ragged 128K
// requests, 2 bf16 heads 80.4 vs 79.0 us, 2 / 3 fp8 heads 52.1 / 68.5 vs
// 43.0 / 61.6 us (each wave's share is too small for its fixed cost), while
// 3 bf16 heads gain (115.7 vs 116.9).  With 4 fp8 heads the four waves win
// on full contexts (153.8 vs 157.5 us) and lose on ragged ones (172.2 vs
// 166.0: the blocks past a context then cost a workgroup each); the
// launcher cannot see the context lengths and keeps the four waves, as
// the long-context workloads want.  Residency: 5 or 6 workgroups per CU
// measured the same as 4, 3 slower (335 and 189 us).
constexpr int kQuarterMinHeadsBf16 = 3;
constexpr int kQuarterMinHeadsFp8 = 4;
constexpr int kQuarterWgsPerCu = 4;

template <int KIND>
hipError_t launch_kind(const Dims& d, const void* idx_q, const void* idx_k, const void* idx_ks,
                       const int32_t* bt, const int32_t* cl, float* scores, hipStream_t s,
                       std::string* note) {
  const long items = (long)d.B * d.MAXB;
  const dim3 grid((unsigned)((items + 3) / 4)), block(256);
  const auto* q = static_cast<const uint16_t*>(idx_q);
  const auto* k = static_cast<const uint8_t*>(idx_k);
  const auto* ks = static_cast<const uint8_t*>(idx_ks);
  const bool mfma = (KIND == kBf16 && d.T >= kMfmaMinRowsBf16) ||
                    (KIND == kFp8 && d.T >= kMfmaMinRowsFp8);
  const int tr = mfma ? (d.Hidx == 1 ? -1 : 0) : (d.T == 1 ? 1 : (d.T == 2 ? 2 : 4));
  const size_t lds = mfma ? 0 : scan_lds_bytes(KIND, grid.x);
  if constexpr (KIND != kFp4) {
    if (tr == 0)
      hipLaunchKernelGGL((index_scan_kernel<KIND, 0>), grid, block, lds, s, q, k, ks, bt, cl,
                         scores, d.B, d.T, d.Hidx, d.MAXB, d.NB - 1);
    else if (tr == -1)
      hipLaunchKernelGGL((index_scan_kernel<KIND, -1>), grid, block, lds, s, q, k, ks, bt, cl,
                         scores, d.B, d.T, d.Hidx, d.MAXB, d.NB - 1);
  }
  if constexpr (KIND != kFp4) {
    if (tr == 1 && d.Hidx >= (KIND == kBf16 ? kQuarterMinHeadsBf16 : kQuarterMinHeadsFp8)) {
      const long wgs = (long)d.B * d.MAXB;
      const size_t lds4 = kLdsPerCu / kQuarterWgsPerCu;
      hipLaunchKernelGGL((index_scan_q4_kernel<KIND>), dim3((unsigned)wgs), block, lds4, s, q, k,
                         bt, cl, scores, d.B, d.Hidx, d.MAXB, d.NB - 1);
      static const char* qnames[2] = {"bf16", "fp8"};
      if (note)
        *note += std::string("index_scan<") + qnames[KIND] + ",quarters>[grid=" +
                 std::to_string(wgs) + "x256,lds=" + std::to_string(lds4) + "]";
      return hipGetLastError();
    }
  }
  if (tr == 1)
    hipLaunchKernelGGL((index_scan_kernel<KIND, 1>), grid, block, lds, s, q, k, ks, bt, cl, scores,
                       d.B, d.T, d.Hidx, d.MAXB, d.NB - 1);
  else if (tr == 2)
    hipLaunchKernelGGL((index_scan_kernel<KIND, 2>), grid, block, lds, s, q, k, ks, bt, cl, scores,
                       d.B, d.T, d.Hidx, d.MAXB, d.NB - 1);
  else if (tr == 4)
    hipLaunchKernelGGL((index_scan_kernel<KIND, 4>), grid, block, lds, s, q, k, ks, bt, cl, scores,
                       d.B, d.T, d.Hidx, d.MAXB, d.NB - 1);
  static const char* names[3] = {"bf16", "fp8", "nvfp4"};
  if (note)
    *note += std::string("index_scan<") + names[KIND] +
             (tr <= 0 ? std::string(tr ? ",mfma1" : ",mfma") : ",rows" + std::to_string(tr)) +
             ">[grid=" + std::to_string(grid.x) + "x256,lds=" + std::to_string(lds) + "]";
  return hipGetLastError();
}

}  // namespace

hipError_t launch_index_scan(const Dims& d, const void* idx_q, const void* idx_k,
                             const void* idx_k_scale, const int32_t* block_table,
                             const int32_t* ctx_lens, float* scores, hipStream_t s,
                             std::string* note) {
  if (d.idx_dtype == kBf16)
    return launch_kind<kBf16>(d, idx_q, idx_k, nullptr, block_table, ctx_lens, scores, s, note);
  if (d.idx_dtype == kFp8)
    return launch_kind<kFp8>(d, idx_q, idx_k, nullptr, block_table, ctx_lens, scores, s, note);
  return launch_kind<kFp4>(d, idx_q, idx_k, idx_k_scale, block_table, ctx_lens, scores, s, note);
}

}  // namespace msa
