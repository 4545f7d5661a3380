// Step 4 of MSA decode: exact split-K sparse GQA attention over the page
// table, and the log-sum-exp merge of the splits.
//
// aisoku.org MiniMax-M3.1-Flash article, section "MSAの仕組み": exact
// attention runs only inside the chosen blocks.  agentlenshq page, section
// "MSA 実行プロセス" step 3: online-softmax attention over the selected KV
// blocks only; section "EAGLE3 を用いた投機的デコード": a decode split-K path
// that takes a unified decode_query_len.  news.ainew.jp MI355X article,
// section 3 and Figure 5: the kernel consumes 16-token pages through a view
// of the KV allocation, never a copy.
//
// Design (gfx950):
//  * A workgroup of 4 or 8 waves owns one (row, KV head, split).  Each wave
//    walks chunks of 32 keys (two 16-token pages) of the row's blocks; when
//    a workgroup holds the whole row it writes the output itself.
//  * Multi-row requests (speculative verification, up to 4 rows) instead
//    give one workgroup the union of the request's rows' blocks, with every
//    (row, query head) pair as an MFMA column, so a block the rows share is
//    read once; fp8 chunks are prefetched into two LDS slots per wave (raw
//    bytes; V^T read from them by transposing 8-bit reads).  Rows of
//    longer requests keep the per-row workgroups, on one XCD per request so
//    that blocks they share can be served from its L2.
//  * QK^T on MFMA v_mfma_f32_16x16x32_bf16 with keys as the M dimension and
//    the query heads of the KV head as N (one tile of 16): S^T = K Q^T; keys
//    past the row's position are masked.  K rows go straight from HBM into
//    the A operand (each lane 64 contiguous bytes of
//    one key row); the result leaves every lane with 4 keys of one head, so
//    the softmax statistics of a head never cross lane groups but four.
//  * P V on the same MFMA as O^T = V^T P^T.  P^T is exactly the S^T
//    accumulator layout (no shuffle); V^T needs a transpose, so the V pages
//    are staged through LDS and read back column-wise: fp8 / 4-bit V (widened
//    in registers) with gfx950's transposing LDS read (ds_read_b64_tr_b16,
//    two per 8 keys x 16 dims operand), bf16 V (loaded straight into LDS)
//    with 16-bit reads, which measured faster there.  The 16-byte slots of a
//    row are XOR-swizzled so that each read spreads over the banks.  bf16 V goes from HBM to LDS with direct global-to-LDS loads
//    and occupies no registers.  P is split into bf16 hi + lo halves (two
//    MFMAs) so the weights keep ~16 bits.
//  * fp8 K/V: e4m3 -> bf16 is exact; the per-token K scale multiplies the
//    logit, the V scale multiplies P.  4-bit K/V: e2m1 x e4m3 -> bf16 is
//    exact (at most 6 significant bits) and happens in registers.
//  * Inside msa_decode, single-row requests and multi-row requests that
//    walk their union select in this launch: every workgroup of a row (of a
//    request) runs the selection (select_device.h) on the block scores first
//    and keeps the page ids in LDS, which saves the selection launch on the
//    dependent chain.
//  * Split partials (m, l, unnormalised O) combine inside the workgroup in
//    LDS; when a row is split over several workgroups a small merge kernel
//    applies the log-sum-exp rule.  (Merging in the last workgroup to finish
//    was measured slower on MI355X: the cross-workgroup hand-off stalls every
//    workgroup on a write-through store and a returning atomic.)
#include "msa_device.h"
#include "msa_internal.h"
#include "select_device.h"

#include <math.h>

namespace msa {
namespace {

constexpr int kD = 128;          // head dim
constexpr int kVRow = 256;       // LDS bytes per staged V row (bf16)
constexpr int kChunk = 32;       // keys per chunk (two pages)
constexpr int kStage = kChunk * kVRow;  // LDS bytes of one wave's staged V
// LDS bytes per wave: the V stage, reused after the chunk loop as the merge
// area (m and l of 16 columns, 16 output rows of kORow floats).  Rows are
// 16-byte aligned so that each lane moves 4 dims per LDS access; the 4
// floats of padding spread a wave's writes over all banks.
constexpr int kORow = 132;       // floats per head row in the merge area
constexpr int kWaveLds = 8576;
static_assert(kWaveLds >= kStage && kWaveLds >= 4 * (32 + 16 * kORow), "LDS per wave");
// s_waitcnt operand (gfx9 encoding) that waits for vmcnt == 0 only.
constexpr int kWaitVmem = 0x0F70;
// Cache-policy operand of a direct-to-LDS load: non-temporal.
constexpr int kNonTemporal = 2;

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef int lds_v2i32_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) lds_v2i32_t lds_v2i32;

__device__ __forceinline__ float neg_inf() { return -INFINITY; }

// Key row index kappa(g4, jj) within a chunk of the k-slot jj of lane group
// g4 = lane / 16: the order of the S^T accumulator rows.
__device__ __forceinline__ int kappa(int g4, int jj) {
  return jj < 4 ? 4 * g4 + jj : 16 + 4 * g4 + (jj - 4);
}

// Staged V rows are 256 bytes of 16 slots of 8 dims.  Slot s of row k sits
// at physical slot s ^ vswz(k).  bf16 V (16-bit column reads): the 4 row
// groups one V^T read touches (rows 4 g4 + c, see kappa) land on distinct
// banks with 2 ((k / 4) mod 4).  fp8 / 4-bit V (transposing reads): one read
// takes 32 bytes (one 16-dim block) from each of rows 0..15 (or 16..31) of
// the chunk, and 2 (k mod 8) sends them to every 32-byte bank group exactly
// twice.
template <int KV>
__device__ __forceinline__ int vswz(int k) {
  return KV == 0 ? 2 * ((k >> 2) & 3) : 2 * (k & 7);
}
template <int KV>
__device__ __forceinline__ int voff(int k, int slot) {
  return k * kVRow + 16 * (slot ^ vswz<KV>(k));
}

template <int KV>
struct Chunk {
  // raw loads of one page: K part for this lane's key row / V part
  u32x4 k[KV == 0 ? 4 : (KV == 1 ? 2 : 1)];
  u32x4 v[KV == 1 ? 2 : 1];  // bf16 V goes straight to LDS
  uint32_t ks, vs;  // nvfp4: the two e4m3 scale codes of this lane's 32 dims
  f32x4 kscale, vscale;  // fp8: per-token scales of this lane's 4 S^T rows
};

// First head dim of the 8-dim slice that lane group g (= lane / 16) feeds
// into K-step kk of the QK^T MFMA.  The contraction order is free as long as
// K and Q agree; each dtype picks the order that makes its K loads cover
// contiguous runs of a key row.
template <int KV>
__device__ __forceinline__ int kdim(int g, int kk) {
  if constexpr (KV == 0) return 32 * kk + 8 * g;                         // 64 B per row per load
  else if constexpr (KV == 1) return 64 * (kk >> 1) + 16 * g + 8 * (kk & 1);  // 64 B per row
  else return 32 * g + 8 * kk;                                            // whole 64 B row
}

// Every KV load carries the non-temporal hint, also where the draft rows of
// a request share pages.  Measured on MI355X (fp8 spec-verify layer, 128
// requests x 4 rows): after a 1 GiB cache flush, the state of a layer's KV
// in a decode step over many layers, a step takes 91.5 us with the hint
// against 116.5 us with cached loads; only when the same layer repeats back
// to back, its ~220 MB of KV then staying in the 256 MB last-level cache,
// do cached loads win (64 vs 75 us).
__device__ __forceinline__ u32x4 ld16(const uint8_t* p) { return ldg128_stream(p); }

// Register loads of one 16-token page.  K: lane (key m = lane % 16, group
// g) holds the slices kdim(g, .) of key m.  fp8 / 4-bit V: each load
// instruction covers a contiguous run (1 KB for fp8, the whole page for
// 4-bit), widened to bf16 by stage_v.  bf16 V takes load_v_lds instead.
template <int KV>
__device__ __forceinline__ void load_page(Chunk<KV>& c, const uint8_t* __restrict__ k_pool,
                                          const uint8_t* __restrict__ v_pool,
                                          const void* __restrict__ k_scale,
                                          const void* __restrict__ v_scale, size_t row0,
                                          int lane) {
  const int m = lane & 15, g = lane >> 4;
  if constexpr (KV == 0) {
    const uint8_t* kp = k_pool + (row0 + m) * 256 + 16 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) c.k[i] = ld16(kp + 64 * i);
  } else if constexpr (KV == 1) {
    const uint8_t* kp = k_pool + (row0 + m) * 128 + 16 * g;
    const uint8_t* vp = v_pool + row0 * 128 + 16 * lane;
    c.k[0] = ld16(kp);
    c.k[1] = ld16(kp + 64);
    c.v[0] = ld16(vp);
    c.v[1] = ld16(vp + 1024);
    c.kscale = *reinterpret_cast<const f32x4*>(static_cast<const float*>(k_scale) + row0 + 4 * g);
    c.vscale = *reinterpret_cast<const f32x4*>(static_cast<const float*>(v_scale) + row0 + 4 * g);
  } else {
    c.k[0] = ld16(k_pool + (row0 + m) * 64 + 16 * g);
    c.v[0] = ld16(v_pool + row0 * 64 + 16 * lane);
    c.ks = *reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(k_scale) +
                                              (row0 + m) * 8 + 2 * g);
    c.vs = *reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(v_scale) +
                                              (row0 + (lane >> 2)) * 8 + 2 * (lane & 3));
  }
}

// bf16 V of one page straight from HBM into its LDS rows, no registers
// involved.  Load i fills rows 4i..4i+3 (1 KB, 16 bytes per lane at LDS
// offset 16 lane); a lane fetches the global slot that the swizzle puts
// there.  The compiler issues these after the chunk's S^T MFMAs, i.e. once
// K has arrived; issuing them ahead of the MFMAs (K and V in flight
// together) measured slower on MI355X.
__device__ __forceinline__ void load_v_lds(const uint8_t* __restrict__ v_pool, size_t row0,
                                           int lane, uint8_t* page_rows) {
  const uint8_t* vp = v_pool + (row0 + (lane >> 4)) * 256;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_global_load_lds(vp + 1024 * i + 16 * ((lane & 15) ^ vswz<0>(4 * i)),
                                     (lds_void*)(page_rows + 1024 * i), 16, 0,
                                     kNonTemporal);
}

// Four packed bf16 pairs from 8 e2m1 codes (one dword) with scale `s`.
__device__ __forceinline__ void e2m1x8_to_bf16(uint32_t w, float s, uint32_t* out) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const f32x2 v = e2m1x2_to_f32x2(w, b);
    out[b] = pack_bf16_trunc(v.x * s, v.y * s);
  }
}

// A operand (16 keys x 8 dims, dims kdim(g, kk)) of K-step kk, as bf16.
template <int KV>
__device__ __forceinline__ bf16x8 k_operand(const Chunk<KV>& c, int kk) {
  if constexpr (KV == 0) {
    return __builtin_bit_cast(bf16x8, c.k[kk]);
  } else if constexpr (KV == 1) {
    const u32x4 src = c.k[kk >> 1];
    const uint32_t lo = (kk & 1) ? src.z : src.x;
    const uint32_t hi = (kk & 1) ? src.w : src.y;
    u32x4 o;
    o.x = e4m3x2_to_bf16x2<false>(lo);
    o.y = e4m3x2_to_bf16x2<true>(lo);
    o.z = e4m3x2_to_bf16x2<false>(hi);
    o.w = e4m3x2_to_bf16x2<true>(hi);
    return __builtin_bit_cast(bf16x8, o);
  } else {
    const u32x4 src = c.k[0];
    const uint32_t w = kk == 0 ? src.x : kk == 1 ? src.y : kk == 2 ? src.z : src.w;
    const float s = e4m3_to_f32((c.ks >> (8 * (kk >> 1))) & 0xFFu);
    uint32_t o[4];
    e2m1x8_to_bf16(w, s, o);
    u32x4 r = {o[0], o[1], o[2], o[3]};
    return __builtin_bit_cast(bf16x8, r);
  }
}

__device__ __forceinline__ void lds_write16(uint8_t* dst, uint32_t a, uint32_t b, uint32_t c,
                                            uint32_t d) {
  *reinterpret_cast<uint2*>(dst) = make_uint2(a, b);
  *reinterpret_cast<uint2*>(dst + 8) = make_uint2(c, d);
}

// Write this lane's share of one V page into the page's 16 LDS rows (bf16,
// kVRow bytes apart), converting fp8 / e2m1 to bf16 on the way.
template <int KV>
__device__ __forceinline__ void stage_v(const Chunk<KV>& c, uint8_t* page_rows, int lane) {
  if constexpr (KV == 1) {
    // load i: key 8i + lane/8, dims 16*(lane%8)..+16
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t src[4] = {c.v[i].x, c.v[i].y, c.v[i].z, c.v[i].w};
      uint32_t o[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        o[2 * w] = e4m3x2_to_bf16x2<false>(src[w]);
        o[2 * w + 1] = e4m3x2_to_bf16x2<true>(src[w]);
      }
      // Slots 2 (lane % 8) and the next stay adjacent under the swizzle.
      // Which of the two a lane writes first alternates with bit 2 of the
      // lane and with the row, so that any 8 consecutive lanes write 8
      // distinct 16-byte slots modulo 128 bytes and any 16 lanes (two
      // rows) 16 distinct slots modulo 256 bytes: no bank conflicts on the
      // 128-bit LDS writes whichever lane grouping serves them.
      const int k = 8 * i + (lane >> 3);
      const bool odd = ((lane >> 2) ^ k) & 1;
      uint8_t* dst = page_rows + voff<KV>(k, 2 * (lane & 7));
      lds_write16(dst + (odd ? 16 : 0), odd ? o[4] : o[0], odd ? o[5] : o[1],
                  odd ? o[6] : o[2], odd ? o[7] : o[3]);
      lds_write16(dst + (odd ? 0 : 16), odd ? o[0] : o[4], odd ? o[1] : o[5],
                  odd ? o[2] : o[6], odd ? o[3] : o[7]);
    }
  } else if constexpr (KV == 2) {
    // key lane/4, dims 32*(lane%4)..+32
    const uint32_t src[4] = {c.v[0].x, c.v[0].y, c.v[0].z, c.v[0].w};
    const float s0 = e4m3_to_f32(c.vs & 0xFFu);
    const float s1 = e4m3_to_f32((c.vs >> 8) & 0xFFu);
    // Write w of a lane stores a rotated piece pc, so that any 8
    // consecutive lanes (two rows) write 8 distinct 16-byte slots modulo
    // 128 bytes and any 16 lanes (four rows) 16 distinct slots modulo 256
    // bytes under the swizzle: no bank conflicts on the 128-bit LDS writes.
    const int k = lane >> 2;
    const int rot = ((lane & 3) >> 1) + (lane & 1);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int pc = (w + rot) & 3;
      const uint32_t word = pc == 0 ? src[0] : (pc == 1 ? src[1] : (pc == 2 ? src[2] : src[3]));
      uint32_t o[4];
      e2m1x8_to_bf16(word, pc < 2 ? s0 : s1, o);
      lds_write16(page_rows + voff<KV>(k, 4 * (lane & 3) + pc), o[0], o[1], o[2], o[3]);
    }
  }
}

// Dims d .. d + 3 of (row, query head) rh: the normalised output when the
// row is not split, else this split's partial O and, once per row, (m, l).
__device__ __forceinline__ void store_result(const f32x4& O, float M, float Ls, size_t rh, int d,
                                             int S, int split, float* __restrict__ out,
                                             float* __restrict__ part_o,
                                             float* __restrict__ part_ml) {
  if (S == 1) {
    f32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = Ls > 0.f ? O[i] / Ls : 0.f;
    *reinterpret_cast<f32x4*>(out + rh * kD + d) = v;
  } else {
    *reinterpret_cast<f32x4*>(part_o + (rh * S + split) * kD + d) = O;
    if (d == 0) {
      part_ml[(rh * S + split) * 2] = M;
      part_ml[(rh * S + split) * 2 + 1] = Ls;
    }
  }
}

// Combines the W waves' softmax states of one 16-column tile through LDS
// (`area`, W * kWaveLds bytes, free on entry).  Per lane: m and l of column
// hl, and dims 16 s + 4 g4 .. + 3 of the column's O in oacc[s].  Column c's
// result is sum_w 2^(m_w - M) O_w and sum_w 2^(m_w - M) l_w with M the
// largest m_w, summed in wave order; emit(c, d, O, M, L) receives 4
// consecutive dims d .. d + 3 of each column c < ncols.  Contains workgroup
// barriers.
template <int W, typename Emit>
__device__ __forceinline__ void combine_tile(uint8_t* area, float m, float l,
                                             const f32x4 (&oacc)[8], int ncols, Emit emit) {
  const int lane = lane_id();
  const int wave = wave_id();
  const int hl = lane & 15;
  const int g4 = lane >> 4;
  float* m_w = reinterpret_cast<float*>(area);  // [W][16]
  float* l_w = m_w + 16 * W;                    // [W][16]
  float* o_w = l_w + 16 * W;                    // [W][16][kORow]
  __syncthreads();
  if (lane < 16) {
    m_w[wave * 16 + lane] = m;
    l_w[wave * 16 + lane] = l;
  }
#pragma unroll
  for (int s = 0; s < 8; ++s)
    *reinterpret_cast<f32x4*>(o_w + (wave * 16 + hl) * kORow + 16 * s + 4 * g4) = oacc[s];
  __syncthreads();
  for (int gi = threadIdx.x; gi < 16 * (kD / 4); gi += 64 * W) {
    const int c = gi / (kD / 4);
    const int d = 4 * (gi % (kD / 4));
    if (c >= ncols) break;  // gi rises with c
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, m_w[w * 16 + c]);
    f32x4 O = {0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mw = m_w[w * 16 + c];
      const float f = mw == neg_inf() ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      const f32x4 o = *reinterpret_cast<const f32x4*>(o_w + (w * 16 + c) * kORow + d);
#pragma unroll
      for (int i = 0; i < 4; ++i) O[i] += f * o[i];
      L += f * l_w[w * 16 + c];
    }
    emit(c, d, O, M, L);
  }
}

// One workgroup owns (row r = b T + t, KV head g, split): the G query heads
// of KV head g are the MFMA columns (zero past G), the row's page table
// lists its blocks, local block last.  Every wave walks chunks of 32 keys
// (two 16-token pages) of the row's blocks, S apart between the splits and
// S W apart between the waves of a split.  SEL (single-row requests, 8
// waves): the workgroup first selects its row's blocks from the block scores
// (the selection kernel's code, page ids into LDS) instead of reading a page
// table; its registers then allow two waves per SIMD, which is all that one
// workgroup per CU needs.
template <int KV, int W, bool SEL>
__global__ __launch_bounds__(64 * W, SEL ? 2 : 4) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ k_pool,
    const uint8_t* __restrict__ v_pool, const void* __restrict__ k_scale,
    const void* __restrict__ v_scale, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ ctx_lens, float* __restrict__ part_o,
    float* __restrict__ part_ml, float* __restrict__ out, int B, int T, int Hq, int Hkv, int PT,
    int S, int max_block, float scale_log2, SelectArgs sa, int MAXB) {
  static_assert(!SEL || W == 8, "the fused selection runs on 8 waves");
  __shared__ __attribute__((aligned(16))) uint8_t smem[W * kWaveLds];

  const int lane = lane_id();
  const int wave = wave_id();
  // Workgroup ids go round-robin over the 8 XCDs.  With several draft rows
  // per request (T > 1), which select mostly the same blocks, ids are
  // permuted so that all of request b's workgroups run on XCD b % 8 and
  // meet in its L2; otherwise ids are request-major.
  const int per = T * Hkv * S;
  int b, x;
  if (T > 1) {
    b = (blockIdx.x / (8 * per)) * 8 + (blockIdx.x & 7);
    x = (blockIdx.x >> 3) % per;
  } else {
    b = blockIdx.x / per;
    x = blockIdx.x % per;
  }
  if (b >= B) return;
  const int split = x % S;
  x /= S;
  const int g = x % Hkv;
  const int t = x / Hkv;
  const int r = b * T + t;
  const int G = Hq / Hkv;

  // Q^T operand: column hl is query head g G + hl of row r (zero past G);
  // lane group g4 holds the dims kdim(g4, kk) of K-step kk
  const int hl = lane & 15;
  const int g4 = lane >> 4;
  bf16x8 qop[4];
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const uint16_t* qp = q + ((size_t)r * Hq + g * G + min(hl, G - 1)) * kD;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u32x4 v = ldg128(qp + kdim<KV>(g4, kk));
      qop[kk] = __builtin_bit_cast(bf16x8, hl < G ? v : z);
    }
  }

  // the row's page table stays in registers: slot k's first page in lane 8k
  int pt_lo, pt_hi;
  if constexpr (SEL) {
    // every workgroup of the row selects (T = 1); one of them exports
    __shared__ SelectLds<8> ssh;
    __shared__ int32_t prow_lds[kMaxTopk * 8];
    const bool exporter = g == 0 && split == 0;
    select_request<8>(b, sa.scores, ctx_lens, sa.block_table, exporter ? sa.selected : nullptr,
                      exporter ? sa.n_selected : nullptr, exporter ? sa.page_table : nullptr, 1,
                      MAXB, PT / 8, ssh, prow_lds);
    pt_lo = lane < PT ? prow_lds[lane] : -1;
    pt_hi = lane + kWave < PT ? prow_lds[lane + kWave] : -1;
  } else {
    const int32_t* prow = page_table + (size_t)r * PT;
    pt_lo = lane < PT ? prow[lane] : -1;
    pt_hi = lane + kWave < PT ? prow[lane + kWave] : -1;
  }
  const int nblk = (__popcll(__ballot(pt_lo >= 0)) + __popcll(__ballot(pt_hi >= 0))) >> 3;
  // keys of the local block that are causal to the row (position L - T + t)
  const int vloc = ((ctx_lens[b] - T + t) & 127) + 1;

  float m = neg_inf(), lsum = 0.f;
  f32x4 oacc[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) oacc[s] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint8_t* stage = smem + wave * kWaveLds;
  const int nchunks = 4 * nblk;  // 4 chunks of 32 keys per block
  // Chunks past the row's position (the tail of its local block, which
  // comes last) are never visited: the loop stops at `limit` instead of
  // skipping them, which measured faster (128K layer 43.6 vs 45.8 us).
  const int limit = min(nchunks, 4 * (nblk - 1) + (vloc + 31) / 32);
  // the registers of chunk ci (two pages); returns its first key row
  auto load_chunk = [&](Chunk<KV> (&ch)[2], int ci) {
    const int u = ci >> 2;         // block slot in the row's table
    const int pg0 = (ci & 3) * 2;  // first page of the chunk inside the block
    const int idx = 8 * u;         // wave-uniform
    const int P = idx < kWave ? __builtin_amdgcn_readlane(pt_lo, idx)
                              : __builtin_amdgcn_readlane(pt_hi, idx - kWave);
    const int phys = min(max(P >> 3, 0), max_block);  // a bad table cannot leave the pools
    const size_t row0 = ((size_t)phys * Hkv + g) * 128 + (size_t)pg0 * 16;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      load_page<KV>(ch[j], k_pool, v_pool, k_scale, v_scale, row0 + 16 * j, lane);
    return row0;
  };
  // the online-softmax update with chunk ci
  auto body = [&](Chunk<KV> (&ch)[2], int ci, size_t row0) {
    const int u = ci >> 2;
    const int pg0 = (ci & 3) * 2;
    const bool local = u == nblk - 1;
    if constexpr (KV == 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        load_v_lds(v_pool, row0 + 16 * j, lane, stage + 16 * j * kVRow);
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) stage_v<KV>(ch[j], stage + 16 * j * kVRow, lane);
    }

    // S^T = K Q^T for the two pages
    f32x4 sacc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      sacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand<KV>(ch[j], kk), qop[kk],
                                                          sacc[j], 0, 0, 0);
    }
    // online softmax over the chunk (log2 domain); keys past the row's
    // position in its local block, and columns past G, are masked
    const int lim = hl < G ? (local ? vloc : 128) : 0;
    float z[8];
    float mc = neg_inf();
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = sacc[j][i] * scale_log2;
        if constexpr (KV == 1) v *= ch[j].kscale[i];
        const int tok = 16 * (pg0 + j) + 4 * g4 + i;
        v = tok < lim ? v : neg_inf();
        z[4 * j + i] = v;
        mc = fmaxf(mc, v);
      }
    mc = fmaxf(mc, __shfl_xor(mc, 16));
    mc = fmaxf(mc, __shfl_xor(mc, 32));
    const float mn = fmaxf(m, mc);
    const float alpha = mn == m ? 1.f : __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    // P as bf16 hi + lo: hi = RNE(p), lo = RNE(p - hi).  bf16 KV: integer
    // rounding; fp8 / 4-bit KV: two values per v_cvt_pk_bf16_f32 (same bits;
    // the bf16-KV kernel measured slower with it, 48.3 vs 43.7 us on the
    // 128K layer, so it keeps its code).
    float psum = 0.f;
    u32x4 bh, bl;
    if constexpr (KV == 0) {
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = z[e] == neg_inf() ? 0.f : __builtin_amdgcn_exp2f(z[e] - mn);
        psum += p;
        float pv = p;
        hi[e] = bf16_rne_bits(pv);
        lo[e] = bf16_rne_bits(pv - bf16_bits_to_f32(hi[e]));
      }
      bh.x = hi[0] | (hi[1] << 16); bh.y = hi[2] | (hi[3] << 16);
      bh.z = hi[4] | (hi[5] << 16); bh.w = hi[6] | (hi[7] << 16);
      bl.x = lo[0] | (lo[1] << 16); bl.y = lo[2] | (lo[3] << 16);
      bl.z = lo[4] | (lo[5] << 16); bl.w = lo[6] | (lo[7] << 16);
    } else {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = z[e] == neg_inf() ? 0.f : __builtin_amdgcn_exp2f(z[e] - mn);
        psum += p;
        pv[e] = p;
        if constexpr (KV == 1) pv[e] *= ch[e >> 2].vscale[e & 3];
      }
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f32x2 pp = {pv[2 * w], pv[2 * w + 1]};
        hw[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pp, bf16x2));
        const f32x2 rest = {pp.x - bf16_bits_to_f32(hw[w] & 0xFFFFu),
                            pp.y - __builtin_bit_cast(float, hw[w] & 0xFFFF0000u)};
        lw[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(rest, bf16x2));
      }
      bh = u32x4{hw[0], hw[1], hw[2], hw[3]};
      bl = u32x4{lw[0], lw[1], lw[2], lw[3]};
    }
    lsum = lsum * alpha + psum;
    const bf16x8 phi = __builtin_bit_cast(bf16x8, bh);
    const bf16x8 plo = __builtin_bit_cast(bf16x8, bl);
#pragma unroll
    for (int s = 0; s < 8; ++s) oacc[s] *= alpha;

    if constexpr (KV == 0) __builtin_amdgcn_s_waitcnt(kWaitVmem);  // V rows landed in LDS
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // O^T += V^T P^T, dims in blocks of 16.  The operand of lane (dim hl,
    // group g4) is keys kappa(g4, 0..7) of its dim, the order of P^T.  A
    // transposing read gives lane i of a 16-lane group element e of lane
    // 4 e + i / 4, so there lane j of the group points at 4 dims
    // (4 (j mod 4) ..) of row 4 g4 + j / 4, and the row 16 further on for
    // the second half.
    const int vrow = 4 * g4 + (hl >> 2);
    const uint8_t* vrd = stage + vrow * kVRow + 8 * (hl & 3);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16x8 aop;
      if constexpr (KV == 0) {
        // dim 16 s + hl of rows kappa(g4, .), all with vswz = 2 g4
        const uint8_t* col = stage + 32 * (s ^ g4) + 2 * hl;
        uint32_t a[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t x0 = *reinterpret_cast<const uint16_t*>(col + kappa(g4, 2 * w) * kVRow);
          const uint32_t x1 =
              *reinterpret_cast<const uint16_t*>(col + kappa(g4, 2 * w + 1) * kVRow);
          a[w] = x0 | (x1 << 16);
        }
        const u32x4 av = {a[0], a[1], a[2], a[3]};
        aop = __builtin_bit_cast(bf16x8, av);
      } else {
        const uint8_t* p0 = vrd + 32 * (s ^ (vrow & 7));
        const v4i16 k0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p0);
        const v4i16 k1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0 + 16 * kVRow));
        const v8i16 kv = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
        aop = __builtin_bit_cast(bf16x8, kv);
      }
      oacc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, phi, oacc[s], 0, 0, 0);
      oacc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, plo, oacc[s], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  for (int ci = split + S * wave; ci < limit; ci += S * W) {
    Chunk<KV> ch[2];
    const size_t row0 = load_chunk(ch, ci);
    body(ch, ci, row0);
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);

  // ---- combine the W waves in LDS (the stage areas are free now)
  combine_tile<W>(smem, m, lsum, oacc, G, [&](int h, int d, const f32x4& O, float M, float Ls) {
    const size_t rh = (size_t)r * Hq + g * G + h;
    store_result(O, M, Ls, rh, d, S, split, out, part_o, part_ml);
  });
}

// ---- multi-row requests: one workgroup per (request, KV head, split)
// The T rows of a speculative-verify request (news.ainew.jp article,
// section "EAGLE3 が第 2 のデコードループを追加": flattened verify rows of one
// request) select mostly the same blocks.  This workgroup walks the union of
// their blocks once, with the T x G (row, query head) pairs of its KV head as
// the MFMA columns (one or two tiles of 16), so each K/V byte of the union is
// fetched once per request -- the reuse of key loads across draft positions
// that section 2 of the same article gets from one indexer workgroup per
// request.  A column masks the keys its row does not attend: blocks outside
// the row's selection, and keys past the row's position in its local block.
constexpr int kUnionMaxRows = 4;  // T x 16 table slots fit one wave

// The union of request b's row selections, built by each wave on its own
// from the rows' page tables (first page of each block group): on return
// lane u < n holds union block u's physical block and its membership bits
// (bit t: row t attends it; bit 8 + t: it is row t's local block, the last
// group of the row).  Returns n.
__device__ __forceinline__ int union_of_rows(const int32_t* __restrict__ page_table, int b,
                                             int T, int PT, int lane, int& u_phys,
                                             int& u_bits) {
  const int t = lane >> 4, k = lane & 15;
  int phys = -1;
  if (t < T && 8 * k < PT) {
    const int e = page_table[(size_t)(b * T + t) * PT + 8 * k];
    phys = e >= 0 ? (e >> 3) : -1;
  }
  const uint64_t valid = __ballot(phys >= 0);
  const int n_row = __popcll((valid >> (16 * t)) & 0xFFFFull);
  const uint64_t localm = __ballot(phys >= 0 && k == n_row - 1);
  // lanes holding the same block as this one
  uint64_t same = 0;
  for (int j = 0; j < kWave; ++j) {
    const int pj = __builtin_amdgcn_readlane(phys, j);
    const uint64_t m = __ballot(phys == pj);
    if (lane == j) same = m;
  }
  const bool first = phys >= 0 && (same & ((1ull << lane) - 1)) == 0;
  int bits = 0;
#pragma unroll
  for (int r = 0; r < kUnionMaxRows; ++r) {
    if ((same >> (16 * r)) & 0xFFFFull) bits |= 1 << r;
    if (((same & localm) >> (16 * r)) & 0xFFFFull) bits |= 1 << (8 + r);
  }
  // compact: the first lane of each block to its rank, the rest behind
  const uint64_t firsts = __ballot(first);
  const int n = __popcll(firsts);
  const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(firsts >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)firsts, 0u));
  const int dst = first ? below : n + (lane - below);
  u_phys = __builtin_amdgcn_ds_permute(dst * 4, phys);
  u_bits = __builtin_amdgcn_ds_permute(dst * 4, bits);
  return n;
}

// fp8 chunks are prefetched: the raw K, V and scale bytes of a wave's next
// chunk go from HBM straight into a per-wave LDS slot (direct-to-LDS loads,
// no registers) while the current chunk is computed; K and the scales are
// read back into the registers load_page would have filled, and V either
// too (then widened into the staging area) or, with two slots per wave
// (RAWV), read as V^T straight from the slot by transposing 8-bit reads.
// Slot layout: K loads (page, half) at 1 KB each, V loads at 4 KB + 1 KB
// each (key rows of 128 bytes), and 64 fp32 scales (32 K scales, then 32 V
// scales) at 8 KB.
constexpr int kSlotBytes = 8192 + 256;
constexpr int kWaitLgkm = 0xC07F;  // s_waitcnt operand: lgkmcnt == 0 only

// One direct-to-LDS load of 16 (or 4) bytes per lane from `src` to LDS
// address `lds` + lane * 16 (4), non-temporal.  Written as inline asm so
// that the compiler does not take every later LDS access of the wave as
// dependent on it and wait for it there (it cannot tell the prefetch slot
// from the staging area); the kernel waits for these loads itself (vmcnt)
// before it reads the slot.  The instructions have no register outputs; m0
// carries the LDS address.
__device__ __forceinline__ void lds_dma_b128(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(src), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_dma_b32(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off nt"
               :
               : "v"(src), "s"(lds)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_address(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// Raw V rows in a slot (RAWV): 16-byte granule c of key row k sits at
// granule c ^ rawv_swz(k) of the row, so that the 8 rows one transposing
// read of a lane group touches (kappa(g4, 0..7): 4 of each parity) fall on
// distinct banks, and so do those of lane groups 0 and 1 (and 2 and 3),
// whose rows differ in bit 2.
__device__ __forceinline__ int rawv_swz(int k) {
  return ((k >> 1) & 1) | ((k >> 3) & 2) | (k & 4);
}

template <bool RAWV>
__device__ __forceinline__ void prefetch_chunk_fp8(uint8_t* slot,
                                                   const uint8_t* __restrict__ k_pool,
                                                   const uint8_t* __restrict__ v_pool,
                                                   const float* __restrict__ k_scale,
                                                   const float* __restrict__ v_scale,
                                                   size_t row0, int lane) {
  const int m = lane & 15, g = lane >> 4;
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_address(slot));
#pragma unroll
  for (int jp = 0; jp < 2; ++jp) {
    const size_t r = row0 + 16 * jp;
    const uint8_t* kp = k_pool + (r + m) * 128 + 16 * g;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      lds_dma_b128(kp + 64 * i, base + (2 * jp + i) * 1024);
      // V: LDS granule `lane` of this 1 KB holds key row 16 jp + 8 i + lane / 8
      const int kr = 16 * jp + 8 * i + (lane >> 3);
      const int c = RAWV ? ((lane & 7) ^ rawv_swz(kr)) : (lane & 7);
      lds_dma_b128(v_pool + (row0 + kr) * 128 + 16 * c, base + 4096 + (2 * jp + i) * 1024);
    }
  }
  const float* sp = (lane < 32 ? k_scale : v_scale) + row0 + (lane & 31);
  lds_dma_b32(sp, base + 8192);
}

// The registers of page jp of a prefetched fp8 chunk, as load_page<1> fills
// them (RAWV: K and the scales only; V stays in the slot).
template <bool RAWV>
__device__ __forceinline__ void read_page_fp8(Chunk<1>& c, const uint8_t* slot, int jp,
                                              int lane) {
  const int g = lane >> 4;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    c.k[i] = *reinterpret_cast<const u32x4*>(slot + (2 * jp + i) * 1024 + 16 * lane);
    if (!RAWV)
      c.v[i] = *reinterpret_cast<const u32x4*>(slot + 4096 + (2 * jp + i) * 1024 + 16 * lane);
  }
  c.kscale = *reinterpret_cast<const f32x4*>(slot + 8192 + (16 * jp + 4 * g) * 4);
  c.vscale = *reinterpret_cast<const f32x4*>(slot + 8192 + 128 + (16 * jp + 4 * g) * 4);
}

// s_waitcnt operand that waits until at most n vector-memory operations
// are outstanding (gfx9 encoding: vmcnt bits [3:0] and [15:14]).
constexpr int vmcnt_imm(int n) { return ((n >> 4) << 14) | 0x0F70 | (n & 15); }
constexpr int kDmaPerChunk = 9;  // direct-to-LDS loads per prefetched fp8 chunk

// Every wave computes all NT tiles of each of its chunks, so each union
// block is loaded once per request.  fp8 (D > 0): each wave keeps up to D
// chunks in flight in a ring of LDS slots.  SEL: the workgroup first
// selects the request's rows itself (its first four waves, from the block
// scores; page ids into LDS) instead of reading a page table.
template <int KV, int W, int NT, int D, bool SEL>
__global__ __launch_bounds__(64 * W, W == 4 ? 1 : 2) void union_attn_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ k_pool,
    const uint8_t* __restrict__ v_pool, const void* __restrict__ k_scale,
    const void* __restrict__ v_scale, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ ctx_lens, float* __restrict__ part_o,
    float* __restrict__ part_ml, float* __restrict__ out, int B, int T, int Hq, int Hkv, int PT,
    int S, int max_block, float scale_log2, SelectArgs sa, int MAXB) {
  constexpr bool kPrefetch = D > 0;
  static_assert(!kPrefetch || KV == 1, "prefetch ring for fp8 chunks");
  static_assert(D <= 3, "vmcnt waits below cover up to 3 chunks in flight");
  // RAWV (fp8, two slots per wave): P V reads V^T straight from the raw fp8
  // rows of the slot (transposing 8-bit reads), so no staging area; the
  // selection and the final combine use the slots' memory instead.
  constexpr bool kRawV = KV == 1 && D == 2;
  static_assert(!kRawV || W * D * kSlotBytes >= W * kWaveLds, "combine area in the slots");
  __shared__ __attribute__((aligned(16))) uint8_t smem_arr[kRawV ? 16 : W * kWaveLds];
  __shared__ __attribute__((aligned(16))) uint8_t slots[kPrefetch ? W * D * kSlotBytes : 16];
  uint8_t* smem = kRawV ? slots : smem_arr;

  const int lane = lane_id();
  const int wave = wave_id();
  int x = blockIdx.x;
  const int split = x % S;
  x /= S;
  const int g = x % Hkv;
  const int b = x / Hkv;
  if (b >= B) return;
  const int G = Hq / Hkv;
  const int L = ctx_lens[b];

  // Column hl of tile j is (row t, query head h) = divmod(16 j + hl, G);
  // Q^T operands as in the per-row kernel, zero for columns past T G.
  const int hl = lane & 15;
  const int g4 = lane >> 4;
  bf16x8 qop[NT][4];
  int trow[NT], vloc[NT];
  bool cvalid[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int col = 16 * j + hl;
    cvalid[j] = col < T * G;
    const int cc = cvalid[j] ? col : 0;
    trow[j] = cc / G;
    vloc[j] = ((L - T + trow[j]) & 127) + 1;
    const u32x4 z = {0u, 0u, 0u, 0u};
    const uint16_t* qp = q + ((size_t)(b * T + trow[j]) * Hq + g * G + cc % G) * kD;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u32x4 v = ldg128(qp + kdim<KV>(g4, kk));
      qop[j][kk] = __builtin_bit_cast(bf16x8, cvalid[j] ? v : z);
    }
  }

  // rows whose columns fall in tile j: a chunk of a block none of them
  // selects skips the tile's work (its columns would all be masked)
  int tmask[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    tmask[j] = 0;
    for (int r = 0; r < T; ++r)
      if (r * G < 16 * j + 16 && (r + 1) * G > 16 * j) tmask[j] |= 1 << r;
  }

  int u_phys, u_bits, nU;
  if constexpr (SEL) {
    // every (KV head, split) workgroup of the request selects (T <= 4 rows,
    // one wave each); the (0, 0) one exports.  The selection's LDS and the
    // rows' page ids sit in the staging area, free until the chunk loop.
    static_assert(W >= 4, "four selecting waves");
    static_assert(((sizeof(SelectLds<4>) + 15) & ~15) +
                          (kUnionMaxRows * kMaxTopk * 8 + 2 * kWave + 1) * sizeof(int32_t) <=
                      (size_t)W * kWaveLds,
                  "the selection, the rows' page ids and the union fit the staging area");
    auto* ssh = reinterpret_cast<SelectLds<4>*>(smem);
    int32_t* prow = reinterpret_cast<int32_t*>(smem + ((sizeof(SelectLds<4>) + 15) & ~15));
    const bool exporter = g == 0 && split == 0;
    select_request<4, W>(b, sa.scores, ctx_lens, sa.block_table,
                         exporter ? sa.selected : nullptr, exporter ? sa.n_selected : nullptr,
                         exporter ? sa.page_table : nullptr, T, MAXB, PT / 8, *ssh, prow);
    // one wave builds the union and hands it to the others through LDS
    int32_t* ushare = prow + kUnionMaxRows * PT;  // phys [64], bits [64], count
    if (wave == 0) {
      const int n = union_of_rows(prow, 0, T, PT, lane, u_phys, u_bits);
      ushare[lane] = u_phys;
      ushare[kWave + lane] = u_bits;
      if (lane == 0) ushare[2 * kWave] = n;
    }
    __syncthreads();
    u_phys = ushare[lane];
    u_bits = ushare[kWave + lane];
    nU = __builtin_amdgcn_readfirstlane(ushare[2 * kWave]);
    __syncthreads();  // the page ids and the union are read: the staging area is free
  } else {
    nU = union_of_rows(page_table, b, T, PT, lane, u_phys, u_bits);
  }
  const int nchunks = 4 * nU;

  float m[NT], lsum[NT];
  f32x4 oacc[NT][8];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    m[j] = neg_inf();
    lsum[j] = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) oacc[j][s] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  uint8_t* stage = smem + wave * kWaveLds;
  uint8_t* ring = slots + (kPrefetch ? wave * D * kSlotBytes : 0);
  // Keys of union block u that some row attends: all of it when it is not
  // the local block of every row that selects it, else up to the position
  // of the last such row (positions rise with t inside one block).  A chunk
  // wholly past that is skipped.
  auto wanted = [&](int ci) {
    const int bits = __builtin_amdgcn_readlane(u_bits, ci >> 2);
    const int rows = bits & 0xFF, locs = (bits >> 8) & 0xFF;
    const int reach = (rows & ~locs) ? 128 : ((L - T + (31 - __builtin_clz(locs))) & 127) + 1;
    return (ci & 3) * 32 < reach;
  };
  auto next_wanted = [&](int ci) {
    while (ci < nchunks && !wanted(ci)) ci += S * W;
    return ci;
  };
  auto chunk_row0 = [&](int ci) {
    const int P = __builtin_amdgcn_readlane(u_phys, ci >> 2);
    const int phys = min(max(P, 0), max_block);  // a bad table cannot leave the pools
    return ((size_t)phys * Hkv + g) * 128 + (size_t)(ci & 3) * 32;
  };

  int ci = next_wanted(split + S * wave);
  // the ring: chunks are consumed in the order they were issued; `ahead`
  // is the next chunk to issue, `inflight` how many sit in the ring
  int ahead = ci, inflight = 0, cur = 0;
  auto issue = [&](int sl) {
    prefetch_chunk_fp8<kRawV>(ring + sl * kSlotBytes, k_pool, v_pool,
                       static_cast<const float*>(k_scale), static_cast<const float*>(v_scale),
                       chunk_row0(ahead), lane);
    ahead = next_wanted(ahead + S * W);
    ++inflight;
  };
  if constexpr (kPrefetch) {
    for (int sl = 0; sl < D && ahead < nchunks; ++sl) issue(sl);
  }
  while (ci < nchunks) {
    const int bits = __builtin_amdgcn_readlane(u_bits, ci >> 2);
    const int pg0 = (ci & 3) * 2;
    const size_t row0 = chunk_row0(ci);
    const int nci = next_wanted(ci + S * W);
    Chunk<KV> ch[2];
    int used = 0;  // RAWV: the slot this chunk's V stays in until P V
    if constexpr (kPrefetch) {
      // this chunk (the oldest in flight) has landed once no more than the
      // younger chunks' loads are outstanding
      if (inflight >= 3)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kDmaPerChunk));
      else if (inflight == 2)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kDmaPerChunk));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      asm volatile("" ::: "memory");
      uint8_t* slot = ring + cur * kSlotBytes;
#pragma unroll
      for (int jp = 0; jp < 2; ++jp) read_page_fp8<kRawV>(ch[jp], slot, jp, lane);
      --inflight;
      used = cur;
      if constexpr (!kRawV) {
        __builtin_amdgcn_s_waitcnt(kWaitLgkm);  // slot read: it may take the next chunk
        asm volatile("" ::: "memory");
        if (ahead < nchunks) issue(cur);
      }
      cur = cur + 1 == D ? 0 : cur + 1;
    } else {
#pragma unroll
      for (int jp = 0; jp < 2; ++jp)
        load_page<KV>(ch[jp], k_pool, v_pool, k_scale, v_scale, row0 + 16 * jp, lane);
    }
    if constexpr (KV == 0) {
#pragma unroll
      for (int jp = 0; jp < 2; ++jp)
        load_v_lds(v_pool, row0 + 16 * jp, lane, stage + 16 * jp * kVRow);
    } else if constexpr (!kRawV) {
#pragma unroll
      for (int jp = 0; jp < 2; ++jp) stage_v<KV>(ch[jp], stage + 16 * jp * kVRow, lane);
    }

    // logit scale per key: the softmax scale (log2 domain) times the fp8
    // K scale, shared by the tiles
    float ks[2][4];
#pragma unroll
    for (int jp = 0; jp < 2; ++jp)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ks[jp][i] = scale_log2;
        if constexpr (KV == 1) ks[jp][i] = scale_log2 * ch[jp].kscale[i];
      }
    // a skipped tile keeps zero P, so its P V products below add nothing
    bf16x8 phi[NT], plo[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const u32x4 z4 = {0u, 0u, 0u, 0u};
      phi[j] = __builtin_bit_cast(bf16x8, z4);
      plo[j] = phi[j];
      if (!(bits & tmask[j])) continue;
      // S^T = K Q^T for the two pages, this tile's columns
      f32x4 sacc[2];
#pragma unroll
      for (int jp = 0; jp < 2; ++jp) {
        sacc[jp] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          sacc[jp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand<KV>(ch[jp], kk),
                                                             qop[j][kk], sacc[jp], 0, 0, 0);
      }
      // this column's keys: none when its row does not select the block, up
      // to its position when the block is its row's local block
      const bool inrow = cvalid[j] && ((bits >> trow[j]) & 1);
      const bool isloc = (bits >> (8 + trow[j])) & 1;
      const int lim = inrow ? (isloc ? vloc[j] : 128) : 0;
      float z[8];
      float mc = neg_inf();
#pragma unroll
      for (int jp = 0; jp < 2; ++jp)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = sacc[jp][i] * ks[jp][i];
          const int tok = 16 * (pg0 + jp) + 4 * g4 + i;
          v = tok < lim ? v : neg_inf();
          z[4 * jp + i] = v;
          mc = fmaxf(mc, v);
        }
      mc = fmaxf(mc, __shfl_xor(mc, 16));
    mc = fmaxf(mc, __shfl_xor(mc, 32));
      const float mn = fmaxf(m[j], mc);
      // exponents relative to a finite maximum: masked logits (-inf) give
      // exactly 0, an unchanged maximum gives alpha = 1, and a column with
      // nothing unmasked yet keeps zero sums
      const float mref = mn == neg_inf() ? 0.f : mn;
      const float alpha = __builtin_amdgcn_exp2f(m[j] - mref);
      m[j] = mn;
      // P as bf16 hi + lo (two values per conversion), V scales folded in
      float psum = 0.f;
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = __builtin_amdgcn_exp2f(z[e] - mref);
        psum += pe;
        pv[e] = pe;
        if constexpr (KV == 1) pv[e] *= ch[e >> 2].vscale[e & 3];
      }
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f32x2 pp = {pv[2 * w], pv[2 * w + 1]};
        hw[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pp, bf16x2));
        const f32x2 rest = {pp.x - bf16_bits_to_f32(hw[w] & 0xFFFFu),
                            pp.y - __builtin_bit_cast(float, hw[w] & 0xFFFF0000u)};
        lw[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(rest, bf16x2));
      }
      phi[j] = __builtin_bit_cast(bf16x8, (u32x4{hw[0], hw[1], hw[2], hw[3]}));
      plo[j] = __builtin_bit_cast(bf16x8, (u32x4{lw[0], lw[1], lw[2], lw[3]}));
      lsum[j] = lsum[j] * alpha + psum;
#pragma unroll
      for (int s = 0; s < 8; ++s) oacc[j][s] *= alpha;
    }

    if constexpr (KV == 0) __builtin_amdgcn_s_waitcnt(kWaitVmem);  // V rows landed in LDS
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // O^T += V^T P^T per tile; the V^T operand is shared by the tiles
    const int vrow = 4 * g4 + (hl >> 2);
    const uint8_t* vrd = stage + vrow * kVRow + 8 * (hl & 3);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16x8 aop;
      if constexpr (KV == 0) {
        const uint8_t* colp = stage + 32 * (s ^ g4) + 2 * hl;
        uint32_t a[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t x0 = *reinterpret_cast<const uint16_t*>(colp + kappa(g4, 2 * w) * kVRow);
          const uint32_t x1 =
              *reinterpret_cast<const uint16_t*>(colp + kappa(g4, 2 * w + 1) * kVRow);
          a[w] = x0 | (x1 << 16);
        }
        const u32x4 av = {a[0], a[1], a[2], a[3]};
        aop = __builtin_bit_cast(bf16x8, av);
      } else if constexpr (kRawV) {
        // lane (dim hl, group g4) needs keys kappa(g4, 0..7) of dim 16 s + hl;
        // a transposing 8-bit read gives lane i of a 16-lane group byte
        // i mod 8 of the 8-byte runs that lanes 2 e + i / 8 point at, so lane
        // j points at dims 16 s + 8 (j % 2) .. of key kappa(g4, j / 2)
        const int kr = kappa(g4, hl >> 1);
        const uint8_t* p0 = ring + used * kSlotBytes + 4096 + kr * 128 +
                            16 * (s ^ rawv_swz(kr)) + 8 * (hl & 1);
        const lds_v2i32_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32*)p0);
        const u32x4 o = {e4m3x2_to_bf16x2<false>((uint32_t)r.x),
                         e4m3x2_to_bf16x2<true>((uint32_t)r.x),
                         e4m3x2_to_bf16x2<false>((uint32_t)r.y),
                         e4m3x2_to_bf16x2<true>((uint32_t)r.y)};
        aop = __builtin_bit_cast(bf16x8, o);
      } else {
        const uint8_t* p0 = vrd + 32 * (s ^ (vrow & 7));
        const v4i16 k0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p0);
        const v4i16 k1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0 + 16 * kVRow));
        const v8i16 kv = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
        aop = __builtin_bit_cast(bf16x8, kv);
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        oacc[j][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, phi[j], oacc[j][s], 0, 0, 0);
        oacc[j][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, plo[j], oacc[j][s], 0, 0, 0);
      }
    }
    if constexpr (kRawV) {
      // the slot's V has been read: it takes the next chunk to issue
      __builtin_amdgcn_s_waitcnt(kWaitLgkm);
      asm volatile("" ::: "memory");
      if (ahead < nchunks) issue(used);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    ci = nci;
  }

  // ---- combine the W waves in LDS, one tile at a time
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    float ls = lsum[j];
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    combine_tile<W>(smem, m[j], ls, oacc[j], T * G - 16 * j,
                    [&](int c, int d, const f32x4& O, float M, float Ls) {
                      const int col = 16 * j + c;
                      const size_t rh = (size_t)(b * T + col / G) * Hq + g * G + col % G;
                      store_result(O, M, Ls, rh, d, S, split, out, part_o, part_ml);
                    });
  }
}

// out[rh][d] = sum_s 2^(m_s - M) O_s[d] / sum_s 2^(m_s - M) l_s
// Splits per row never exceed kMaxSplits (plan_splits caps them); every
// split's (m, l) and partial row load in one round trip, then combine in
// split order.
constexpr int kMaxSplits = 8;

__global__ __launch_bounds__(128) void lse_merge_kernel(const float* __restrict__ part_o,
                                                        const float* __restrict__ part_ml,
                                                        float* __restrict__ out, int S) {
  const size_t rh = blockIdx.x;
  const int d = threadIdx.x;
  const float* ml = part_ml + rh * S * 2;
  float ms[kMaxSplits], ls[kMaxSplits], os[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    ms[s] = s < S ? ml[2 * s] : neg_inf();
    ls[s] = s < S ? ml[2 * s + 1] : 0.f;
    os[s] = s < S ? part_o[(rh * S + s) * kD + d] : 0.f;
  }
  float M = neg_inf();
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) M = fmaxf(M, ms[s]);
  float O = 0.f, Ls = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    if (s >= S) break;
    const float f = ms[s] == neg_inf() ? 0.f : __builtin_amdgcn_exp2f(ms[s] - M);
    O += f * os[s];
    Ls += f * ls[s];
  }
  out[rh * kD + d] = Ls > 0.f ? O / Ls : 0.f;
}

__global__ void selftest_kernel(float* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < 256) {
    const uint32_t pair = e4m3x2_to_bf16x2<false>((uint32_t)i);
    out[i] = bf16_bits_to_f32(pair & 0xFFFFu);
  } else if (i < 256 + 16) {
    out[i] = e2m1x2_to_f32x2((uint32_t)(i - 256), 0).x;
  } else if (i < 256 + 32) {
    out[i] = e2m1x2_to_f32x2((uint32_t)(i - 272) << 4, 0).y;
  } else if (i < 544) {
    out[i] = e4m3_to_f32((uint32_t)(i - 288));
  } else if (i < 560) {
    out[i] = bf16_bits_to_f32(e2m1x2_to_bf16x2<0>((uint32_t)(i - 544)) & 0xFFFFu);
  } else if (i < 576) {
    out[i] = bf16_bits_to_f32(e2m1x2_to_bf16x2<0>((uint32_t)(i - 560) << 4) >> 16);
  } else if (i < 832) {
    out[i] = e4m3x2_to_f32x2((uint32_t)(i - 576) << 8).y;
  }
}

// Workgroups of one launch; with T > 1 the request count is padded to a
// multiple of 8 for the XCD-aware id mapping.
long attention_workgroups(const Dims& d, const SplitPlan& sp) {
  if (sp.rows_union) return (long)d.B * d.Hkv * sp.splits;
  const long reqs = d.T > 1 ? (d.B + 7) / 8 * 8 : d.B;
  return reqs * d.T * d.Hkv * sp.splits;
}

// fp8 union workgroups: 8 waves, each with two LDS slots of raw chunk
// bytes: the next chunk lands in one while the current one is computed from
// the other, V^T read straight from its raw rows (one workgroup per CU:
// 135 KB of LDS, about 210 registers); other formats: 8 waves, no prefetch.
// Measured on MI355X (fp8 spec-verify layer, 128 requests x 4 rows, step
// after a 1 GiB cache flush / back to back): one slot per wave with V
// widened into a bf16 staging area 81.5 / 77.8 us, against 90.9 / 74.5 us
// for one workgroup per row; 4 waves with 3 chunks in flight each took
// 97.4 / 92.7 us (one wave per SIMD leaves the per-chunk compute exposed).
// The raw-V slots then cut the chunk loop from 716 to 671 instructions (40
// to 20 LDS instructions per chunk): attention alone 50.0-50.1 vs
// 50.4-51.5 us on two boxes; the whole step moved within the boxes' noise.
constexpr int kUnionWavesFp8 = 8;
constexpr int kUnionDepthFp8 = 2;

template <int KV, int NT, bool SEL>
hipError_t launch_union(const Dims& d, const SplitPlan& sp, const void* q, const void* k_pool,
                        const void* v_pool, const void* k_scale, const void* v_scale,
                        const int32_t* page_table, const int32_t* ctx_lens, float* part_o,
                        float* part_ml, float* out, const SelectArgs& sa, hipStream_t s) {
  constexpr int W = KV == 1 ? kUnionWavesFp8 : 8;
  constexpr int D = KV == 1 ? kUnionDepthFp8 : 0;
  hipLaunchKernelGGL((union_attn_kernel<KV, W, NT, D, SEL>),
                     dim3((unsigned)attention_workgroups(d, sp)), dim3(64 * W), 0, s,
                     static_cast<const uint16_t*>(q), static_cast<const uint8_t*>(k_pool),
                     static_cast<const uint8_t*>(v_pool), k_scale, v_scale, page_table,
                     ctx_lens, part_o, part_ml, out, d.B, d.T, d.Hq, d.Hkv, d.PT(), sp.splits,
                     d.NB - 1, d.scale_log2, sa, d.MAXB);
  return hipGetLastError();
}

template <int KV, int W, bool SEL>
hipError_t launch_kvw(const Dims& d, const SplitPlan& sp, const void* q, const void* k_pool,
                      const void* v_pool, const void* k_scale, const void* v_scale,
                      const int32_t* page_table, const int32_t* ctx_lens, float* part_o,
                      float* part_ml, float* out, const SelectArgs& sa, hipStream_t s) {
  hipLaunchKernelGGL((sparse_attn_kernel<KV, W, SEL>),
                     dim3((unsigned)attention_workgroups(d, sp)), dim3(64 * W), 0, s,
                     static_cast<const uint16_t*>(q), static_cast<const uint8_t*>(k_pool),
                     static_cast<const uint8_t*>(v_pool), k_scale, v_scale, page_table,
                     ctx_lens, part_o, part_ml, out, d.B, d.T, d.Hq, d.Hkv, d.PT(), sp.splits,
                     d.NB - 1, d.scale_log2, sa, d.MAXB);
  return hipGetLastError();
}

template <int KV>
hipError_t launch_kv(const Dims& d, const SplitPlan& sp, const void* q, const void* k_pool,
                     const void* v_pool, const void* k_scale, const void* v_scale,
                     const int32_t* page_table, const int32_t* ctx_lens, float* part_o,
                     float* part_ml, float* out, const SelectArgs* sel, hipStream_t s) {
  if (sp.rows_union) {
    const SelectArgs none{};
    if (sel) {
      if (sp.tiles == 1)
        return launch_union<KV, 1, true>(d, sp, q, k_pool, v_pool, k_scale, v_scale, nullptr,
                                         ctx_lens, part_o, part_ml, out, *sel, s);
      return launch_union<KV, 2, true>(d, sp, q, k_pool, v_pool, k_scale, v_scale, nullptr,
                                       ctx_lens, part_o, part_ml, out, *sel, s);
    }
    if (sp.tiles == 1)
      return launch_union<KV, 1, false>(d, sp, q, k_pool, v_pool, k_scale, v_scale, page_table,
                                        ctx_lens, part_o, part_ml, out, none, s);
    return launch_union<KV, 2, false>(d, sp, q, k_pool, v_pool, k_scale, v_scale, page_table,
                                      ctx_lens, part_o, part_ml, out, none, s);
  }
  if (sel)
    return launch_kvw<KV, 8, true>(d, sp, q, k_pool, v_pool, k_scale, v_scale, nullptr,
                                   ctx_lens, part_o, part_ml, out, *sel, s);
  const SelectArgs none{};
  if (sp.waves == 8)
    return launch_kvw<KV, 8, false>(d, sp, q, k_pool, v_pool, k_scale, v_scale, page_table,
                                    ctx_lens, part_o, part_ml, out, none, s);
  return launch_kvw<KV, 4, false>(d, sp, q, k_pool, v_pool, k_scale, v_scale, page_table,
                                  ctx_lens, part_o, part_ml, out, none, s);
}

}  // namespace

// Multi-row requests with at most this many rows walk the union of their
// rows' blocks in one workgroup (the rows' table slots fit one wave), when
// their (row, query head) pairs fit two 16-column tiles.
bool union_eligible(const Dims& d) {
  return d.T > 1 && d.T <= kUnionMaxRows && d.T * d.G() <= 32;
}

SplitPlan plan_splits(const Dims& d) {
  // One workgroup per (row, KV head, split), or per (request, KV head,
  // split) for multi-row requests that walk their union.  Work is split
  // only until there is one workgroup per CU (256), keeping at least one
  // chunk of 32 keys per wave of 8.  On MI355X 8 waves per workgroup
  // measured faster than 4 or 16, and fewer splits faster than more (less
  // merging).
  SplitPlan p;
  p.rows_union = union_eligible(d);
  p.tiles = p.rows_union ? (d.T * d.G() + 15) / 16 : 1;
  // at most 4 chunks per selected block (of the union: T times the rows')
  const int chunks = 4 * d.topk * (p.rows_union ? d.T : 1);
  const long pairs = p.rows_union ? (long)d.B * d.Hkv : (long)d.R() * d.Hkv;
  const long target = 256;
  int S = 1;
  while (S * 2 <= chunks / 8 && S * 2 <= kMaxSplits && pairs * S < target) S *= 2;
  p.splits = S;
  if (p.rows_union)
    p.waves = d.kv_dtype == 1 ? kUnionWavesFp8 : 8;
  else
    p.waves = (chunks + S - 1) / S >= 8 ? 8 : 4;
  return p;
}

// Rows of at most this many blocks select inside the attention launch.
// Every workgroup of a row reads the row's scores (64 KB at this bound);
// measured on MI355X the fused launch is faster up to the 1M context (8192
// blocks: 177 vs 181 us per step, 182.5 vs 187.7 after a cache flush).
constexpr int kFusedSelectMaxBlocks = 16384;

bool fused_select_eligible(const Dims& d) {
  if (d.MAXB > kFusedSelectMaxBlocks) return false;
  return union_eligible(d) || (d.T == 1 && plan_splits(d).waves == 8);
}

hipError_t launch_sparse_attention(const Dims& d, const void* q, const void* k_pool,
                                   const void* v_pool, const void* k_scale,
                                   const void* v_scale, const int32_t* page_table,
                                   const int32_t* ctx_lens, float* part_o, float* part_ml,
                                   float* out, hipStream_t s, std::string* note,
                                   const SelectArgs* sel) {
  const SplitPlan sp = plan_splits(d);
  if (sel && !fused_select_eligible(d)) return hipErrorInvalidValue;
  hipError_t e;
  if (d.kv_dtype == 0)
    e = launch_kv<0>(d, sp, q, k_pool, v_pool, k_scale, v_scale, page_table, ctx_lens, part_o,
                     part_ml, out, sel, s);
  else if (d.kv_dtype == 1)
    e = launch_kv<1>(d, sp, q, k_pool, v_pool, k_scale, v_scale, page_table, ctx_lens, part_o,
                     part_ml, out, sel, s);
  else
    e = launch_kv<2>(d, sp, q, k_pool, v_pool, k_scale, v_scale, page_table, ctx_lens, part_o,
                     part_ml, out, sel, s);
  if (e != hipSuccess) return e;
  static const char* names[3] = {"bf16", "fp8", "nvfp4"};
  if (note)
    *note += std::string(sp.rows_union ? "sparse_attn_union<" : "sparse_attn<") +
             names[d.kv_dtype] + ">" +
             (sel ? "+select_topk" : "") + "[grid=" +
             std::to_string(attention_workgroups(d, sp)) + "x" + std::to_string(64 * sp.waves) +
             ",splits=" + std::to_string(sp.splits) + "]";
  if (sp.splits > 1) {
    if (sp.splits > kMaxSplits) return hipErrorInvalidValue;
    const unsigned rows = (unsigned)((long)d.R() * d.Hq);
    hipLaunchKernelGGL(lse_merge_kernel, dim3(rows), dim3(kD), 0, s, part_o, part_ml, out,
                       sp.splits);
    if (note) *note += " lse_merge[grid=" + std::to_string(rows) + "x128]";
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_selftest_decoders(float* out, hipStream_t s) {
  hipLaunchKernelGGL(selftest_kernel, dim3(4), dim3(256), 0, s, out);
  return hipGetLastError();
}

}  // namespace msa
