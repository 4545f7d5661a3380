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
//  * A workgroup of 4 waves owns one (row, KV head, split).  Each wave walks
//    chunks of 32 keys (two 16-token pages) of the row's page table.
//  * QK^T on MFMA v_mfma_f32_16x16x32_bf16 with keys as the M dimension and
//    the GQA group's query heads (up to 16) as N: S^T = K Q^T.  K rows go
//    straight from HBM into the A operand (each lane 64 contiguous bytes of
//    one key row); the result leaves every lane with 4 keys of one head, so
//    the softmax statistics of a head never cross lane groups but four.
//  * P V on the same MFMA as O^T = V^T P^T.  P^T is exactly the S^T
//    accumulator layout (no shuffle); V^T needs a transpose, so the V pages
//    are staged through LDS (row stride 264 B keeps the four lane groups on
//    disjoint banks) and read back column-wise.  P is split into bf16 hi + lo
//    halves (two MFMAs) so the weights keep ~16 bits.
//  * fp8 K/V: e4m3 -> bf16 is exact; the per-token K scale multiplies the
//    logit, the V scale multiplies P.  4-bit K/V: e2m1 x e4m3 -> bf16 is
//    exact (at most 6 significant bits) and happens in registers.
//  * Split partials (m, l, unnormalised O) combine inside the workgroup in
//    LDS; across workgroups a small merge kernel applies the LSE rule.
#include "msa_device.h"
#include "msa_internal.h"

#include <math.h>

namespace msa {
namespace {

constexpr int kD = 128;          // head dim
constexpr int kVRow = 264;       // LDS bytes per staged V row (256 + 8 pad)
constexpr int kChunk = 32;       // keys per chunk (two pages)
constexpr int kStage = kChunk * kVRow;  // LDS bytes per wave
constexpr int kORow = 129;       // floats per head row in the merge area

__device__ __forceinline__ float neg_inf() { return -INFINITY; }

// Key row index kappa(g4, jj) within a chunk of the k-slot jj of lane group
// g4 = lane / 16: the order of the S^T accumulator rows.
__device__ __forceinline__ int kappa(int g4, int jj) {
  return jj < 4 ? 4 * g4 + jj : 16 + 4 * g4 + (jj - 4);
}

template <int KV>
struct Chunk {
  // raw loads of one page: K part for this lane's key row / V part
  u32x4 k[KV == 0 ? 4 : (KV == 1 ? 2 : 1)];
  u32x4 v[KV == 0 ? 4 : (KV == 1 ? 2 : 1)];
  uint32_t ks, vs;  // nvfp4: the two e4m3 scale codes of this lane's 32 dims
  f32x4 kscale, vscale;  // fp8: per-token scales of this lane's 4 S^T rows
};

template <int KV>
__device__ __forceinline__ void load_page(Chunk<KV>& c, const uint8_t* __restrict__ k_pool,
                                          const uint8_t* __restrict__ v_pool,
                                          const void* __restrict__ k_scale,
                                          const void* __restrict__ v_scale, size_t row0,
                                          int lane) {
  const int kr = lane & 15, kg = lane >> 4;  // K: key row, 32-dim group
  const int vr = lane >> 2, vg = lane & 3;   // V: key row, 32-dim group
  if constexpr (KV == 0) {
    const uint8_t* kp = k_pool + (row0 + kr) * 256 + kg * 64;
    const uint8_t* vp = v_pool + (row0 + vr) * 256 + vg * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) c.k[i] = ldg128(kp + 16 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) c.v[i] = ldg128(vp + 16 * i);
  } else if constexpr (KV == 1) {
    const uint8_t* kp = k_pool + (row0 + kr) * 128 + kg * 32;
    const uint8_t* vp = v_pool + (row0 + vr) * 128 + vg * 32;
    c.k[0] = ldg128(kp);
    c.k[1] = ldg128(kp + 16);
    c.v[0] = ldg128(vp);
    c.v[1] = ldg128(vp + 16);
    c.kscale = *reinterpret_cast<const f32x4*>(static_cast<const float*>(k_scale) + row0 + 4 * kg);
    c.vscale = *reinterpret_cast<const f32x4*>(static_cast<const float*>(v_scale) + row0 + 4 * kg);
  } else {
    c.k[0] = ldg128(k_pool + (row0 + kr) * 64 + kg * 16);
    c.v[0] = ldg128(v_pool + (row0 + vr) * 64 + vg * 16);
    c.ks = *reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(k_scale) +
                                              (row0 + kr) * 8 + kg * 2);
    c.vs = *reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(v_scale) +
                                              (row0 + vr) * 8 + vg * 2);
  }
}

// Four packed bf16 pairs from 8 e2m1 codes (one dword) with scale `s`.
__device__ __forceinline__ void e2m1x8_to_bf16(uint32_t w, float s, uint32_t* out) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const f32x2 v = e2m1x2_to_f32x2(w, b);
    out[b] = pack_bf16_trunc(v.x * s, v.y * s);
  }
}

// A operand (16 keys x 8 dims) of K-step kk for this lane, as bf16.
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

// This lane's 32 V values of its key row, as 16 packed bf16 dwords.
template <int KV>
__device__ __forceinline__ void v_bf16(const Chunk<KV>& c, uint32_t* o) {
  if constexpr (KV == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[4 * i] = c.v[i].x; o[4 * i + 1] = c.v[i].y; o[4 * i + 2] = c.v[i].z; o[4 * i + 3] = c.v[i].w;
    }
  } else if constexpr (KV == 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t src[4] = {c.v[i].x, c.v[i].y, c.v[i].z, c.v[i].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        o[8 * i + 2 * w] = e4m3x2_to_bf16x2<false>(src[w]);
        o[8 * i + 2 * w + 1] = e4m3x2_to_bf16x2<true>(src[w]);
      }
    }
  } else {
    const uint32_t src[4] = {c.v[0].x, c.v[0].y, c.v[0].z, c.v[0].w};
    const float s0 = e4m3_to_f32(c.vs & 0xFFu);
    const float s1 = e4m3_to_f32((c.vs >> 8) & 0xFFu);
#pragma unroll
    for (int w = 0; w < 4; ++w) e2m1x8_to_bf16(src[w], w < 2 ? s0 : s1, o + 4 * w);
  }
}

template <int KV>
__global__ __launch_bounds__(256, 2) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ k_pool,
    const uint8_t* __restrict__ v_pool, const void* __restrict__ k_scale,
    const void* __restrict__ v_scale, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ ctx_lens, float* __restrict__ part_o,
    float* __restrict__ part_ml, float* __restrict__ out, int T, int Hq, int Hkv, int PT,
    int S, int cpw, float scale_log2) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * kStage];

  const int lane = lane_id();
  const int wave = wave_id();
  const int wid = blockIdx.x;
  const int split = wid % S;
  const int rg = wid / S;
  const int g = rg % Hkv;
  const int r = rg / Hkv;
  const int b = r / T;
  const int t = r - b * T;
  const int G = Hq / Hkv;
  const int pos = ctx_lens[b] - T + t;

  // valid pages of the row (the table is -1 padded at the end)
  const int32_t* prow = page_table + (size_t)r * PT;
  int nvp = __popcll(__ballot(lane < PT && prow[lane] >= 0));
  if (PT > kWave) nvp += __popcll(__ballot(lane + kWave < PT && prow[lane + kWave] >= 0));
  const int nblk = nvp >> 3;
  const int kv_len = nblk > 0 ? 128 * (nblk - 1) + (pos & 127) + 1 : 0;

  // Q^T operand: lane holds head (lane & 15) of the group, dims 32*(lane>>4)..+32
  const int hl = lane & 15;
  const int g4 = lane >> 4;
  bf16x8 qop[4];
  {
    u32x4 z = {0u, 0u, 0u, 0u};
    const uint16_t* qp = q + ((size_t)r * Hq + g * G + min(hl, G - 1)) * kD + 32 * g4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 v = ldg128(qp + 8 * kk);
      qop[kk] = __builtin_bit_cast(bf16x8, hl < G ? v : z);
    }
  }

  float m = neg_inf(), lsum = 0.f;
  f32x4 oacc[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) oacc[s] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint8_t* stage = smem + wave * kStage;
  const size_t kv_head_rows = 128;
  for (int k = 0; k < cpw; ++k) {
    const int ci = split * 4 * cpw + wave + 4 * k;
    if (ci * kChunk >= kv_len) break;
    Chunk<KV> ch[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int P = __builtin_amdgcn_readfirstlane(prow[2 * ci + j]);
      const size_t row0 = ((size_t)(P >> 3) * Hkv + g) * kv_head_rows + (size_t)(P & 7) * 16;
      load_page<KV>(ch[j], k_pool, v_pool, k_scale, v_scale, row0, lane);
    }
    // stage V rows into LDS: lane writes 64 B of key row 16*j + lane/4
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t vb[16];
      v_bf16<KV>(ch[j], vb);
      uint8_t* dst = stage + (16 * j + (lane >> 2)) * kVRow + (lane & 3) * 64;
#pragma unroll
      for (int w = 0; w < 8; ++w)
        *reinterpret_cast<uint2*>(dst + 8 * w) = make_uint2(vb[2 * w], vb[2 * w + 1]);
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
    // online softmax over this chunk (log2 domain)
    float z[8];
    float mc = neg_inf();
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = sacc[j][i] * scale_log2;
        if constexpr (KV == 1) v *= ch[j].kscale[i];
        const int n = ci * kChunk + 16 * j + 4 * g4 + i;
        v = n < kv_len ? v : neg_inf();
        z[4 * j + i] = v;
        mc = fmaxf(mc, v);
      }
    mc = fmaxf(mc, __shfl_xor(mc, 16));
    mc = fmaxf(mc, __shfl_xor(mc, 32));
    const float mn = fmaxf(m, mc);
    const float alpha = mn == m ? 1.f : __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    float psum = 0.f;
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = z[e] == neg_inf() ? 0.f : __builtin_amdgcn_exp2f(z[e] - mn);
      psum += p;
      float pv = p;
      if constexpr (KV == 1) pv *= ch[e >> 2].vscale[e & 3];
      hi[e] = bf16_rne_bits(pv);
      lo[e] = bf16_rne_bits(pv - bf16_bits_to_f32(hi[e]));
    }
    lsum = lsum * alpha + psum;
    u32x4 bh, bl;
    bh.x = hi[0] | (hi[1] << 16); bh.y = hi[2] | (hi[3] << 16);
    bh.z = hi[4] | (hi[5] << 16); bh.w = hi[6] | (hi[7] << 16);
    bl.x = lo[0] | (lo[1] << 16); bl.y = lo[2] | (lo[3] << 16);
    bl.z = lo[4] | (lo[5] << 16); bl.w = lo[6] | (lo[7] << 16);
    const bf16x8 phi = __builtin_bit_cast(bf16x8, bh);
    const bf16x8 plo = __builtin_bit_cast(bf16x8, bl);
#pragma unroll
    for (int s = 0; s < 8; ++s) oacc[s] *= alpha;

    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // O^T += V^T P^T, dims in blocks of 16
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint8_t* col = stage + (16 * s + hl) * 2;
      uint32_t a[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x0 = *reinterpret_cast<const uint16_t*>(col + kappa(g4, 2 * w) * kVRow);
        const uint32_t x1 = *reinterpret_cast<const uint16_t*>(col + kappa(g4, 2 * w + 1) * kVRow);
        a[w] = x0 | (x1 << 16);
      }
      const u32x4 av = {a[0], a[1], a[2], a[3]};
      const bf16x8 aop = __builtin_bit_cast(bf16x8, av);
      oacc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, phi, oacc[s], 0, 0, 0);
      oacc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, plo, oacc[s], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);

  // combine the four waves in LDS
  __syncthreads();
  float* m_w = reinterpret_cast<float*>(smem);  // [4][16]
  float* l_w = m_w + 64;                        // [4][16]
  float* o_w = l_w + 64;                        // [4][16][kORow]
  if (lane < 16) {
    m_w[wave * 16 + lane] = m;
    l_w[wave * 16 + lane] = lsum;
  }
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) o_w[(wave * 16 + hl) * kORow + 16 * s + 4 * g4 + i] = oacc[s][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * kD; idx += 256) {
    const int h = idx >> 7;
    const int d = idx & (kD - 1);
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, m_w[w * 16 + h]);
    float O = 0.f, Ls = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = m_w[w * 16 + h];
      const float f = mw == neg_inf() ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      O += f * o_w[(w * 16 + h) * kORow + d];
      Ls += f * l_w[w * 16 + h];
    }
    const size_t rh = (size_t)r * Hq + g * G + h;
    if (S == 1) {
      out[rh * kD + d] = Ls > 0.f ? O / Ls : 0.f;
    } else {
      part_o[(rh * S + split) * kD + d] = O;
      if (d == 0) {
        part_ml[(rh * S + split) * 2] = M;
        part_ml[(rh * S + split) * 2 + 1] = Ls;
      }
    }
  }
}

// out[rh][d] = sum_s 2^(m_s - M) O_s[d] / sum_s 2^(m_s - M) l_s
__global__ __launch_bounds__(128) void lse_merge_kernel(const float* __restrict__ part_o,
                                                        const float* __restrict__ part_ml,
                                                        float* __restrict__ out, int S) {
  const size_t rh = blockIdx.x;
  const int d = threadIdx.x;
  const float* ml = part_ml + rh * S * 2;
  float M = neg_inf();
  for (int s = 0; s < S; ++s) M = fmaxf(M, ml[2 * s]);
  float O = 0.f, Ls = 0.f;
  for (int s = 0; s < S; ++s) {
    const float ms = ml[2 * s];
    const float f = ms == neg_inf() ? 0.f : __builtin_amdgcn_exp2f(ms - M);
    O += f * part_o[(rh * S + s) * kD + d];
    Ls += f * ml[2 * s + 1];
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
  } else if (i < 256 + 32 + 256) {
    out[i] = e4m3_to_f32((uint32_t)(i - 288));
  }
}

template <int KV>
hipError_t launch_kv(const Dims& d, const SplitPlan& sp, const void* q, const void* k_pool,
                     const void* v_pool, const void* k_scale, const void* v_scale,
                     const int32_t* page_table, const int32_t* ctx_lens, float* part_o,
                     float* part_ml, float* out, hipStream_t s) {
  const long wgs = (long)d.R() * d.Hkv * sp.splits;
  hipLaunchKernelGGL((sparse_attn_kernel<KV>), dim3((unsigned)wgs), dim3(256), 0, s,
                     static_cast<const uint16_t*>(q), static_cast<const uint8_t*>(k_pool),
                     static_cast<const uint8_t*>(v_pool), k_scale, v_scale, page_table,
                     ctx_lens, part_o, part_ml, out, d.T, d.Hq, d.Hkv, d.PT(), sp.splits,
                     sp.cpw, d.scale_log2);
  return hipGetLastError();
}

}  // namespace

SplitPlan plan_splits(const Dims& d) {
  // Aim at ~4096 waves (16 per CU) while keeping split partials small.
  const int chunks = d.PT() / 2;
  const long pairs = (long)d.R() * d.Hkv;
  int cpw = 1;
  while (cpw < chunks / 4 && pairs * 4 * ((chunks + 4 * cpw - 1) / (4 * cpw)) > 4096) cpw *= 2;
  SplitPlan p;
  p.cpw = cpw;
  p.splits = (chunks + 4 * cpw - 1) / (4 * cpw);
  return p;
}

hipError_t launch_sparse_attention(const Dims& d, const void* q, const void* k_pool,
                                   const void* v_pool, const void* k_scale,
                                   const void* v_scale, const int32_t* page_table,
                                   const int32_t* ctx_lens, float* part_o, float* part_ml,
                                   float* out, hipStream_t s, std::string* note) {
  const SplitPlan sp = plan_splits(d);
  hipError_t e;
  if (d.kv_dtype == 0)
    e = launch_kv<0>(d, sp, q, k_pool, v_pool, k_scale, v_scale, page_table, ctx_lens, part_o,
                     part_ml, out, s);
  else if (d.kv_dtype == 1)
    e = launch_kv<1>(d, sp, q, k_pool, v_pool, k_scale, v_scale, page_table, ctx_lens, part_o,
                     part_ml, out, s);
  else
    e = launch_kv<2>(d, sp, q, k_pool, v_pool, k_scale, v_scale, page_table, ctx_lens, part_o,
                     part_ml, out, s);
  if (e != hipSuccess) return e;
  static const char* names[3] = {"bf16", "fp8", "nvfp4"};
  if (note)
    *note += std::string("sparse_attn<") + names[d.kv_dtype] + ">[grid=" +
             std::to_string((long)d.R() * d.Hkv * sp.splits) + "x256,splits=" +
             std::to_string(sp.splits) + ",chunks_per_wave=" + std::to_string(sp.cpw) + "]";
  if (sp.splits > 1) {
    const unsigned rows = (unsigned)((long)d.R() * d.Hq);
    hipLaunchKernelGGL(lse_merge_kernel, dim3(rows), dim3(kD), 0, s, part_o, part_ml, out,
                       sp.splits);
    if (note) *note += " lse_merge[grid=" + std::to_string(rows) + "x128]";
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_selftest_decoders(float* out, hipStream_t s) {
  hipLaunchKernelGGL(selftest_kernel, dim3(3), dim3(256), 0, s, out);
  return hipGetLastError();
}

}  // namespace msa
