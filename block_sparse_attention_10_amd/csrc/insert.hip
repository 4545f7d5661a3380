// The write path: each new token's K, V and index key go into the pools,
// quantised to the pools' formats.
//
// news.ainew.jp MI355X article, section 3: the fused projection writes the
// index cache of each new token; aisoku.org MiniMax-M3.1-Flash article,
// section "何が新しいか": the KV cache is stored as fp8 or NVFP4.  Row r =
// b T + t is the token at position p = ctx_lens[b] - T + t: it lands in slot
// p mod 128 of physical block block_table[b][p / 128], so the attention of
// the same step already sees it.
//
// Formats (the pools' layouts are the attention's):
//  * fp8 K / V: per (token, head) scale = amax / 448 (1 when amax is 0),
//    codes = E4M3 round-to-nearest-even of x / scale, clamped to +-448;
//  * 4-bit K / V / index keys: per 16 elements s = E4M3 of amax / 6, codes =
//    E2M1 round-to-nearest-even of x / s (saturating at 6), zero codes when
//    s is 0; a negative value that rounds to 0 is stored as +0;
//  * fp8 index keys: the E4M3 code of the value itself.
// Every decision runs in fp32 (IEEE division) and the codes come from the
// gfx950 conversion instructions (v_cvt_scalef32_pk_fp8_f32 /
// v_cvt_scalef32_pk_fp4_f32 at scale 1, round-to-nearest-even).
//
// Design: one wave per (row, tensor, head): a K or V row of 128 values is
// one dword (two bf16) per lane, an index row of 64 values one bf16 per
// lane; row and group maxima are lane shuffles.  The kernel is tiny and
// latency-bound (a decode step writes R rows).
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {
namespace {

typedef short v2i16 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;      // head dim
constexpr int kIdxDim = 64;  // index head dim

// E4M3 codes of two fp32 values (|x| <= 448) in the low 16 bits.
__device__ __forceinline__ uint32_t f32x2_to_e4m3x2(float a, float b) {
  const v2i16 old = {0, 0};
  const v2i16 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(old, a, b, 1.0f, false);
  return (uint32_t)(uint16_t)r.x;
}

// E2M1 codes of two fp32 values (element a in the low nibble), -0 as +0.
__device__ __forceinline__ uint32_t f32x2_to_e2m1x2(float a, float b) {
  uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0) & 0xFFu;
  if ((c & 0x7u) == 0) c &= 0xF0u;
  if ((c & 0x70u) == 0) c &= 0x0Fu;
  return c;
}

// Max over the aligned group of N lanes (N a power of two <= 64).
template <int N>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = 1; m < N; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

// E4M3 scale code for a group of 4-bit codes: amax / 6, saturating.
__device__ __forceinline__ uint32_t fp4_scale_code(float amax) {
  return f32x2_to_e4m3x2(fminf(amax / 6.0f, 448.0f), 0.0f) & 0xFFu;
}

// KV, IDX: 0 bf16, 1 fp8, 2 4-bit.
template <int KV, int IDX>
__global__ __launch_bounds__(256) void insert_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const uint16_t* __restrict__ idx_new, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ ctx_lens, uint8_t* __restrict__ k_pool,
    uint8_t* __restrict__ v_pool, uint8_t* __restrict__ k_scale, uint8_t* __restrict__ v_scale,
    uint8_t* __restrict__ idx_k, uint8_t* __restrict__ idx_ks, int R, int T, int Hkv, int Hidx,
    int MAXB, int max_block) {
  const int lane = lane_id();
  const int per = 2 * Hkv + Hidx;
  const long item = (long)blockIdx.x * 4 + wave_id();
  if (item >= (long)R * per) return;
  const int r = (int)(item / per);
  const int j = (int)(item - (long)r * per);
  const int b = r / T;
  const int pos = ctx_lens[b] - T + (r - b * T);
  // a bad context length or table entry cannot leave the table or the pools
  const int lb = min(max(pos >> 7, 0), MAXB - 1);
  const size_t phys = (size_t)min(max(block_table[(size_t)b * MAXB + lb], 0), max_block);
  const int slot = pos & 127;

  if (j < 2 * Hkv) {
    const bool is_v = j >= Hkv;
    const int g = is_v ? j - Hkv : j;
    const uint32_t pair = reinterpret_cast<const uint32_t*>(
        (is_v ? v_new : k_new) + ((size_t)r * Hkv + g) * kD)[lane];
    const float x0 = bf16_bits_to_f32(pair & 0xFFFFu);
    const float x1 = bf16_bits_to_f32(pair >> 16);
    const size_t row = (phys * Hkv + g) * 128 + slot;
    uint8_t* pool = is_v ? v_pool : k_pool;
    uint8_t* scale = is_v ? v_scale : k_scale;
    if constexpr (KV == 0) {
      reinterpret_cast<uint32_t*>(pool + row * 256)[lane] = pair;
    } else if constexpr (KV == 1) {
      const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
      const float s = amax > 0.f ? amax / 448.0f : 1.0f;
      const float y0 = fminf(fmaxf(x0 / s, -448.f), 448.f);
      const float y1 = fminf(fmaxf(x1 / s, -448.f), 448.f);
      reinterpret_cast<uint16_t*>(pool + row * 128)[lane] = (uint16_t)f32x2_to_e4m3x2(y0, y1);
      if (lane == 0) reinterpret_cast<float*>(scale)[row] = s;
    } else {
      // 16 values per scale: 8 lanes
      const uint32_t sc = fp4_scale_code(group_max<8>(fmaxf(fabsf(x0), fabsf(x1))));
      const float s = e4m3_to_f32(sc);
      const uint32_t codes = s > 0.f ? f32x2_to_e2m1x2(x0 / s, x1 / s) : 0u;
      pool[row * 64 + lane] = (uint8_t)codes;
      if ((lane & 7) == 0) scale[row * 8 + (lane >> 3)] = (uint8_t)sc;
    }
    return;
  }

  const int h = j - 2 * Hkv;
  const uint16_t bits = (idx_new + ((size_t)r * Hidx + h) * kIdxDim)[lane];
  const float x = bf16_bits_to_f32(bits);
  const size_t row = (phys * Hidx + h) * 128 + slot;
  if constexpr (IDX == 0) {
    reinterpret_cast<uint16_t*>(idx_k + row * 128)[lane] = bits;
  } else if constexpr (IDX == 1) {
    idx_k[row * 64 + lane] = (uint8_t)f32x2_to_e4m3x2(fminf(fmaxf(x, -448.f), 448.f), 0.f);
  } else {
    // 16 values per scale: 16 lanes; lane pairs share a byte
    const uint32_t sc = fp4_scale_code(group_max<16>(fabsf(x)));
    const float s = e4m3_to_f32(sc);
    const uint32_t c = s > 0.f ? (f32x2_to_e2m1x2(x / s, 0.f) & 0xFu) : 0u;
    const uint32_t hi = (uint32_t)__shfl_xor((int)c, 1);
    if ((lane & 1) == 0) idx_k[row * 32 + (lane >> 1)] = (uint8_t)(c | (hi << 4));
    if ((lane & 15) == 0) idx_ks[row * 4 + (lane >> 4)] = (uint8_t)sc;
  }
}

template <int KV, int IDX>
hipError_t launch_typed(const Dims& d, const void* k_new, const void* v_new,
                        const void* idx_new, const int32_t* bt, const int32_t* cl,
                        const InsertPools& pl, hipStream_t s, long waves) {
  hipLaunchKernelGGL((insert_kernel<KV, IDX>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                     s, static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                     static_cast<const uint16_t*>(idx_new), bt, cl,
                     static_cast<uint8_t*>(pl.k_pool), static_cast<uint8_t*>(pl.v_pool),
                     static_cast<uint8_t*>(pl.k_scale), static_cast<uint8_t*>(pl.v_scale),
                     static_cast<uint8_t*>(pl.idx_k_pool), static_cast<uint8_t*>(pl.idx_k_scale),
                     d.R(), d.T, d.Hkv, d.Hidx, d.MAXB, d.NB - 1);
  return hipGetLastError();
}

template <int KV>
hipError_t launch_kv_typed(const Dims& d, const void* k_new, const void* v_new,
                           const void* idx_new, const int32_t* bt, const int32_t* cl,
                           const InsertPools& pl, hipStream_t s, long waves) {
  if (d.idx_dtype == 0) return launch_typed<KV, 0>(d, k_new, v_new, idx_new, bt, cl, pl, s, waves);
  if (d.idx_dtype == 1) return launch_typed<KV, 1>(d, k_new, v_new, idx_new, bt, cl, pl, s, waves);
  return launch_typed<KV, 2>(d, k_new, v_new, idx_new, bt, cl, pl, s, waves);
}

}  // namespace

hipError_t launch_insert(const Dims& d, const void* k_new, const void* v_new,
                         const void* idx_new, const int32_t* block_table,
                         const int32_t* ctx_lens, const InsertPools& pools, hipStream_t s,
                         std::string* note) {
  const long waves = (long)d.R() * (2 * d.Hkv + d.Hidx);
  hipError_t e;
  if (d.kv_dtype == 0)
    e = launch_kv_typed<0>(d, k_new, v_new, idx_new, block_table, ctx_lens, pools, s, waves);
  else if (d.kv_dtype == 1)
    e = launch_kv_typed<1>(d, k_new, v_new, idx_new, block_table, ctx_lens, pools, s, waves);
  else
    e = launch_kv_typed<2>(d, k_new, v_new, idx_new, block_table, ctx_lens, pools, s, waves);
  static const char* names[3] = {"bf16", "fp8", "nvfp4"};
  if (note)
    *note += std::string("insert<") + names[d.kv_dtype] + "," + names[d.idx_dtype] + ">[grid=" +
             std::to_string((waves + 3) / 4) + "x256]";
  return e;
}

}  // namespace msa
