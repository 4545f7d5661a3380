// Device helpers for the gfx950 (CDNA4) MSA kernels: vector types, bf16 /
// fp8 / fp4 conversions, wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Wave index inside the workgroup, made provably uniform for the compiler.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

__device__ __forceinline__ u32x4 ldg128(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Streaming 16-byte load with the non-temporal hint: data read once (index
// keys, KV pages) should not displace reusable lines.  Measured on MI355X it
// also lifts a pure read stream from ~6.2 to ~6.9 TB/s.
__device__ __forceinline__ u32x4 ldg128_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// fp32 += a.x * b.x + a.y * b.y over packed bf16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// Two OCP E4M3 codes (16-bit half HI of `codes`) -> packed bf16 pair.
// Exact: every E4M3 value is a bf16 value.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t codes) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, HI));
}

// Two OCP E4M3 codes (low 16 bits of `codes`) -> fp32 pair, exact.
__device__ __forceinline__ f32x2 e4m3x2_to_f32x2(uint32_t codes) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(codes, 1.0f, false);
}

// One OCP E4M3 code (low byte of `code`) -> fp32.
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(code & 0xFFu, 1.0f, false);
  return v.x;
}

// Byte `sel` of `packed` holds two OCP E2M1 codes (element 2j in the low
// nibble, 2j+1 in the high nibble) -> the two values as fp32.
__device__ __forceinline__ f32x2 e2m1x2_to_f32x2(uint32_t packed, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 3);
  }
}

// Byte SEL of `packed` holds two OCP E2M1 codes (element 2j in the low
// nibble) -> the two values, unscaled, as a packed bf16 pair (exact).
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_to_bf16x2(uint32_t packed) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, 1.0f, SEL));
}

// Pack the upper halves of two fp32 values into a bf16 pair (truncation).
// Exact whenever the values carry at most 8 significant bits, as decoded
// fp8 codes and e2m1 x e4m3 products do.
__device__ __forceinline__ uint32_t pack_bf16_trunc(float lo, float hi) {
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hi),
                               __builtin_bit_cast(uint32_t, lo), 0x07060302u);
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __builtin_bit_cast(float, b << 16);
}

// `v` from lane l ^ MASK of the same wave, for MASK 1, 2 or 4, by DPP lane
// moves (no LDS round trip): quad permutes for 1 and 2; for 4 the lanes
// without bit 2 take row_shl:4, the others row_shr:4.
template <int MASK>
__device__ __forceinline__ float dpp_xor(float v) {
  const int x = __builtin_bit_cast(int, v);
  if constexpr (MASK == 1) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true));
  } else if constexpr (MASK == 2) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true));
  } else {
    static_assert(MASK == 4, "DPP xor for lane masks 1, 2 and 4");
    const int up = __builtin_amdgcn_mov_dpp(x, 0x104, 0xF, 0xF, true);    // lane + 4
    const int down = __builtin_amdgcn_mov_dpp(x, 0x114, 0xF, 0xF, true);  // lane - 4
    return __builtin_bit_cast(float, (lane_id() & 4) ? down : up);
  }
}

// One DPP step of a wave max; lanes outside `ROW_MASK` keep their value.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max_step(float v) {
  const int x = __builtin_bit_cast(int, v);
  return fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(x, x, CTRL, ROW_MASK,
                                                                        0xF, false)));
}

// Wave-wide max, returned to every lane: DPP within rows of 16 (quad swaps,
// half-row and row mirrors), row broadcasts across rows, then lane 63.
__device__ __forceinline__ float wave_max(float v) {
  v = dpp_max_step<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_max_step<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_max_step<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_max_step<0x140, 0xF>(v);  // row_mirror
  v = dpp_max_step<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_max_step<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

}  // namespace msa
