// Device-side building blocks shared by the gfx950 kernels of libtwell.
//
// Wave64 everywhere. Matrix products use the CDNA4 instruction
// v_mfma_f32_32x32x16_bf16: per wave, A is 32x16 (rows x k), B is 16x32
// (k x cols), the accumulator is 32x32 fp32 held as 16 floats per lane.
//   operand lane layout: lane l holds row/col (l % 32) and the 8 consecutive
//   k values 8*(l / 32) .. 8*(l / 32) + 7 (A and B use the same k split, so
//   the product is the same whatever order the hardware walks k in);
//   accumulator: lane l holds column (l % 32); its element v (0..15) is row
//   8*(v / 4) + 4*(l / 32) + (v % 4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace twell {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ f32x16_t mfma_32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Row of the accumulator element v held by a lane in half `half` (= lane / 32).
__device__ __forceinline__ constexpr int acc_row(int v, int half) {
  return 8 * (v >> 2) + 4 * half + (v & 3);
}

// ------------------------------------------------------------------ bf16 <-> fp32
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two products of bf16 pairs accumulated in fp32 (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ------------------------------------------------------------------ wave collectives
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// Sum over the 64 lanes; every lane receives the total.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v);  // row_half_mirror: pairs the two quads of each 8 lanes
  v += dpp_f32<0x140>(v);  // row_mirror: pairs the two halves of each 16 lanes
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Inclusive prefix sum over the lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

// Orders this wave's LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ------------------------------------------------------------------ LDS tiles
// A K-chunk of 32 bf16 per row is 64 bytes = four 16-byte pieces. Piece c of
// row r is stored at piece (c ^ ((r >> 1) & 3)) so that the 32 rows read by an
// MFMA fragment load spread over all banks.
__device__ __forceinline__ uint32_t lds_off(int row, int piece) {
  return static_cast<uint32_t>(row * 64 + ((piece ^ ((row >> 1) & 3)) << 4));
}

__device__ __forceinline__ void lds_store16(uint8_t* base, uint32_t off, u32x4_t v) {
  *reinterpret_cast<u32x4_t*>(base + off) = v;
}

__device__ __forceinline__ u32x4_t lds_load16(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const u32x4_t*>(base + off);
}

// MFMA operand of a 32-row slab at k-step ks (0 or 1) of the 32-wide chunk.
__device__ __forceinline__ u32x4_t lds_frag(const uint8_t* tile, int row0, int ks, int lane) {
  return lds_load16(tile, lds_off(row0 + (lane & 31), ks * 2 + (lane >> 5)));
}

__device__ __forceinline__ u32x4_t gload16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

}  // namespace twell
