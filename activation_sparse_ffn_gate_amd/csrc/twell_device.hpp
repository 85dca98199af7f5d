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

#include <type_traits>

namespace twell {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
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

// ------------------------------------------------------------------ lane helpers
// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, class Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Write the wave-uniform value `val` into lane LANE of `dst` (v_writelane_b32).
template <int LANE>
__device__ __forceinline__ int writelane(int dst, int val) {
  static_assert(LANE >= 0 && LANE < 64, "lane");
  asm("v_writelane_b32 %0, %1, %2" : "+v"(dst) : "s"(val), "i"(LANE));
  return dst;
}

// Number of set bits of the 64-bit wave mask `m` in lanes below this lane.
__device__ __forceinline__ uint32_t mask_rank(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

// Stores through a wave-uniform base pointer and a 32-bit byte offset, so the
// address needs no 64-bit vector arithmetic.
template <class T>
__device__ __forceinline__ void store_at(T* base, uint32_t byte_off, T v) {
  *reinterpret_cast<T*>(reinterpret_cast<char*>(base) + byte_off) = v;
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

// Value held by lane (this lane ^ X), X in 1..16 (ds_swizzle bit mode, which
// permutes within each 32 lanes).
template <int X>
__device__ __forceinline__ float xor_lanes(float v) {
  static_assert(X >= 1 && X <= 16, "xor within 32 lanes");
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (X << 10) | 0x1F));
}

// v[l] + v[l ^ 32] on every lane l (v_permlane32_swap exchanges the two
// halves); both lanes of a pair add the same operands in the same order.
__device__ __forceinline__ float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
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
// A K-chunk of 32 bf16 per row is 64 bytes = four 16-byte pieces. An MFMA
// fragment load reads one piece of 32 consecutive rows (ds_read_b128); the LDS
// serves such a read 16 lanes (rows) at a time from 64 four-byte banks, i.e.
// 256 bytes = four 64-byte rows per bank sweep. Piece c of row r is stored at
// piece c ^ swz(r), swz(r) = ((r >> 1) ^ (r >> 3)) & 3: among any 16
// consecutive rows the four rows sharing r % 4 get four different pieces, so
// the 16 reads hit 16 different 16-byte bank groups (and any 8 consecutive
// rows also spread over a 128-byte sweep).
__device__ __forceinline__ constexpr int lds_swz(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

__device__ __forceinline__ uint32_t lds_off(int row, int piece) {
  return static_cast<uint32_t>(row * 64 + ((piece ^ lds_swz(row)) << 4));
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

// 16-byte store with the non-temporal hint, for output written once and not
// read again by the launch: it keeps L2 for the data the launch reuses.
__device__ __forceinline__ void store16_nt(float* p, float a, float b, float c, float d) {
  const f32x4_t v = {a, b, c, d};
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p));
}

// ------------------------------------------------------------------ LDS DMA
// gfx950 global_load_lds_dwordx4: every lane fetches 16 bytes from its own
// global address; the wave writes them to 1024 contiguous LDS bytes at
// `lds_block` (wave-uniform), lane l at byte 16 * l. Counted by vmcnt.
__device__ __forceinline__ void dma16(const uint16_t* g, uint8_t* lds_block) {
  __builtin_amdgcn_global_load_lds(g, lds_block, 16, 0, 0);
}

// s_waitcnt with vmcnt = VM (0..63) and lgkmcnt = LGKM (0..15), expcnt free.
template <int VM, int LGKM>
__device__ __forceinline__ void waitcnt() {
  static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "waitcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LGKM << 8));
}

// Workgroup barrier without the memory fence __syncthreads() implies (that
// fence waits for every outstanding load, which would drain the DMA pipeline).
// Callers wait for their own loads with waitcnt<> first; the empty asm
// statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace twell
