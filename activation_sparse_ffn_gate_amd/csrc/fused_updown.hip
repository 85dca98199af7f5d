// Fused up + down projection over a TwELL packing, for gfx950.
//
// The pages' inference kernel (Telegram post on TwELL at tgviewer.app, part
// "Инференс"; aimodeling.com summary, paragraph 3; Tencent Cloud article,
// section 2): walk the packed non-zeros, fetch only the Wu and Wd rows they
// need, form each unit's up-projection dot product and add its share of the
// down projection to the output, never materialising the hidden matrix.
//
// MI355X mapping. One wave per token. The token's x row sits in registers
// (d / 64 bf16 per lane) and its fp32 output row too. The wave first turns the
// token's per-tile counts, indices and values into a flat list of (unit, gate
// value) in LDS (a wave prefix sum over tiles gives each tile's offset), then
// walks the list a few units at a time:
//   u_j = x . WuT[j]   one coalesced 2d-byte row read, v_dot2_f32_bf16 per lane,
//                      DPP reduction across the wave
//   h_j = g_j * u_j    (scalar, fp32)
//   y  += h_j * Wd[j]  one coalesced 2d-byte row read, fp32 FMA per lane
// Several units are in flight per wave (their row loads are issued together)
// to keep enough bytes outstanding. Rows whose packing overflowed (some tile
// count > C) are skipped; the dense fallback writes them.
#include <type_traits>

#include "twell_device.hpp"
#include "twell_internal.hpp"

namespace twell {
namespace {

constexpr int kRowsPerWG = 4;  // one wave per token
constexpr int kListCap = 512;  // (unit, value) entries staged per wave per round

// VEC bf16 per lane per chunk (8: one 16-byte load, 4: one 8-byte load);
// NCH chunks cover d = 64 * VEC * NCH.
template <int VEC>
struct Vec;
template <>
struct Vec<8> {
  using T = u32x4_t;
  static constexpr int kWords = 4;
};
template <>
struct Vec<4> {
  using T = u32x2_t;
  static constexpr int kWords = 2;
};

template <int VEC, int NCH, int UNROLL>
__global__ __launch_bounds__(256) void fused_updown_kernel(FusedArgs a) {
  using LoadT = typename Vec<VEC>::T;
  constexpr int kW = Vec<VEC>::kWords;
  constexpr int kChunk = 64 * VEC;

  __shared__ int s_j[kRowsPerWG][kListCap];
  __shared__ float s_g[kRowsPerWG][kListCap];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int row = blockIdx.x * kRowsPerWG + w;
  if (row >= a.M) return;

  const int nT = a.F / a.T;
  const int C = a.C;
  const uint16_t* cnt_row = a.counts + static_cast<size_t>(row) * nT;

  bool over = false;
  for (int t = lane; t < nT; t += 64) over |= cnt_row[t] > C;
  if (__ballot(over) != 0) return;  // overflow row: owned by the dense fallback

  LoadT xv[NCH];
  const uint16_t* xr = a.x + static_cast<size_t>(row) * a.d + lane * VEC;
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) xv[ch] = *reinterpret_cast<const LoadT*>(xr + ch * kChunk);

  float acc[NCH][VEC];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
    for (int k = 0; k < VEC; ++k) acc[ch][k] = 0.f;

  const int tmask = a.T - 1;  // T is a power of two: keeps every unit index < F
  int* lj = s_j[w];
  float* lg = s_g[w];

  for (int t0 = 0; t0 < nT; t0 += 64) {
    const int t = t0 + lane;
    const int c = (t < nT) ? static_cast<int>(cnt_row[t]) : 0;
    const int incl = wave_inclusive_scan(c);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    const int off = incl - c;
    const size_t slot0 = (static_cast<size_t>(row) * nT + t) * C;
    for (int base = 0; base < total; base += kListCap) {
      const int s_lo = max(0, base - off);
      const int s_hi = min(c, base + kListCap - off);
      for (int s = s_lo; s < s_hi; ++s) {
        lj[off + s - base] = t * a.T + (static_cast<int>(a.idx[slot0 + s]) & tmask);
        lg[off + s - base] = a.vals[slot0 + s];
      }
      wave_lds_sync();
      const int n = min(kListCap, total - base);
      for (int e = 0; e < n; e += UNROLL) {
        int j[UNROLL];
        float g[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const int ee = min(e + u, n - 1);
          j[u] = __builtin_amdgcn_readfirstlane(lj[ee]);
          g[u] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(lg[ee])));
        }
        LoadT wu[UNROLL][NCH], wd[UNROLL][NCH];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const uint16_t* pu = a.WuT + static_cast<size_t>(j[u]) * a.d + lane * VEC;
          const uint16_t* pd = a.Wd + static_cast<size_t>(j[u]) * a.d + lane * VEC;
#pragma unroll
          for (int ch = 0; ch < NCH; ++ch) {
            wu[u][ch] = *reinterpret_cast<const LoadT*>(pu + ch * kChunk);
            wd[u][ch] = *reinterpret_cast<const LoadT*>(pd + ch * kChunk);
          }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          if (e + u < n) {  // uniform
            float part = 0.f;
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
              for (int q = 0; q < kW; ++q) part = dot2_bf16(xv[ch][q], wu[u][ch][q], part);
            const float h = g[u] * wave_sum(part);
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
              for (int q = 0; q < kW; ++q) {
                acc[ch][2 * q] = fmaf(h, bf16_lo(wd[u][ch][q]), acc[ch][2 * q]);
                acc[ch][2 * q + 1] = fmaf(h, bf16_hi(wd[u][ch][q]), acc[ch][2 * q + 1]);
              }
          }
        }
      }
      wave_lds_sync();
    }
  }

  float* yr = a.y + static_cast<size_t>(row) * a.d + lane * VEC;
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
    for (int k = 0; k < VEC; k += 4) {
      float4 v = make_float4(acc[ch][k], acc[ch][k + 1], acc[ch][k + 2], acc[ch][k + 3]);
      *reinterpret_cast<float4*>(yr + ch * kChunk + k) = v;
    }
  }
}

template <int NCH>
constexpr int unroll_for() {
#ifdef TWELL_FUSED_UNROLL
  return TWELL_FUSED_UNROLL;
#else
  return NCH <= 2 ? 8 : (NCH <= 5 ? 4 : (NCH <= 8 ? 2 : 1));
#endif
}

template <int VEC, int NCH>
hipError_t launch_vec(const FusedArgs& a, hipStream_t s) {
  const dim3 grid((a.M + kRowsPerWG - 1) / kRowsPerWG), block(64 * kRowsPerWG);
  fused_updown_kernel<VEC, NCH, unroll_for<NCH>()><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

template <int... N>
hipError_t dispatch8(int nch, const FusedArgs& a, hipStream_t s, std::integer_sequence<int, N...>) {
  hipError_t r = hipErrorInvalidValue;
  ((nch == N + 1 ? (r = launch_vec<8, N + 1>(a, s), 0) : 0), ...);
  return r;
}

template <int... N>
hipError_t dispatch4(int nch, const FusedArgs& a, hipStream_t s, std::integer_sequence<int, N...>) {
  hipError_t r = hipErrorInvalidValue;
  ((nch == 2 * N + 1 ? (r = launch_vec<4, 2 * N + 1>(a, s), 0) : 0), ...);
  return r;
}

}  // namespace

// d = 512 * n (n = 1..16) uses 16-byte lanes; other multiples of 256 up to
// 7936 use 8-byte lanes.
bool fused_supports_d(int d) {
  return d >= 256 && d <= 8192 && d % 256 == 0;
}

hipError_t launch_fused_updown(const FusedArgs& a, hipStream_t s) {
  if (a.d % 512 == 0) return dispatch8(a.d / 512, a, s, std::make_integer_sequence<int, 16>{});
  return dispatch4(a.d / 256, a, s, std::make_integer_sequence<int, 16>{});
}

}  // namespace twell
