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
#include <algorithm>
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

// Few tokens: one workgroup of kWideWaves waves per token, so a token's units
// are not walked by a single wave in a chain of dependent load rounds. The
// waves build the token's (unit, value) list together, then
//   up:   wave w takes list entries in chunks of UP (chunk c goes to wave
//         c mod kWideWaves), computes u_j exactly as above (same lane layout of
//         x, same reduction) and leaves h_j = g_j * u_j in the list;
//   down: wave w, lane l owns the 4-column groups q = 64 w + l (+ 64 kWideWaves
//         i); every wave walks the whole list in order, DN units' Wd loads in
//         flight at a time (kShortDn for a round of a few-token row), and adds
//         h_j * Wd[j] to its columns.
// A wave reads a round's entries with one LDS load, lane u holding entry u,
// and takes each unit's index and value from lane u with v_readlane.
// Every product and every per-column sum is taken in the same order as in the
// one-wave form, so both forms give the same bits.
constexpr int kWideWaves = 8;
constexpr int kWideCap = 1024;  // list entries per round
constexpr int kSplitMinEntries = 384;  // longer rows may be cut into parts
constexpr int kSplitChunk = 192;       // entries per part at least
constexpr int kShortDn = 16;           // down-pass step of short rounds

// Down product over list entries lo .. n - 1 of a round (wide kernel): S
// entries' Wd loads issued at a time, each lane adding h_j Wd[j] into its NQ
// 4-column groups in list order.
template <int S, int NQ>
__device__ __forceinline__ void wide_down(float (&acc)[NQ][4], const int* s_j, const float* s_h, int lo, int n,
                                          const char* wdb, uint32_t row_bytes, int quads, int w, int lane) {
  for (int e0 = lo; e0 < n; e0 += S) {
    const int jv = s_j[min(e0 + min(lane, S - 1), n - 1)];
    const float hv = s_h[min(e0 + min(lane, S - 1), n - 1)];
    u32x2_t wd[S][NQ];
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const size_t rb = static_cast<size_t>(__builtin_amdgcn_readlane(jv, u)) * row_bytes;
#pragma unroll
      for (int i = 0; i < NQ; ++i) {  // unconditional (column clamped): keeps the waits counted
        const int q = min((i * kWideWaves + w) * 64 + lane, quads - 1);
        wd[u][i] = *reinterpret_cast<const u32x2_t*>(wdb + rb + static_cast<uint32_t>(q) * 8u);
      }
    }
#pragma unroll
    for (int u = 0; u < S; ++u) {
      if (e0 + u < n) {  // uniform
        const float h = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hv), u));
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          if ((i * kWideWaves + w) * 64 < quads) {  // uniform
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              acc[i][2 * q] = fmaf(h, bf16_lo(wd[u][i][q]), acc[i][2 * q]);
              acc[i][2 * q + 1] = fmaf(h, bf16_hi(wd[u][i][q]), acc[i][2 * q + 1]);
            }
          }
        }
      }
    }
  }
}

template <int VEC, int NCH, int UP, int NQ, int DN>
__global__ __launch_bounds__(64 * kWideWaves) void fused_updown_wide_kernel(FusedArgs a) {
  using LoadT = typename Vec<VEC>::T;
  constexpr int kW = Vec<VEC>::kWords;
  constexpr int kChunk = 64 * VEC;

  __shared__ int s_j[kWideCap];
  __shared__ float s_h[kWideCap];  // gate value, then h

  __shared__ int s_last;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // splits > 1: workgroup k M + row takes part k of a long row (the first M
  // workgroups are the whole of every short row).
  const int row = blockIdx.x % a.M;
  const int part_k = blockIdx.x / a.M;

  const int nT = a.F / a.T;
  const int C = a.C;
  const uint16_t* cnt_row = a.counts + static_cast<size_t>(row) * nT;

  // Every wave reads the counts, so all of them take the same decision. An
  // overflow row is left to the dense fallback, unless its overflowing tiles
  // were spilled: then their units are read from the spilled z.
  bool over = false;
  int row_total = 0;
  for (int t = lane; t < nT; t += 64) {
    const int c = cnt_row[t];
    over |= c > C;
    row_total += c;
  }
  if (__ballot(over) != 0 && a.spill == nullptr) return;
  // A long row is cut into P contiguous runs of its ascending unit list, run k
  // done by part k; each part's y row goes to a partial buffer and the last
  // part to finish adds them in part order.
  row_total = __builtin_amdgcn_readlane(wave_inclusive_scan(row_total), 63);
  const int P = (a.splits > 1 && row_total > kSplitMinEntries)
                    ? min(a.splits, (row_total + kSplitChunk - 1) / kSplitChunk)
                    : 1;
  if (part_k >= P) return;
  const int e_lo = static_cast<int>(static_cast<int64_t>(part_k) * row_total / P);
  const int e_hi = static_cast<int>(static_cast<int64_t>(part_k + 1) * row_total / P);

  LoadT xv[NCH];
  const uint16_t* xr = a.x + static_cast<size_t>(row) * a.d + lane * VEC;
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) xv[ch] = *reinterpret_cast<const LoadT*>(xr + ch * kChunk);

  const int quads = a.d / 4;  // multiple of 64: the guard below is wave-uniform
  float acc[NQ][4];
#pragma unroll
  for (int i = 0; i < NQ; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[i][k] = 0.f;

  const int tmask = a.T - 1;
  const uint32_t row_bytes = static_cast<uint32_t>(a.d) * 2u;
  const char* wdb = reinterpret_cast<const char*>(a.Wd);

  int gbase = 0;  // entries of the row before this tile group
  for (int t0 = 0; t0 < nT; t0 += 64) {
    const int t = t0 + lane;
    const int c = (t < nT) ? static_cast<int>(cnt_row[t]) : 0;
    const int incl = wave_inclusive_scan(c);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    const int off = incl - c;
    const size_t slot0 = (static_cast<size_t>(row) * nT + t) * C;
    if (gbase + total <= e_lo || gbase >= e_hi) {  // no entry of this part here (uniform)
      gbase += total;
      continue;
    }
    for (int base = 0; base < total; base += kWideCap) {
      // Fill: lane t of wave w copies slots s = s_lo + w, s_lo + w + kWideWaves, ...
      const int s_lo = max(0, base - off);
      const int s_hi = min(c, base + kWideCap - off);
      if (c <= C) {
        for (int s = s_lo + w; s < s_hi; s += kWideWaves) {
          s_j[off + s - base] = t * a.T + (static_cast<int>(a.idx[slot0 + s]) & tmask);
          s_h[off + s - base] = a.vals[slot0 + s];
        }
      }
      // Spilled tiles (count > C; only when a spill is given): the i-th one of
      // this group goes to wave i mod kWideWaves, which reads its T z values
      // 64 at a time; a ballot ranks the active units in ascending order and
      // the s-th one goes to slot s.
      uint64_t spilled = __ballot(t < nT && c > C);
      for (int i = 0; spilled != 0; ++i, spilled &= spilled - 1) {
        if (i % kWideWaves != w) continue;  // uniform
        const int tl = __builtin_ctzll(spilled);
        const int ct = __builtin_amdgcn_readlane(c, tl), ot = __builtin_amdgcn_readlane(off, tl);
        const int lo_t = max(0, base - ot), hi_t = min(ct, base + kWideCap - ot);
        if (lo_t >= hi_t) continue;
        const int tt = t0 + tl;
        const float* seg = a.spill + (static_cast<size_t>(row) * nT + tt) * a.T;
        int k = 0;
        for (int u0 = 0; u0 < a.T; u0 += 64) {  // T is 64 or 128
          const float z = seg[u0 + lane];
          const uint64_t b = __ballot(z > 0.f);
          const int sl = k + static_cast<int>(mask_rank(b));
          if (z > 0.f && sl >= lo_t && sl < hi_t) {
            s_j[ot + sl - base] = tt * a.T + u0 + lane;
            s_h[ot + sl - base] = z;
          }
          k += __popcll(b);
        }
      }
      __syncthreads();
      // this round's entries that belong to this part: [lo, n)
      const int lo = max(0, e_lo - gbase - base);
      const int n = min(min(kWideCap, total - base), e_hi - gbase - base);

      // Up: chunks of UP entries round-robin over the waves.
      for (int e0 = lo + w * UP; e0 < n; e0 += kWideWaves * UP) {
        // lane u holds entry e0 + u (the last entry for lanes past the list)
        const int jv = s_j[min(e0 + min(lane, UP - 1), n - 1)];
        const float gv = s_h[min(e0 + min(lane, UP - 1), n - 1)];
        LoadT wu[UP][NCH];
#pragma unroll
        for (int u = 0; u < UP; ++u) {
          const int ju = __builtin_amdgcn_readlane(jv, u);
          const uint16_t* pu = a.WuT + static_cast<size_t>(ju) * a.d + lane * VEC;
#pragma unroll
          for (int ch = 0; ch < NCH; ++ch) wu[u][ch] = *reinterpret_cast<const LoadT*>(pu + ch * kChunk);
        }
#pragma unroll
        for (int u = 0; u < UP; ++u) {
          float part = 0.f;
#pragma unroll
          for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
            for (int q = 0; q < kW; ++q) part = dot2_bf16(xv[ch][q], wu[u][ch][q], part);
          const float h = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), u)) * wave_sum(part);
          if (e0 + u < n && lane == 0) s_h[e0 + u] = h;
        }
      }
      __syncthreads();

      // Down: the whole list in order, DN entries' loads at a time, or
      // kShortDn for a round of at most 4 kShortDn entries (a few-token row),
      // whose loads past the list would otherwise outnumber its own.
      if (DN > kShortDn && n - lo <= 4 * kShortDn)  // uniform
        wide_down<(DN > kShortDn ? kShortDn : DN), NQ>(acc, s_j, s_h, lo, n, wdb, row_bytes, quads, w, lane);
      else
        wide_down<DN, NQ>(acc, s_j, s_h, lo, n, wdb, row_bytes, quads, w, lane);
      __syncthreads();  // the list is refilled next round
    }
    gbase += total;
  }

  float* yr = a.y + static_cast<size_t>(row) * a.d;
  if (P == 1) {
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int q = (i * kWideWaves + w) * 64 + lane;
      if (q < quads) *reinterpret_cast<float4*>(yr + 4 * q) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
    }
    return;
  }
  // Partial y row of this part; the last part to arrive (a per-row counter,
  // reset by it) adds parts 0 .. P-1 in order.
  float* prow = a.part + (static_cast<size_t>(part_k) * a.M + row) * a.d;
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int q = (i * kWideWaves + w) * 64 + lane;
    if (q < quads) *reinterpret_cast<float4*>(prow + 4 * q) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
  }
  __threadfence();  // release this part
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t done = atomicAdd(&a.counters[row], 1u);
    s_last = done == static_cast<uint32_t>(P - 1);
    if (s_last) __hip_atomic_store(&a.counters[row], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();  // acquire the other parts
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int q = (i * kWideWaves + w) * 64 + lane;
    if (q < quads) {
      float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int k = 0; k < P; ++k) {
        const float4 v = reinterpret_cast<const float4*>(a.part + (static_cast<size_t>(k) * a.M + row) * a.d)[q];
        sum.x += v.x;
        sum.y += v.y;
        sum.z += v.z;
        sum.w += v.w;
      }
      *reinterpret_cast<float4*>(yr + 4 * q) = sum;
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
  if (a.M <= kFewRows) {
    // d = 64 * VEC * NCH; NQ 4-column groups per lane cover it with 8 waves
    constexpr int kD = 64 * VEC * NCH;
    constexpr int kNQ = (kD / 4 + 64 * kWideWaves - 1) / (64 * kWideWaves);
    // entries per up round per wave / per down round: as deep as registers allow
    constexpr int kUp = NCH <= 2 ? 8 : (NCH <= 4 ? 4 : (NCH <= 8 ? 2 : 1));
    constexpr int kDn = kNQ == 1 ? 64 : (kNQ == 2 ? 24 : 8);
    fused_updown_wide_kernel<VEC, NCH, kUp, kNQ, kDn>
        <<<dim3(a.M * std::max(a.splits, 1)), dim3(64 * kWideWaves), 0, s>>>(a);
    return hipGetLastError();
  }
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
