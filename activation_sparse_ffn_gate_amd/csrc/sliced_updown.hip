// Up + down projections over a TwELL packing, split by model-dimension slice
// so that every XCD's weight gathers stay in its own L2 (gfx950).
//
// What is computed is the fused kernel's operation (Telegram post on TwELL at
// tgviewer.app, part "Инференс"; aimodeling.com summary, paragraph 3): for
// each stored unit j of a row, u_j = x_r . WuT[j], h_j = g_j * u_j, and
// y_r = sum_j h_j * Wd[j]. The difference is where the bytes come from.
//
// MI355X has 8 XCDs, each with its own 4 MB L2, and workgroups are dispatched
// to the XCDs round-robin, so blockIdx % 8 names the XCD a workgroup runs on.
// The one-wave-per-token kernel gathers whole 2d-byte rows of WuT and Wd from
// every XCD, so the gathers miss L2 and run at the HBM/MALL rate. Here the d
// columns are cut into 8 slices and the workgroups of XCD k only touch slice k
// of WuT and Wd: F * (d / 8) * 2 bytes per matrix (4 MB at F = 8192,
// d = 2048), which that XCD's L2 can hold, so the repeated per-unit gathers
// become L2 hits.
//
// The price is one exchange between the slices, since u_j needs all d
// columns. Three launches:
//   lists: wave per row: the row's TwELL tiles become one contiguous list of
//         (unit j_e, gate value g_e) entries in (tile, slot) order, and its
//         length n (-1 for an overflow row). The packing is read once per row
//         here, not once per slice: a sparse row touches a cache line of
//         values in most of its tiles, so reading it in every slice's pass
//         was the largest share of the up pass's traffic.
//   up:   wave per (row, slice s): part[s][r][e] = g_e * (x_r[s] . WuT[j_e][s]);
//   down: wave per (row, slice s): h_e = sum over s' of part[s'][r][e] in the
//         fixed order s' = 0..7, y_r[s] = sum_e h_e * Wd[j_e][s].
// So a stored unit's hidden value does pass through memory: 8 fp32 partials per
// stored unit (the dense hidden matrix is still never formed). part is laid
// out [8][M][nT * C] so each row's partials of a slice are contiguous; the
// list is [M][nT * C] entries of 8 bytes. Every list and partial read starts
// at a fixed offset of its row, so a wave issues the row's length, its first
// 64 entries and its x slice together, and the weight gathers are its second
// round trip.
//
// Lane layout. A slice is d / 8 bf16 = d / 64 sixteen-byte pieces. A row of a
// slice is read by a group of L lanes (L = the largest power of two <= 64
// dividing d / 64), each lane holding V = (d / 64) / L pieces, so one load
// instruction of the wave reads G = 64 / L different stored units, each
// group's lanes covering 16 * L contiguous bytes. The up pass reduces within
// the group; the down pass keeps G partial output slices and sums them across
// groups once at the end. Overflow rows (some count > C) are skipped, as in the
// fused kernel; the dense fallback writes them.
#include "twell_device.hpp"
#include "twell_internal.hpp"

namespace twell {
namespace {

// One wave per (row, slice), one wave per workgroup (no wave of these kernels
// waits for another). Measured against 2, 4 and 8 waves a workgroup,
// single-wave workgroups were the fastest: 93 against 99 us for the pair at
// M = 4096, d = 2048, F = 8192, and 373 against 402 us at M = 16384,
// d = 2560, F = 10240.
constexpr int kRowsPerWG = 1;
constexpr int kListCap = 256;       // stored units staged per wave per round
constexpr int kListPad = 64;        // staged lists are padded (unit 0, value 0) to a whole step
constexpr int kCountGroups = 2;     // rows of up to 128 tiles keep their counts in registers

// 16 bytes at a 32-bit byte offset from a wave-uniform base (the weight
// matrices are below 2 GiB, checked by the host), so the address needs no
// 64-bit vector arithmetic.
__device__ __forceinline__ u32x4_t ldg16(const void* base, uint32_t off) {
  return *reinterpret_cast<const u32x4_t*>(static_cast<const char*>(base) + off);
}

// Sum over aligned groups of L lanes; every lane of a group gets the sum.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (L >= 2) v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  if constexpr (L >= 4) v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  if constexpr (L >= 8) v += dpp_f32<0x141>(v);  // row_half_mirror: other quad of the 8
  if constexpr (L >= 16) v += dpp_f32<0x140>(v); // row_mirror: other 8 of the 16
  if constexpr (L >= 32) v += xor_lanes<16>(v);
  if constexpr (L >= 64) v = sum_halves(v);
  return v;
}

// Stages the stored units of one row into LDS in (tile, slot) order, kListCap
// at a time, and runs body(n, e0) with units e0 .. e0 + n - 1 staged (unit
// index lj[i] and, if kWithValues, gate value lg[i]). Counts of the first
// 64 * kCountGroups tiles come in `c` (lane l: tile 64 q + l); the usual case,
// a row with at most that many tiles and kListCap units, is staged in one
// round. Returns the row's number of stored units.
template <bool kWithValues, class Body>
__device__ __forceinline__ int stage_row(const SlicedArgs& a, int row, const int (&c)[kCountGroups],
                                         int* lj, float* lg, Body&& body) {
  const int lane = threadIdx.x & 63;
  const int nT = a.F / a.T;
  const int C = a.C;
  const int tmask = a.T - 1;  // T is a power of two: keeps every unit index < F
  const uint16_t* cnt_row = a.counts + static_cast<size_t>(row) * nT;

  int off[kCountGroups];
  int total = 0;
#pragma unroll
  for (int q = 0; q < kCountGroups; ++q) {
    off[q] = 0;
    if (q * 64 < nT) {  // uniform
      const int incl = wave_inclusive_scan(c[q]);
      off[q] = total + incl - c[q];
      total += __builtin_amdgcn_readlane(incl, 63);
    }
  }
  if (nT <= 64 * kCountGroups && total <= kListCap) {
#pragma unroll
    for (int q = 0; q < kCountGroups; ++q) {
      const int t = q * 64 + lane;
      const size_t slot0 = (static_cast<size_t>(row) * nT + t) * C;
      for (int s = 0; s < c[q]; ++s) {
        lj[off[q] + s] = t * a.T + (static_cast<int>(a.idx[slot0 + s]) & tmask);
        if constexpr (kWithValues) lg[off[q] + s] = a.vals[slot0 + s];
      }
    }
    wave_lds_sync();
    if (total > 0) body(total, 0);
    wave_lds_sync();
    return total;
  }

  // General case: tile groups of 64 one after another, kListCap units a round.
  int ebase = 0;
  for (int t0 = 0; t0 < nT; t0 += 64) {
    const int t = t0 + lane;
    const int ct = (t < nT) ? static_cast<int>(cnt_row[t]) : 0;
    const int incl = wave_inclusive_scan(ct);
    const int gtotal = __builtin_amdgcn_readlane(incl, 63);
    const int o = incl - ct;
    const size_t slot0 = (static_cast<size_t>(row) * nT + t) * C;
    for (int base = 0; base < gtotal; base += kListCap) {
      const int s_lo = max(0, base - o);
      const int s_hi = min(ct, base + kListCap - o);
      for (int s = s_lo; s < s_hi; ++s) {
        lj[o + s - base] = t * a.T + (static_cast<int>(a.idx[slot0 + s]) & tmask);
        if constexpr (kWithValues) lg[o + s - base] = a.vals[slot0 + s];
      }
      wave_lds_sync();
      body(min(kListCap, gtotal - base), ebase + base);
      wave_lds_sync();
    }
    ebase += gtotal;
  }
  return ebase;
}

// Row lists: one wave per row, four rows a workgroup. Lane l holds the
// count of tile t0 + l; a prefix sum over the lanes gives each tile's first
// entry. A row with a count above C is an overflow row: its length is -1 and
// the entries it may have written are never read.
__global__ __launch_bounds__(256) void row_list_kernel(SlicedArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.M) return;
  const int nT = a.F / a.T;
  const int C = a.C;
  const int tmask = a.T - 1;  // T is a power of two: keeps every unit index < F
  const size_t cap = static_cast<size_t>(nT) * C;
  const uint16_t* cnt_row = a.counts + static_cast<size_t>(row) * nT;
  int2* lrow = a.list + static_cast<size_t>(row) * cap;
  int base = 0;
  for (int t0 = 0; t0 < nT; t0 += 64) {
    const int t = t0 + lane;
    const int c = (t < nT) ? static_cast<int>(cnt_row[t]) : 0;
    if (__ballot(c > C) != 0) {
      if (lane == 0) a.row_len[row] = -1;
      return;
    }
    const int incl = wave_inclusive_scan(c);
    const int o = base + incl - c;
    const size_t slot0 = (static_cast<size_t>(row) * nT + t) * C;
    for (int e = 0; e < c; ++e)
      lrow[o + e] = make_int2(t * a.T + (static_cast<int>(a.idx[slot0 + e]) & tmask),
                              __float_as_int(a.vals[slot0 + e]));
    base += __builtin_amdgcn_readlane(incl, 63);
  }
  if (lane == 0) a.row_len[row] = base;
}

// Entries a wave takes from the row list per round: one per lane.
constexpr int kRound = 64;

// Waves per SIMD the up pass is compiled for. The kernel waits on dependent
// global round trips (list, weight rows), so more resident waves hide more of
// them. Shapes other than V = 4 (d = 2048) keep the compiler's choice.
template <int V>
constexpr int up_waves_per_simd() {
  return V == 4 ? 6 : 1;
}

template <int L, int V, int U>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(up_waves_per_simd<V>(), 8)))
void sliced_up_kernel(SlicedArgs a) {
  constexpr int G = 64 / L;
  __shared__ int s_j[kRound + kListPad];
  __shared__ float s_g[kRound + kListPad];

  const int lane = threadIdx.x;
  const int slice = blockIdx.x % kSlices;
  const int row = blockIdx.x / kSlices;
  if (row >= a.M) return;

  const int cap = (a.F / a.T) * a.C;
  const int2* lrow = a.list + static_cast<size_t>(row) * cap;
  // First round trip, all issued together: the row's first kRound list
  // entries (whatever the row holds past its length is dropped below), its
  // length, and the x slice.
  int2 ent = (lane < cap) ? lrow[lane] : make_int2(0, 0);
  const int n = __builtin_amdgcn_readfirstlane(a.row_len[row]);  // -1: overflow row

  const int grp = lane / L, li = lane % L;
  const int col0 = slice * (a.d / kSlices) + li * 8;  // piece v of this lane: col0 + v * 8L
  u32x4_t xv[V];
  const uint16_t* xr = a.x + static_cast<size_t>(row) * a.d + col0;
#pragma unroll
  for (int v = 0; v < V; ++v) xv[v] = gload16(xr + v * 8 * L);

  float* prow = a.part + (static_cast<size_t>(slice) * a.M + row) * cap;
  const uint32_t row_bytes = static_cast<uint32_t>(a.d) * 2u;
  const uint32_t col_bytes = static_cast<uint32_t>(col0) * 2u;
  static_assert(G * U <= kListPad, "a step reads at most kListPad entries past the round");
  if (lane < kListPad) {  // steps past a round's last entry read unit 0 (a valid row), value 0
    s_j[kRound + lane] = 0;
    s_g[kRound + lane] = 0.f;
  }
  for (int e0 = 0; e0 < n; e0 += kRound) {
    const int m = min(kRound, n - e0);
    int2 nxt = make_int2(0, 0);  // the next round's entries, loaded behind this round's gathers
    if (e0 + kRound + lane < n) nxt = lrow[e0 + kRound + lane];
    s_j[lane] = (lane < m) ? ent.x : 0;
    s_g[lane] = (lane < m) ? __int_as_float(ent.y) : 0.f;
    wave_lds_sync();
    for (int e = 0; e < m; e += G * U) {
      u32x4_t wu[U][V];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t off = static_cast<uint32_t>(s_j[e + u * G + grp]) * row_bytes + col_bytes;
#pragma unroll
        for (int v = 0; v < V; ++v) wu[u][v] = ldg16(a.WuT, off + v * 16 * L);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float part = 0.f;
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int q = 0; q < 4; ++q) part = dot2_bf16(xv[v][q], wu[u][v][q], part);
        part = group_sum<L>(part);
        const int k = e + u * G + grp;
        if (li == 0 && k < m) prow[e0 + k] = s_g[k] * part;
      }
    }
    wave_lds_sync();
    ent = nxt;
  }
}

// L > 32 (one group, lanes >= L idle) avoids the cross-group sum for the
// slice widths that are not a power-of-two number of pieces.
template <int L, int V, int U>
__global__ __launch_bounds__(64) void sliced_down_kernel(SlicedArgs a) {
  constexpr int G = 64 / L;
  __shared__ int s_j[kRound + kListPad];
  __shared__ float s_h[kRound + kListPad];

  const int lane = threadIdx.x;
  const int slice = blockIdx.x % kSlices;
  const int row = blockIdx.x / kSlices;
  if (row >= a.M) return;

  const int cap = (a.F / a.T) * a.C;
  const int2* lrow = a.list + static_cast<size_t>(row) * cap;
  // The row's length and the units of its first kRound entries together; the
  // empty asm keeps the entry load ahead of the length test.
  int j = (lane < cap) ? lrow[lane].x : 0;
  asm volatile("" ::"v"(j));
  const int n = __builtin_amdgcn_readfirstlane(a.row_len[row]);
  if (n < 0) return;  // overflow row: the dense fallback writes it

  const int grp = (G == 1) ? 0 : lane / L;
  const int li = (G == 1) ? min(lane, L - 1) : lane % L;  // idle lanes repeat the last piece
  const int col0 = slice * (a.d / kSlices) + li * 8;
  const size_t slice_stride = static_cast<size_t>(a.M) * cap;
  const float* prow = a.part + static_cast<size_t>(row) * cap;
  const uint32_t row_bytes = static_cast<uint32_t>(a.d) * 2u;
  const uint32_t col_bytes = static_cast<uint32_t>(col0) * 2u;

  float acc[V][8];
#pragma unroll
  for (int v = 0; v < V; ++v)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[v][k] = 0.f;

  static_assert(G * U <= kListPad, "a step reads at most kListPad entries past the round");
  if (lane < kListPad) {  // steps past a round's last entry read unit 0 (a valid row), h 0
    s_j[kRound + lane] = 0;
    s_h[kRound + lane] = 0.f;
  }
  for (int e0 = 0; e0 < n; e0 += kRound) {
    const int m = min(kRound, n - e0);
    int jn = 0;  // the next round's units, loaded behind this round's gathers
    if (e0 + kRound + lane < n) jn = lrow[e0 + kRound + lane].x;
    // h of the round's entries: the slices' partial products summed in slice order
    float h = 0.f;
    if (lane < m) {
#pragma unroll
      for (int s = 0; s < kSlices; ++s) h += prow[s * slice_stride + e0 + lane];
    }
    s_j[lane] = (lane < m) ? j : 0;
    s_h[lane] = h;
    wave_lds_sync();
    for (int e = 0; e < m; e += G * U) {
      u32x4_t wd[U][V];
      float hv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = e + u * G + grp;
        hv[u] = s_h[k];
        const uint32_t off = static_cast<uint32_t>(s_j[k]) * row_bytes + col_bytes;
#pragma unroll
        for (int v = 0; v < V; ++v) wd[u][v] = ldg16(a.Wd, off + v * 16 * L);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[v][2 * q] = fmaf(hv[u], bf16_lo(wd[u][v][q]), acc[v][2 * q]);
            acc[v][2 * q + 1] = fmaf(hv[u], bf16_hi(wd[u][v][q]), acc[v][2 * q + 1]);
          }
    }
    wave_lds_sync();
    j = jn;
  }

  // The G groups hold partial sums of the same output columns.
  static_for<0, 6>([&](auto I) {
    constexpr int X = 1 << I.value;
    if constexpr (X >= L && X < 64) {
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if constexpr (X == 32)
            acc[v][k] = sum_halves(acc[v][k]);
          else
            acc[v][k] += xor_lanes<X>(acc[v][k]);
        }
    }
  });

  // y is stored non-temporal: an XCD's slice of it (4 MB at M = 4096,
  // d = 2048, as large as its L2) would otherwise evict its Wd slice.
  float* yr = a.y + static_cast<size_t>(row) * a.d + col0;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    if (v % G == grp && (G > 1 || lane < L)) {
      store16_nt(yr + v * 8 * L, acc[v][0], acc[v][1], acc[v][2], acc[v][3]);
      store16_nt(yr + v * 8 * L + 4, acc[v][4], acc[v][5], acc[v][6], acc[v][7]);
    }
  }
}

// Down product of the gate-only variant: the packing holds h itself, so one
// pass does it. Wave per (row, slice s): the row's stored units and their h
// are staged from the packing (as the up pass stages units and g), then
// y_r[s] = sum_e h_e * Wd[j_e][s] exactly as in the down pass. Overflow rows
// are left untouched (the dense fallback owns them).
template <int L, int V, int U>
__global__ __launch_bounds__(64 * kRowsPerWG) void hidden_down_kernel(SlicedArgs a) {
  constexpr int G = 64 / L;
  __shared__ int s_j[kRowsPerWG][kListCap + kListPad];
  __shared__ float s_h[kRowsPerWG][kListCap + kListPad];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int slice = blockIdx.x % kSlices;
  const int row = (blockIdx.x / kSlices) * kRowsPerWG + w;
  if (row >= a.M) return;

  const int nT = a.F / a.T;
  const uint16_t* cnt_row = a.counts + static_cast<size_t>(row) * nT;
  int c[kCountGroups];
  bool over = false;
#pragma unroll
  for (int q = 0; q < kCountGroups; ++q) {
    const int t = q * 64 + lane;
    c[q] = (t < nT) ? static_cast<int>(cnt_row[t]) : 0;
    over |= c[q] > a.C;
  }
  for (int t = 64 * kCountGroups + lane; t < nT; t += 64) over |= cnt_row[t] > a.C;
  if (__ballot(over) != 0) return;  // owned by the dense fallback

  const int grp = (G == 1) ? 0 : lane / L;
  const int li = (G == 1) ? min(lane, L - 1) : lane % L;  // idle lanes repeat the last piece
  const int col0 = slice * (a.d / kSlices) + li * 8;
  const uint32_t row_bytes = static_cast<uint32_t>(a.d) * 2u;
  const uint32_t col_bytes = static_cast<uint32_t>(col0) * 2u;
  int* lj = s_j[w];
  float* lh = s_h[w];

  float acc[V][8];
#pragma unroll
  for (int v = 0; v < V; ++v)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[v][k] = 0.f;

  stage_row<true>(a, row, c, lj, lh, [&](int n, int) {
    static_assert(G * U <= kListPad, "a step reads at most kListPad entries past the list");
    if (lane < kListPad) {  // pad to a whole step: unit 0 (a valid row), h 0
      lj[n + lane] = 0;
      lh[n + lane] = 0.f;
    }
    wave_lds_sync();
    for (int e = 0; e < n; e += G * U) {
      u32x4_t wd[U][V];
      float hv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = e + u * G + grp;
        hv[u] = lh[k];
        const uint32_t off = static_cast<uint32_t>(lj[k]) * row_bytes + col_bytes;
#pragma unroll
        for (int v = 0; v < V; ++v) wd[u][v] = ldg16(a.Wd, off + v * 16 * L);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[v][2 * q] = fmaf(hv[u], bf16_lo(wd[u][v][q]), acc[v][2 * q]);
            acc[v][2 * q + 1] = fmaf(hv[u], bf16_hi(wd[u][v][q]), acc[v][2 * q + 1]);
          }
    }
  });

  static_for<0, 6>([&](auto I) {
    constexpr int X = 1 << I.value;
    if constexpr (X >= L && X < 64) {
#pragma unroll
      for (int v = 0; v < V; ++v)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if constexpr (X == 32)
            acc[v][k] = sum_halves(acc[v][k]);
          else
            acc[v][k] += xor_lanes<X>(acc[v][k]);
        }
    }
  });

  float* yr = a.y + static_cast<size_t>(row) * a.d + col0;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    if (v % G == grp && (G > 1 || lane < L)) {
      *reinterpret_cast<float4*>(yr + v * 8 * L) = make_float4(acc[v][0], acc[v][1], acc[v][2], acc[v][3]);
      *reinterpret_cast<float4*>(yr + v * 8 * L + 4) = make_float4(acc[v][4], acc[v][5], acc[v][6], acc[v][7]);
    }
  }
}

// Loads in flight per lane per step. Up pass: about 8 sixteen-byte vectors.
// Down pass: about 4 (deeper unrolling costs more in occupancy than it gains).
template <int L, int V>
constexpr int unroll_up() {  // also at most L, so a step spans at most 64 entries
  return (V >= 8 ? 1 : 8 / V) < L ? (V >= 8 ? 1 : 8 / V) : L;
}
template <int V>
constexpr int unroll_down() {
  return V <= 1 ? 4 : (V <= 2 ? 2 : 1);
}

template <int L, int V>
hipError_t launch_up(const SlicedArgs& a, hipStream_t s, dim3 grid, dim3 block) {
  sliced_up_kernel<L, V, unroll_up<L, V>()><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

template <int L, int V>
hipError_t launch_down(const SlicedArgs& a, hipStream_t s, dim3 grid, dim3 block) {
  sliced_down_kernel<L, V, unroll_down<V>()><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

template <int L, int V>
hipError_t launch_hdown(const SlicedArgs& a, hipStream_t s, dim3 grid, dim3 block) {
  hidden_down_kernel<L, V, unroll_down<V>()><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

// A slice row is pieces = d / 64 sixteen-byte pieces, read by groups of L
// lanes holding V = pieces / L pieces each.
// Up pass: narrow groups (L = 8 where it divides, else 4; doubled while V > 8),
// since every stored unit's partial product is summed within its group.
// Down pass: wide groups (L = the largest power of two <= 64 dividing pieces,
// V <= 7, or one group of `pieces` lanes when 32 < pieces < 64), since its
// cross-group sum happens once per row.
bool lane_split_up(int d, int* L, int* V) {
  if (d < 256 || d > 8192 || d % 256 != 0) return false;
  const int pieces = d / 64;
  int l = (pieces % 8 == 0) ? 8 : 4;
  while (pieces / l > 8 && l < 64 && pieces % (2 * l) == 0) l *= 2;
  *L = l;
  *V = pieces / l;
  return *V <= 8;
}

bool lane_split_down(int d, int* L, int* V) {
  if (d < 256 || d > 8192 || d % 256 != 0) return false;
  const int pieces = d / 64;
  if (pieces > 32 && pieces < 64) {
    *L = pieces;
    *V = 1;
    return true;
  }
  int l = 64;
  while (pieces % l != 0) l >>= 1;
  *L = l;
  *V = pieces / l;
  return *V <= 7;
}

// Instantiated (L, V) pairs, one per supported d; the switch key is L * 16 + V.
#define TWELL_UP_SHAPES(X)                                                                          \
  X(4, 1) X(8, 1) X(4, 3) X(8, 2) X(4, 5) X(8, 3) X(4, 7) X(8, 4) X(8, 5) X(8, 6) X(8, 7) X(8, 8) \
      X(16, 5) X(16, 6) X(16, 7) X(16, 8)
#define TWELL_DOWN_SHAPES(X)                                                                      \
  X(4, 1) X(8, 1) X(4, 3) X(16, 1) X(4, 5) X(8, 3) X(4, 7) X(32, 1) X(40, 1) X(48, 1) X(56, 1) \
      X(64, 1) X(16, 5) X(32, 3) X(16, 7) X(64, 2)

}  // namespace

bool sliced_supports(int64_t d, int64_t F) {
  int L, V;
  if (!lane_split_up(int(d), &L, &V) || !lane_split_down(int(d), &L, &V)) return false;
  return F * d * 2 < (int64_t(1) << 31);  // 32-bit byte offsets into WuT and Wd
}

SlicedLayout sliced_layout(int64_t M, int64_t F, int T, int C) {
  const size_t cap = size_t(F / T) * size_t(C);
  SlicedLayout l;
  l.part = 0;
  l.list = align256(size_t(kSlices) * size_t(M) * cap * sizeof(float));
  l.row_len = l.list + align256(size_t(M) * cap * sizeof(int2));
  l.total = l.row_len + align256(size_t(M) * sizeof(int32_t));
  return l;
}

hipError_t launch_sliced_updown(const SlicedArgs& a, hipStream_t s) {
  int Lu, Vu, Ld, Vd;
  if (!sliced_supports(a.d, a.F)) return hipErrorInvalidValue;
  lane_split_up(a.d, &Lu, &Vu);
  lane_split_down(a.d, &Ld, &Vd);
  row_list_kernel<<<(a.M + 3) / 4, 256, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(a.M * kSlices), block(64);
  e = hipErrorInvalidValue;
  switch (Lu * 16 + Vu) {
#define TWELL_CASE(L, V) \
  case L * 16 + V: e = launch_up<L, V>(a, s, grid, block); break;
    TWELL_UP_SHAPES(TWELL_CASE)
#undef TWELL_CASE
    default: break;
  }
  if (e != hipSuccess) return e;
  e = hipErrorInvalidValue;
  switch (Ld * 16 + Vd) {
#define TWELL_CASE(L, V) \
  case L * 16 + V: e = launch_down<L, V>(a, s, grid, block); break;
    TWELL_DOWN_SHAPES(TWELL_CASE)
#undef TWELL_CASE
    default: break;
  }
  return e;
}

hipError_t launch_hidden_down(const SlicedArgs& a, hipStream_t s) {
  int L, V;
  if (!sliced_supports(a.d, a.F)) return hipErrorInvalidValue;
  lane_split_down(a.d, &L, &V);
  const dim3 grid(((a.M + kRowsPerWG - 1) / kRowsPerWG) * kSlices), block(64 * kRowsPerWG);
  switch (L * 16 + V) {
#define TWELL_CASE(L, V) \
  case L * 16 + V: return launch_hdown<L, V>(a, s, grid, block);
    TWELL_DOWN_SHAPES(TWELL_CASE)
#undef TWELL_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace twell
