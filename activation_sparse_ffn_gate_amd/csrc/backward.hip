// Training side of TwELL for gfx950: the hybrid format and the sparse
// backward of the gated FFN.
//
// The pages' training kernels (Telegram post on TwELL at tgviewer.app, part
// "Обучение"; Tencent Cloud article, section 3): every row of the gate output
// is kept either as one sparse block of the same width K for all rows, or,
// when it has too many active units, as a dense row in a reserve; with it the
// backward pass multiplies no two dense matrices. For y = (ReLU(z) ⊙ u) Wd,
// z = x Wg^T, u = x WuT^T and upstream gradient dy, only active units (z > 0)
// carry gradient:
//   dh_j = dy . Wd_j,  dz_j = dh_j u_j,  du_j = dh_j g_j,  h_j = g_j u_j
//   dx   = sum_j dz_j Wg_j + du_j WuT_j
//   dWg_j = sum_r dz_rj x_r,  dWuT_j = sum_r du_rj x_r,  dWd_j = sum_r h_rj dy_r
// so every product is a gather of weight rows (per token) or of activation
// rows (per unit).
//
// MI355X mapping.
//  * hybrid_pack: one wave per row turns a complete TwELL packing (C = T, so
//    no tile drops units) into the row's block (global unit indices,
//    ascending) or, past K, a reserve row.
//  * row_backward: one wave per token, x and dy rows in registers, the dx row
//    accumulated in fp32; per listed unit three coalesced 2d-byte row gathers
//    (WuT_j gives u and the du term, Wd_j gives dh, Wg_j the dz term), two
//    v_dot2_f32_bf16 wave reductions. Each unit's (h, dz, du) is written to
//    an entry list laid out row by row.
//  * The entry list is sorted by unit with a stable radix sort, so each
//    unit's entries stay in row order; unit_grads then gives each unit one
//    wave that walks its entries in that order and accumulates its three
//    gradient rows from gathered x and dy rows. Every sum has a fixed order:
//    results do not depend on scheduling.
#include <hipcub/hipcub.hpp>

#include "twell_device.hpp"
#include "twell_internal.hpp"

namespace twell {
namespace {

constexpr int kRowsPerWG = 4;
constexpr int kListCap = 512;

// ------------------------------------------------------------- hybrid pack
__global__ __launch_bounds__(64 * kRowsPerWG) void hybrid_pack_kernel(HybridArgs a) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * kRowsPerWG + (threadIdx.x >> 6);
  if (r >= a.M) return;
  const int nT = a.F / a.T;
  const uint16_t* cnt = a.counts + static_cast<size_t>(r) * nT;
  int total = 0;
  for (int t = lane; t < nT; t += 64) total += cnt[t];
  total = __builtin_amdgcn_readlane(wave_inclusive_scan(total), 63);
  if (lane == 0) a.h_count[r] = total;
  const size_t slot0 = static_cast<size_t>(r) * nT * a.C;
  if (total <= a.K) {
    int32_t* bi = a.h_idx + static_cast<size_t>(r) * a.K;
    float* bv = a.h_vals + static_cast<size_t>(r) * a.K;
    int base = 0;
    for (int t0 = 0; t0 < nT; t0 += 64) {
      const int t = t0 + lane;
      const int c = t < nT ? static_cast<int>(cnt[t]) : 0;
      const int incl = wave_inclusive_scan(c);
      const int off = base + incl - c;
      for (int s = 0; s < c; ++s) {
        const size_t k = slot0 + static_cast<size_t>(t) * a.C + s;
        bi[off + s] = t * a.T + static_cast<int>(a.idx[k]);
        bv[off + s] = a.vals[k];
      }
      base += __builtin_amdgcn_readlane(incl, 63);
    }
    return;
  }
  // Reserve row: the whole g row, densely.
  int pos = 0;
  if (lane == 0) pos = atomicAdd(a.n_res, 1);
  pos = __builtin_amdgcn_readfirstlane(pos);
  if (pos >= a.R) return;  // the reserve is full: n_res reports it
  if (lane == 0) {
    a.res_rows[pos] = r;
    if (a.K > 0) a.h_idx[static_cast<size_t>(r) * a.K] = pos;  // a reserve row's block holds its slot
  }
  float* dense = a.res_vals + static_cast<size_t>(pos) * a.F;
  for (int j = lane; j < a.F; j += 64) dense[j] = 0.f;
  __threadfence();  // the zeros are in place before the values go over them
  for (int t = lane; t < nT; t += 64) {
    const int c = cnt[t];
    for (int s = 0; s < c; ++s) {
      const size_t k = slot0 + static_cast<size_t>(t) * a.C + s;
      dense[t * a.T + static_cast<int>(a.idx[k])] = a.vals[k];
    }
  }
}

// ----------------------------------------------------- entry list set-up
// row_off[r] = entries before row r (exclusive scan of h_count), row_off[M] =
// all entries. One workgroup of 1024 threads, each scanning a run of rows.
__global__ __launch_bounds__(1024) void scan_rows_kernel(const int32_t* count, int M, int32_t* row_off) {
  __shared__ int64_t s_sum[1024];
  const int tid = threadIdx.x;
  const int per = (M + 1023) / 1024;
  const int lo = min(M, tid * per), hi = min(M, lo + per);
  int64_t sum = 0;
  for (int r = lo; r < hi; ++r) sum += count[r];
  s_sum[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan of the 1024 run sums
    const int64_t v = tid >= off ? s_sum[tid - off] : 0;
    __syncthreads();
    s_sum[tid] += v;
    __syncthreads();
  }
  int64_t run = s_sum[tid] - sum;
  for (int r = lo; r < hi; ++r) {
    row_off[r] = static_cast<int32_t>(min<int64_t>(run, INT32_MAX));
    run += count[r];
  }
  if (tid == 1023) row_off[M] = static_cast<int32_t>(min<int64_t>(s_sum[1023], INT32_MAX));
}

// Every entry slot starts past the last unit (the sort moves unused slots to
// the end) and carries its own index as the sort's value.
__global__ void init_entries_kernel(int32_t* keys, int32_t* perm_in, int64_t n, int F) {
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    keys[e] = F;
    perm_in[e] = static_cast<int32_t>(e);
  }
}

// ------------------------------------------------------------ row backward
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
__global__ __launch_bounds__(64 * kRowsPerWG) void row_backward_kernel(BackwardArgs a) {
  using LoadT = typename Vec<VEC>::T;
  constexpr int kW = Vec<VEC>::kWords;
  constexpr int kChunk = 64 * VEC;
  __shared__ int s_j[kRowsPerWG][kListCap];
  __shared__ float s_g[kRowsPerWG][kListCap];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int r = blockIdx.x * kRowsPerWG + w;
  if (r >= a.M) return;
  const int n = a.h_count[r];
  const bool reserve = n > a.K;
  const float* dense = nullptr;
  if (reserve) {
    const int slot = a.K > 0 ? a.h_idx[static_cast<size_t>(r) * a.K] : -1;
    const int stored = min(*a.n_res, a.R);
    if (slot < 0 || slot >= stored) return;  // not held by the reserve: no valid gradient
    dense = a.res_vals + static_cast<size_t>(slot) * a.F;
  }

  LoadT xv[NCH], dyv[NCH];
  const uint16_t* xr = a.x + static_cast<size_t>(r) * a.d + lane * VEC;
  const uint16_t* dr = a.dy + static_cast<size_t>(r) * a.d + lane * VEC;
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    xv[ch] = *reinterpret_cast<const LoadT*>(xr + ch * kChunk);
    dyv[ch] = *reinterpret_cast<const LoadT*>(dr + ch * kChunk);
  }
  float acc[NCH][VEC];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
    for (int k = 0; k < VEC; ++k) acc[ch][k] = 0.f;

  int* lj = s_j[w];
  float* lg = s_g[w];
  const int64_t e0 = a.row_off[r];
  int done = 0;      // entries of this row handled so far
  int scan_at = 0;   // reserve rows: next unit to scan
  while (done < n) {
    // Stage up to kListCap of the row's (unit, g) in LDS.
    int m = 0;
    if (!reserve) {
      m = min(kListCap, n - done);
      for (int k = lane; k < m; k += 64) {
        lj[k] = a.h_idx[static_cast<size_t>(r) * a.K + done + k];
        lg[k] = a.h_vals[static_cast<size_t>(r) * a.K + done + k];
      }
    } else {
      while (scan_at < a.F && m <= kListCap - 64) {
        const int j = scan_at + lane;
        const float g = j < a.F ? dense[j] : 0.f;
        const uint64_t bal = __ballot(g > 0.f);
        if (g > 0.f) {
          const int at = m + static_cast<int>(mask_rank(bal));
          lj[at] = j;
          lg[at] = g;
        }
        m += __popcll(bal);
        scan_at += 64;
      }
      m = min(m, n - done);
      if (m == 0) break;  // fewer active units than the count says: stop rather than spin
    }
    wave_lds_sync();
    for (int e = 0; e < m; e += UNROLL) {
      int j[UNROLL];
      float g[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int ee = min(e + u, m - 1);
        j[u] = __builtin_amdgcn_readfirstlane(lj[ee]);
        g[u] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(lg[ee])));
      }
      LoadT wu[UNROLL][NCH], wd[UNROLL][NCH], wg[UNROLL][NCH];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const size_t rb = static_cast<size_t>(j[u]) * a.d + lane * VEC;
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
          wu[u][ch] = *reinterpret_cast<const LoadT*>(a.WuT + rb + ch * kChunk);
          wd[u][ch] = *reinterpret_cast<const LoadT*>(a.Wd + rb + ch * kChunk);
          wg[u][ch] = *reinterpret_cast<const LoadT*>(a.Wg + rb + ch * kChunk);
        }
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        if (e + u < m) {  // uniform
          float pu = 0.f, pd = 0.f;
#pragma unroll
          for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
            for (int q = 0; q < kW; ++q) {
              pu = dot2_bf16(xv[ch][q], wu[u][ch][q], pu);
              pd = dot2_bf16(dyv[ch][q], wd[u][ch][q], pd);
            }
          const float uu = wave_sum(pu);
          const float dh = wave_sum(pd);
          const float dz = dh * uu;
          const float du = dh * g[u];
#pragma unroll
          for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
            for (int q = 0; q < kW; ++q) {
              acc[ch][2 * q] = fmaf(dz, bf16_lo(wg[u][ch][q]), acc[ch][2 * q]);
              acc[ch][2 * q + 1] = fmaf(dz, bf16_hi(wg[u][ch][q]), acc[ch][2 * q + 1]);
              acc[ch][2 * q] = fmaf(du, bf16_lo(wu[u][ch][q]), acc[ch][2 * q]);
              acc[ch][2 * q + 1] = fmaf(du, bf16_hi(wu[u][ch][q]), acc[ch][2 * q + 1]);
            }
          const int64_t ent = e0 + done + e + u;
          if (lane == 0 && ent < a.E_max) {
            a.keys[ent] = j[u];
            a.e_row[ent] = r;
            a.e_h[ent] = g[u] * uu;
            a.e_dz[ent] = dz;
            a.e_du[ent] = du;
          }
        }
      }
    }
    done += m;
    wave_lds_sync();
  }

  float* dxr = a.dx + static_cast<size_t>(r) * a.d + lane * VEC;
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
    for (int k = 0; k < VEC; k += 4)
      *reinterpret_cast<float4*>(dxr + ch * kChunk + k) =
          make_float4(acc[ch][k], acc[ch][k + 1], acc[ch][k + 2], acc[ch][k + 3]);
}

// ------------------------------------------------------ per-unit gradients
// First position of the sorted keys holding a value >= v (keys ascending).
__device__ __forceinline__ int64_t lower_bound(const int32_t* keys, int64_t n, int v) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (keys[mid] < v) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

template <int VEC, int NCH, int UNROLL>
__global__ __launch_bounds__(64 * kRowsPerWG) void unit_grads_kernel(BackwardArgs a) {
  using LoadT = typename Vec<VEC>::T;
  constexpr int kW = Vec<VEC>::kWords;
  constexpr int kChunk = 64 * VEC;
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * kRowsPerWG + (threadIdx.x >> 6);
  if (j >= a.F) return;
  int64_t lo = 0, hi = 0;
  if (lane == 0) {
    lo = lower_bound(a.keys_sorted, a.E_max, j);
    hi = lower_bound(a.keys_sorted, a.E_max, j + 1);
  }
  lo = __builtin_amdgcn_readfirstlane(static_cast<int>(lo));
  hi = __builtin_amdgcn_readfirstlane(static_cast<int>(hi));

  float gd[NCH][VEC], gg[NCH][VEC], gu[NCH][VEC];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
    for (int k = 0; k < VEC; ++k) gd[ch][k] = gg[ch][k] = gu[ch][k] = 0.f;

  for (int64_t k0 = lo; k0 < hi; k0 += UNROLL) {
    int row[UNROLL];
    float h[UNROLL], dz[UNROLL], du[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t kk = min(k0 + u, hi - 1);
      const int e = a.perm[kk];
      row[u] = __builtin_amdgcn_readfirstlane(a.e_row[e]);
      h[u] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.e_h[e])));
      dz[u] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.e_dz[e])));
      du[u] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.e_du[e])));
    }
    LoadT xv[UNROLL][NCH], dyv[UNROLL][NCH];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const size_t rb = static_cast<size_t>(row[u]) * a.d + lane * VEC;
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        xv[u][ch] = *reinterpret_cast<const LoadT*>(a.x + rb + ch * kChunk);
        dyv[u][ch] = *reinterpret_cast<const LoadT*>(a.dy + rb + ch * kChunk);
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      if (k0 + u < hi) {  // uniform
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
          for (int q = 0; q < kW; ++q) {
            const float x0 = bf16_lo(xv[u][ch][q]), x1 = bf16_hi(xv[u][ch][q]);
            gg[ch][2 * q] = fmaf(dz[u], x0, gg[ch][2 * q]);
            gg[ch][2 * q + 1] = fmaf(dz[u], x1, gg[ch][2 * q + 1]);
            gu[ch][2 * q] = fmaf(du[u], x0, gu[ch][2 * q]);
            gu[ch][2 * q + 1] = fmaf(du[u], x1, gu[ch][2 * q + 1]);
            gd[ch][2 * q] = fmaf(h[u], bf16_lo(dyv[u][ch][q]), gd[ch][2 * q]);
            gd[ch][2 * q + 1] = fmaf(h[u], bf16_hi(dyv[u][ch][q]), gd[ch][2 * q + 1]);
          }
      }
    }
  }
  const size_t ob = static_cast<size_t>(j) * a.d + lane * VEC;
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
    for (int k = 0; k < VEC; k += 4) {
      *reinterpret_cast<float4*>(a.dWg + ob + ch * kChunk + k) =
          make_float4(gg[ch][k], gg[ch][k + 1], gg[ch][k + 2], gg[ch][k + 3]);
      *reinterpret_cast<float4*>(a.dWu + ob + ch * kChunk + k) =
          make_float4(gu[ch][k], gu[ch][k + 1], gu[ch][k + 2], gu[ch][k + 3]);
      *reinterpret_cast<float4*>(a.dWd + ob + ch * kChunk + k) =
          make_float4(gd[ch][k], gd[ch][k + 1], gd[ch][k + 2], gd[ch][k + 3]);
    }
}

template <int NCH>
constexpr int row_unroll() {
  return NCH <= 2 ? 4 : (NCH <= 4 ? 2 : 1);
}
template <int NCH>
constexpr int unit_unroll() {
  return NCH <= 2 ? 8 : (NCH <= 4 ? 4 : (NCH <= 8 ? 2 : 1));
}

template <int VEC, int NCH>
hipError_t launch_rows(const BackwardArgs& a, hipStream_t s) {
  row_backward_kernel<VEC, NCH, row_unroll<NCH>()>
      <<<dim3((a.M + kRowsPerWG - 1) / kRowsPerWG), dim3(64 * kRowsPerWG), 0, s>>>(a);
  return hipGetLastError();
}
template <int VEC, int NCH>
hipError_t launch_units(const BackwardArgs& a, hipStream_t s) {
  unit_grads_kernel<VEC, NCH, unit_unroll<NCH>()>
      <<<dim3((a.F + kRowsPerWG - 1) / kRowsPerWG), dim3(64 * kRowsPerWG), 0, s>>>(a);
  return hipGetLastError();
}

// d = 512 n (n = 1..16): 16-byte lanes; other multiples of 256 below 4096:
// 8-byte lanes.
template <bool kUnits, int... N>
hipError_t dispatch8(int nch, const BackwardArgs& a, hipStream_t s, std::integer_sequence<int, N...>) {
  hipError_t r = hipErrorInvalidValue;
  ((nch == N + 1 ? (r = kUnits ? launch_units<8, N + 1>(a, s) : launch_rows<8, N + 1>(a, s), 0) : 0), ...);
  return r;
}
template <bool kUnits, int... N>
hipError_t dispatch4(int nch, const BackwardArgs& a, hipStream_t s, std::integer_sequence<int, N...>) {
  hipError_t r = hipErrorInvalidValue;
  ((nch == 2 * N + 1 ? (r = kUnits ? launch_units<4, 2 * N + 1>(a, s) : launch_rows<4, 2 * N + 1>(a, s), 0) : 0),
   ...);
  return r;
}
template <bool kUnits>
hipError_t dispatch(const BackwardArgs& a, hipStream_t s) {
  if (a.d % 512 == 0) return dispatch8<kUnits>(a.d / 512, a, s, std::make_integer_sequence<int, 16>{});
  return dispatch4<kUnits>(a.d / 256, a, s, std::make_integer_sequence<int, 8>{});
}

int key_bits(int F) {  // keys are 0..F
  int b = 1;
  while ((int64_t(1) << b) <= F) ++b;
  return b;
}

}  // namespace

bool backward_supports_d(int d) { return d >= 256 && d % 256 == 0 && (d % 512 == 0 ? d <= 8192 : d < 4096); }

hipError_t launch_hybrid_pack(const HybridArgs& a, hipStream_t s) {
  hipError_t e = launch_set_i32(a.n_res, 0, s);
  if (e != hipSuccess) return e;
  hybrid_pack_kernel<<<dim3((a.M + kRowsPerWG - 1) / kRowsPerWG), dim3(64 * kRowsPerWG), 0, s>>>(a);
  return hipGetLastError();
}

size_t backward_sort_bytes(int64_t n, int F) {
  size_t bytes = 0;
  hipcub::DeviceRadixSort::SortPairs(nullptr, bytes, static_cast<const int32_t*>(nullptr),
                                     static_cast<int32_t*>(nullptr), static_cast<const int32_t*>(nullptr),
                                     static_cast<int32_t*>(nullptr), static_cast<int>(n), 0, key_bits(F),
                                     hipStream_t(nullptr));
  return bytes;
}

hipError_t launch_backward(const BackwardArgs& a, hipStream_t s) {
  scan_rows_kernel<<<dim3(1), dim3(1024), 0, s>>>(a.h_count, a.M, a.row_off);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t blocks = std::min<int64_t>((a.E_max + 255) / 256, 4096);
  init_entries_kernel<<<dim3(static_cast<unsigned>(std::max<int64_t>(blocks, 1))), dim3(256), 0, s>>>(
      a.keys, a.perm_in, a.E_max, a.F);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.M > 0 && (e = dispatch<false>(a, s)) != hipSuccess) return e;
  size_t bytes = a.sort_bytes;
  e = hipcub::DeviceRadixSort::SortPairs(a.sort_tmp, bytes, a.keys, a.keys_sorted, a.perm_in, a.perm,
                                         static_cast<int>(a.E_max), 0, key_bits(a.F), s);
  if (e != hipSuccess) return e;
  return dispatch<true>(a, s);
}

}  // namespace twell
