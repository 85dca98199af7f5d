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
//  * hybrid_pack: one wave per row turns a TwELL packing into the row's
//    block (global unit indices, ascending) or, past K active units, a
//    reserve row. Tiles within capacity C come from the packing's slots; with
//    C < T a tile over C comes from the training gate's spill record (every z
//    of that tile), so no active unit is lost.
//  * row_backward: one wave per token, x and dy rows in registers, the dx row
//    accumulated in fp32; per listed unit three coalesced 2d-byte row gathers
//    (WuT_j gives u and the du term, Wd_j gives dh, Wg_j the dz term), two
//    v_dot2_f32_bf16 wave reductions. Each unit's (h, dz, du) is written to
//    an entry list laid out row by row.
//  * The entry list is reordered by unit with a stable counting sort: the
//    row kernel also counts entries per (block of kSortRows rows, unit); a
//    column scan turns the counts into each (block, unit)'s first position;
//    one workgroup per block then places its rows' entries in row order. So
//    each unit's entries stay in row order, and unit_grads gives each unit
//    one wave that walks them in that order and accumulates its three
//    gradient rows from gathered x and dy rows. Every sum has a fixed order:
//    results do not depend on scheduling.
#include "twell_device.hpp"
#include "twell_internal.hpp"

namespace twell {
namespace {

constexpr int kRowsPerWG = 4;
constexpr int kListCap = 512;
constexpr int kSortRows = 64;  // rows per block of the counting sort

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
  // A tile with more than C active units (only when C < T) is read from its
  // spill record: all T pre-activations, the active ones (z > 0) in ascending
  // order. A record past the list's capacity was not stored: the tile then
  // reads as empty (the caller sees n_spill > capacity).
  auto record = [&](int t) -> const float* {
    const int rec = a.rec_slot[static_cast<size_t>(r) * nT + t];
    return (rec >= 0 && rec < a.rec_cap) ? a.rec_z + static_cast<size_t>(rec) * a.T : nullptr;
  };
  if (total <= a.K) {
    int32_t* bi = a.h_idx + static_cast<size_t>(r) * a.K;
    float* bv = a.h_vals + static_cast<size_t>(r) * a.K;
    int base = 0;
    for (int t0 = 0; t0 < nT; t0 += 64) {
      const int t = t0 + lane;
      const int c = t < nT ? static_cast<int>(cnt[t]) : 0;
      const int incl = wave_inclusive_scan(c);
      const int off = base + incl - c;
      if (c <= a.C) {
        for (int s = 0; s < c; ++s) {
          const size_t k = slot0 + static_cast<size_t>(t) * a.C + s;
          bi[off + s] = t * a.T + static_cast<int>(a.idx[k]);
          bv[off + s] = a.vals[k];
        }
      } else if (const float* z = record(t)) {
        int s = 0;
        for (int i = 0; i < a.T && s < c; ++i) {
          const float v = z[i];
          if (v > 0.f) {
            bi[off + s] = t * a.T + i;
            bv[off + s] = v;
            ++s;
          }
        }
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
    if (c <= a.C) {
      for (int s = 0; s < c; ++s) {
        const size_t k = slot0 + static_cast<size_t>(t) * a.C + s;
        dense[t * a.T + static_cast<int>(a.idx[k])] = a.vals[k];
      }
    } else if (const float* z = record(t)) {
      for (int i = 0; i < a.T; ++i) {
        const float v = z[i];
        if (v > 0.f) dense[t * a.T + i] = v;
      }
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

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[e] = v;
}

// unit_base[j] = entries of units below j (exclusive scan over F; one
// workgroup of 1024 threads, each scanning a run of units); unit_base[F] = all.
__global__ __launch_bounds__(1024) void scan_units_kernel(const int32_t* tot, int F, int32_t* unit_base) {
  __shared__ int s_sum[1024];
  const int tid = threadIdx.x;
  const int per = (F + 1023) / 1024;
  const int lo = min(F, tid * per), hi = min(F, lo + per);
  int sum = 0;
  for (int j = lo; j < hi; ++j) sum += tot[j];
  s_sum[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? s_sum[tid - off] : 0;
    __syncthreads();
    s_sum[tid] += v;
    __syncthreads();
  }
  int run = s_sum[tid] - sum;
  for (int j = lo; j < hi; ++j) {
    unit_base[j] = run;
    run += tot[j];
  }
  if (tid == 1023) unit_base[F] = s_sum[1023];
}

// The per-block counts become first positions: (b, j) starts after unit j's
// entries of blocks < b.
__global__ void block_offsets_kernel(int32_t* hist, int nb, int F, const int32_t* unit_base) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= F) return;
  int run = unit_base[j];
  for (int b = 0; b < nb; ++b) {
    const size_t k = static_cast<size_t>(b) * F + j;
    const int c = hist[k];
    hist[k] = run;
    run += c;
  }
}

// One workgroup per block of kSortRows rows: rows in order, a row's entries
// (distinct units) in parallel; perm[position] = entry.
__global__ __launch_bounds__(256) void place_entries_kernel(const int32_t* row_off, const int32_t* e_unit,
                                                            const int32_t* offs, int M, int F, int64_t E_max,
                                                            int32_t* perm) {
  extern __shared__ int32_t s_off[];  // [F]
  const int b = blockIdx.x;
  for (int j = threadIdx.x; j < F; j += blockDim.x) s_off[j] = offs[static_cast<size_t>(b) * F + j];
  __syncthreads();
  const int r_end = min(M, (b + 1) * kSortRows);
  for (int r = b * kSortRows; r < r_end; ++r) {
    const int64_t e_lo = row_off[r], e_hi = min<int64_t>(row_off[r + 1], E_max);
    for (int64_t e = e_lo + threadIdx.x; e < e_hi; e += blockDim.x) {
      const int j = e_unit[e];
      if (j < 0 || j >= F) continue;  // unused entry
      const int pos = s_off[j];
      s_off[j] = pos + 1;
      perm[pos] = static_cast<int32_t>(e);
    }
    __syncthreads();  // the next row may hold the same units
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

// The per-unit work of one token row r: entries lj/lg[0 .. m) (LDS), entry
// numbers ent0 + k. Adds the row's dx terms to acc and writes each entry.
template <int VEC, int NCH, int UNROLL>
__device__ __forceinline__ void process_entries(const BackwardArgs& a, int r, const int* lj, const float* lg,
                                                int m, int64_t ent0, const typename Vec<VEC>::T (&xv)[NCH],
                                                const typename Vec<VEC>::T (&dyv)[NCH], float (&acc)[NCH][VEC]) {
  using LoadT = typename Vec<VEC>::T;
  constexpr int kW = Vec<VEC>::kWords;
  constexpr int kChunk = 64 * VEC;
  const int lane = threadIdx.x & 63;
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
        const int64_t ent = ent0 + e + u;
        if (lane == 0 && ent < a.E_max) {
          a.e_unit[ent] = j[u];
          atomicAdd(&a.hist[static_cast<size_t>(r / kSortRows) * a.F + j[u]], 1);
          atomicAdd(&a.unit_tot[j[u]], 1);
          a.e_row[ent] = r;
          a.e_h[ent] = g[u] * uu;
          a.e_dz[ent] = dz;
          a.e_du[ent] = du;
        }
      }
    }
  }
}

template <int VEC, int NCH>
__device__ __forceinline__ void load_row(const uint16_t* base, int d, int r, typename Vec<VEC>::T (&v)[NCH]) {
  using LoadT = typename Vec<VEC>::T;
  const uint16_t* p = base + static_cast<size_t>(r) * d + (threadIdx.x & 63) * VEC;
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) v[ch] = *reinterpret_cast<const LoadT*>(p + ch * 64 * VEC);
}

// Entries [from, e0 + n) of a row that are not produced are marked unused.
__device__ __forceinline__ void mark_unused(const BackwardArgs& a, int64_t from, int64_t end) {
  for (int64_t e = from + (threadIdx.x & 63); e < min<int64_t>(end, a.E_max); e += 64) a.e_unit[e] = -1;
}

// Rows held as sparse blocks: one wave per row. Reserve rows are left to
// reserve_backward_kernel (rows the reserve could not hold get no gradient).
template <int VEC, int NCH, int UNROLL>
__global__ __launch_bounds__(64 * kRowsPerWG) void row_backward_kernel(BackwardArgs a) {
  using LoadT = typename Vec<VEC>::T;
  constexpr int kChunk = 64 * VEC;
  __shared__ int s_j[kRowsPerWG][kListCap];
  __shared__ float s_g[kRowsPerWG][kListCap];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int r = blockIdx.x * kRowsPerWG + w;
  if (r >= a.M) return;
  const int n = a.h_count[r];
  const int64_t e0 = a.row_off[r];
  if (n > a.K) {
    const int slot = a.K > 0 ? a.h_idx[static_cast<size_t>(r) * a.K] : -1;
    if (slot < 0 || slot >= min(*a.n_res, a.R)) mark_unused(a, e0, e0 + n);
    return;
  }
  LoadT xv[NCH], dyv[NCH];
  load_row<VEC, NCH>(a.x, a.d, r, xv);
  load_row<VEC, NCH>(a.dy, a.d, r, dyv);
  float acc[NCH][VEC];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
    for (int k = 0; k < VEC; ++k) acc[ch][k] = 0.f;

  int* lj = s_j[w];
  float* lg = s_g[w];
  for (int done = 0; done < n; done += kListCap) {
    const int m = min(kListCap, n - done);
    for (int k = lane; k < m; k += 64) {
      lj[k] = a.h_idx[static_cast<size_t>(r) * a.K + done + k];
      lg[k] = a.h_vals[static_cast<size_t>(r) * a.K + done + k];
    }
    wave_lds_sync();
    process_entries<VEC, NCH, UNROLL>(a, r, lj, lg, m, e0 + done, xv, dyv, acc);
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

// Reserve rows. A row's active units are cut into runs of about kResRunMin
// (at most kResMaxRuns runs), and a persistent grid of workgroups of
// kResWaves waves walks the (row, run) work items: a few long rows then spread
// over the chip instead of keeping one workgroup busy each, while a short row
// stays one item. reserve_plan_kernel numbers the items (the first item of
// each row, a prefix over the rows). An item compacts its row's dense g into
// the ascending (unit, g) list (each wave counts a contiguous column range, a
// prefix over the waves places them) but keeps only its run in LDS; each wave
// takes a contiguous part of the run; the waves' dx rows are added in wave
// order through LDS (kRedCols columns at a time) into the run's partial dx
// row, and reserve_sum_kernel adds a row's runs in run order. kResWaves: 16
// while a wave's rows fit in 128 registers (d <= 2048), else 8.
constexpr int kResRunMin = 192;  // units per run (the last runs of a row may hold more)
constexpr int kResListCap = (kBackwardMaxF + kResMaxRuns - 1) / kResMaxRuns;  // a run's entries at most
constexpr int kResLdsBytes = 32768;  // the run's list, then the reduction
static_assert(kResListCap * 8 <= kResLdsBytes, "a run's list fits");

__device__ __forceinline__ int reserve_runs(int n) {
  return min(kResMaxRuns, max(1, (n + kResRunMin - 1) / kResRunMin));
}

// One workgroup: res_prefix[s] = first item of reserve row s, res_prefix[n_res]
// = the number of items.
__global__ __launch_bounds__(1024) void reserve_plan_kernel(BackwardArgs a) {
  __shared__ int s_sum[1024];
  const int n_res = min(*a.n_res, a.R);
  const int t = threadIdx.x;
  const int per = (n_res + 1023) / 1024;
  const int lo = min(n_res, t * per), hi = min(n_res, lo + per);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += reserve_runs(a.h_count[a.res_rows[i]]);
  s_sum[t] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan over the threads' sums
    const int v = t >= off ? s_sum[t - off] : 0;
    __syncthreads();
    s_sum[t] += v;
    __syncthreads();
  }
  int run = s_sum[t] - sum;
  for (int i = lo; i < hi; ++i) {
    a.res_prefix[i] = run;
    run += reserve_runs(a.h_count[a.res_rows[i]]);
  }
  if (t == 1023) a.res_prefix[n_res] = s_sum[1023];
}

template <int VEC, int NCH, int UNROLL, int kResWaves>
__global__ __launch_bounds__(64 * kResWaves) void reserve_backward_kernel(BackwardArgs a) {
  constexpr int kRedCols = kResLdsBytes / 4 / kResWaves;
  using LoadT = typename Vec<VEC>::T;
  constexpr int kChunk = 64 * VEC;
  static_assert(kRedCols % kChunk == 0, "a chunk's columns lie in one reduction pass");
  __shared__ __attribute__((aligned(16))) uint8_t smem[kResLdsBytes];
  __shared__ int s_cnt[kResWaves];
  int* lj = reinterpret_cast<int*>(smem);
  float* lg = reinterpret_cast<float*>(smem + kResListCap * 4);
  float* red = reinterpret_cast<float*>(smem);  // [kResWaves][kRedCols], after the list is done

  const int n_res = min(*a.n_res, a.R);
  if (n_res <= 0) return;
  const int items = a.res_prefix[n_res];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    // the item's row: the last s with res_prefix[s] <= item
    int lo = 0, hi = n_res - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.res_prefix[mid] <= item) lo = mid;
      else hi = mid - 1;
    }
    const int slot = lo;
    const int run = item - a.res_prefix[slot];
    const int r = a.res_rows[slot];
    const int n = a.h_count[r];
    const int runs = reserve_runs(n);
    const int64_t e0 = a.row_off[r];
    const float* dense = a.res_vals + static_cast<size_t>(slot) * a.F;

    // Compaction: wave w scans columns [w span, (w + 1) span).
    const int span = ((a.F + 64 * kResWaves - 1) / (64 * kResWaves)) * 64;
    const int c_lo = min(a.F, w * span), c_hi = min(a.F, c_lo + span);
    int cnt = 0;
#pragma unroll 4
    for (int c = c_lo; c < c_hi; c += 64) {  // four columns' loads in flight
      const int j = c + lane;
      cnt += __popcll(__ballot(j < c_hi && dense[j] > 0.f));
    }
    if (lane == 0) s_cnt[w] = cnt;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int v = 0; v < kResWaves; ++v) {
      base += v < w ? s_cnt[v] : 0;
      total += s_cnt[v];
    }
    const int m = min(total, n);
    // this item's run of the list: entries [k_run, k_run + m_run)
    const int k_run = static_cast<int>(static_cast<int64_t>(m) * run / runs);
    const int m_run = static_cast<int>(static_cast<int64_t>(m) * (run + 1) / runs) - k_run;
    // only waves whose columns hold some of the run's entries place any
    const bool mine = base < k_run + m_run && base + cnt > k_run;
    for (int c = c_lo; mine && c < c_hi; c += 64) {
      const int j = c + lane;
      const float g = j < c_hi ? dense[j] : 0.f;
      const uint64_t bal = __ballot(g > 0.f);
      if (g > 0.f) {
        const int at = base + static_cast<int>(mask_rank(bal)) - k_run;
        if (at >= 0 && at < m_run) {
          lj[at] = j;
          lg[at] = g;
        }
      }
      base += __popcll(bal);
    }
    __syncthreads();

    LoadT xv[NCH], dyv[NCH];
    load_row<VEC, NCH>(a.x, a.d, r, xv);
    load_row<VEC, NCH>(a.dy, a.d, r, dyv);
    float acc[NCH][VEC];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
      for (int k = 0; k < VEC; ++k) acc[ch][k] = 0.f;
    const int per = (m_run + kResWaves - 1) / kResWaves;
    const int k_lo = min(m_run, w * per), k_hi = min(m_run, k_lo + per);
    if (k_hi > k_lo)
      process_entries<VEC, NCH, UNROLL>(a, r, lj + k_lo, lg + k_lo, k_hi - k_lo, e0 + k_run + k_lo, xv, dyv, acc);
    if (run == 0 && w == 0 && m < n) mark_unused(a, e0 + m, e0 + n);
    __syncthreads();  // the list is no longer read

    float* prow = a.res_part + (static_cast<size_t>(slot) * kResMaxRuns + run) * a.d;
    for (int col0 = 0; col0 < a.d; col0 += kRedCols) {
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        const int c = ch * kChunk + lane * VEC;  // this lane's first column of chunk ch
        if (ch * kChunk >= col0 && ch * kChunk < col0 + kRedCols) {  // uniform
#pragma unroll
          for (int k = 0; k < VEC; ++k) red[w * kRedCols + (c - col0) + k] = acc[ch][k];
        }
      }
      __syncthreads();
      for (int c = threadIdx.x; c < kRedCols && col0 + c < a.d; c += 64 * kResWaves) {
        float sum = 0.f;
#pragma unroll
        for (int v = 0; v < kResWaves; ++v) sum += red[v * kRedCols + c];
        prow[col0 + c] = sum;
      }
      __syncthreads();  // before the next pass, or the next item's list, writes
    }
  }
}

// dx of each reserve row: its runs' partial rows added in run order.
__global__ __launch_bounds__(256) void reserve_sum_kernel(BackwardArgs a) {
  const int n_res = min(*a.n_res, a.R);
  for (int slot = blockIdx.x; slot < n_res; slot += gridDim.x) {
    const int runs = a.res_prefix[slot + 1] - a.res_prefix[slot];
    const int r = a.res_rows[slot];
    const float* p0 = a.res_part + static_cast<size_t>(slot) * kResMaxRuns * a.d;
    float* dxr = a.dx + static_cast<size_t>(r) * a.d;
    for (int c = threadIdx.x * 4; c < a.d; c += 256 * 4) {
      float4 s = *reinterpret_cast<const float4*>(p0 + c);
      for (int q = 1; q < runs; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(p0 + static_cast<size_t>(q) * a.d + c);
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
      }
      *reinterpret_cast<float4*>(dxr + c) = s;
    }
  }
}

// ------------------------------------------------------ per-unit gradients
template <int VEC, int NCH, int UNROLL>
__global__ __launch_bounds__(64 * kRowsPerWG) void unit_grads_kernel(BackwardArgs a) {
  using LoadT = typename Vec<VEC>::T;
  constexpr int kW = Vec<VEC>::kWords;
  constexpr int kChunk = 64 * VEC;
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * kRowsPerWG + (threadIdx.x >> 6);
  if (j >= a.F) return;
  const int64_t lo = a.unit_base[j], hi = a.unit_base[j + 1];

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
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.R == 0) return e;
  // 16 waves of a workgroup leave 128 registers a wave: one unit at a time
  constexpr int kWaves = VEC * NCH <= 32 ? 16 : 8;
  reserve_plan_kernel<<<dim3(1), dim3(1024), 0, s>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // persistent: one workgroup per CU at most (16 waves of 128 registers)
  const int grid = static_cast<int>(std::min<int64_t>(256, int64_t(a.R) * kResMaxRuns));
  reserve_backward_kernel<VEC, NCH, kWaves == 16 ? 1 : row_unroll<NCH>(), kWaves>
      <<<dim3(grid), dim3(64 * kWaves), 0, s>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  reserve_sum_kernel<<<dim3(static_cast<unsigned>(std::min<int64_t>(a.R, 1024))), dim3(256), 0, s>>>(a);
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

}  // namespace

bool backward_supports_d(int d) { return d >= 256 && d % 256 == 0 && (d % 512 == 0 ? d <= 8192 : d < 4096); }

hipError_t launch_hybrid_pack(const HybridArgs& a, hipStream_t s) {
  hipError_t e = launch_set_i32(a.n_res, 0, s);
  if (e != hipSuccess) return e;
  hybrid_pack_kernel<<<dim3((a.M + kRowsPerWG - 1) / kRowsPerWG), dim3(64 * kRowsPerWG), 0, s>>>(a);
  return hipGetLastError();
}

int backward_sort_blocks(int64_t M) { return static_cast<int>((M + kSortRows - 1) / kSortRows); }

hipError_t launch_backward(const BackwardArgs& a, hipStream_t s) {
  const int nb = backward_sort_blocks(a.M);
  const int64_t nh = static_cast<int64_t>(nb + 1) * a.F;  // per-block counts, then unit totals
  scan_rows_kernel<<<dim3(1), dim3(1024), 0, s>>>(a.h_count, a.M, a.row_off);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    fill_i32_kernel<<<dim3(static_cast<unsigned>(std::min<int64_t>((nh + 255) / 256, 4096))), dim3(256), 0, s>>>(
        a.hist, nh, 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.M > 0 && (e = dispatch<false>(a, s)) != hipSuccess) return e;
  const dim3 ug((a.F + 255) / 256), ub(256);
  scan_units_kernel<<<dim3(1), dim3(1024), 0, s>>>(a.unit_tot, a.F, a.unit_base);
  block_offsets_kernel<<<ug, ub, 0, s>>>(a.hist, nb, a.F, a.unit_base);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (nb > 0) {
    place_entries_kernel<<<dim3(nb), dim3(256), static_cast<size_t>(a.F) * 4, s>>>(a.row_off, a.e_unit, a.hist,
                                                                                   a.M, a.F, a.E_max, a.perm);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return dispatch<true>(a, s);
}

}  // namespace twell
