// Dense gated FFN on MFMA with register-staged 128 x 128 tiles, for gfx950:
// the dense fallback of overflow rows (every list but those long enough for
// the ring kernels of dense_ring.hip), and the dense baseline for shapes whose
// operands exceed the ring kernels' 32-bit offsets.
//
// Kernel 1 (gated up): for a block of rows, z = x Wg^T and u = x WuT^T share
// one A tile; the epilogue forms h = ReLU(z) * u and stores it as bf16, or as
// a bf16 hi/lo pair (h ~ hi + lo to about 2^-16 relative) when the result must
// stay within 1e-3 of the fp64 definition.
// Kernel 2 (down): y = h Wd (and + h_lo Wd) in fp32. Wd is [F, d] with d
// contiguous while the MFMA wants 8 consecutive k (= F) values per lane, so
// each thread loads a 4 (k) x 4 (d) block, transposes it in registers and
// stores it to LDS in [d][k] order.
//
// The fallback runs the same kernels over a device-side row list whose length
// is only known on the device: both kernels are persistent (a fixed grid that
// strides over the work the list needs), so no host synchronisation is needed
// and an empty list costs one short launch each.
//
// A short list (a few overflow rows) gives few output tiles, each with a long
// K loop (K = F = 8192 for the down product), which would leave most of the GPU
// idle. Then the K loop of every tile is split S ways (S chosen on the device
// from the list length): each split stores its fp32 partial tile in the
// workspace and a reduce launch after each product (persistent too, empty when
// there is no split) adds the S partial tiles in split order and runs the
// epilogue. The sum order is fixed. The launch boundary makes the partial
// tiles of every XCD visible to the reducer; an in-kernel last-arriver
// reduction measured at about half of each product's time (a device-scope
// fence per split to publish its partial tile, then one workgroup per tile
// reading all S partial tiles).
//
// Workgroup tile 128 x 128, 4 waves as 2 x 2, each wave 64 x 64 (2 x 2 MFMA
// 32x32x16 blocks), 32-wide K chunks double-buffered in LDS.
#include "twell_device.hpp"
#include "twell_internal.hpp"

namespace twell {
namespace {

constexpr int kDM = 128, kDN = 128, kDK = 32;
constexpr int kTile = kDM * kDK * 2;  // bytes of one 128 x 32 bf16 LDS tile
constexpr int kPersistentWGs = 512;

// Split-K policy of the gathering (fallback) kernels.
constexpr int kSplitBelow = 128;   // split when there are fewer output tiles than this
constexpr int kTargetItems = 256;  // aim for about this many (tile, split) work items
constexpr int kMaxSplit = 16;
constexpr int kMinSplitChunks = 8;  // K chunks of 32 per split at least

struct SplitPlan {
  int S, items;
};

__device__ __forceinline__ SplitPlan plan_split(bool allowed, int tiles, int nk) {
  static_assert(2 * kTargetItems <= kDenseSplitSlots, "partial slots of the gated-up kernel");
  if (!allowed || tiles == 0 || tiles >= kSplitBelow) return {1, tiles};
  int S = kTargetItems / tiles;
  S = min(S, min(kMaxSplit, max(nk / kMinSplitChunks, 1)));
  S = max(S, 1);
  return {S, tiles * S};
}

// Output tile and K split of work item `item`. Unsplit, with whole passes of
// the persistent grid: workgroups are dispatched round-robin over the 8 XCDs,
// so each XCD takes a contiguous run of every pass's items, walked in groups
// of kGroupM token tiles (unit tiles within a group): the tiles an XCD runs
// at once form a block of 8 x 8 that shares its x and weight tiles in that
// XCD's L2. Otherwise token tiles vary fastest.
constexpr int kGroupM = 8;
struct DenseTile {
  int m0, n0, sp;
};
__device__ __forceinline__ DenseTile dense_tile(int item, const SplitPlan& plan, int tiles_m, int tiles_n) {
  const int G = gridDim.x;
  if (plan.S == 1 && G % 8 == 0 && plan.items % G == 0 && tiles_m >= kGroupM) {
    const int pass = item / G, b = item - pass * G;
    const int lin = pass * G + (b % 8) * (G / 8) + b / 8;
    const int group = lin / (kGroupM * tiles_n);
    const int within = lin - group * kGroupM * tiles_n;
    const int gm = min(kGroupM, tiles_m - group * kGroupM);
    return {(group * kGroupM + within % gm) * kDM, (within / gm) * kDN, 0};
  }
  const int tile = item / plan.S;
  return {(tile % tiles_m) * kDM, (tile / tiles_m) * kDN, item % plan.S};
}

// Element (row, column) of float4 q of thread t in a tile's flattened
// accumulators (flatten below): rows row0 .. row0 + 3 of one column.
struct PartPos {
  int row0, col;
};
__device__ __forceinline__ PartPos part_pos(int q, int t) {
  const int w = t >> 6, lane = t & 63;
  const int k = 4 * q;  // flattened index (i * 2 + j) * 16 + v, v % 4 == 0
  const int i = k >> 5, j = (k >> 4) & 1, v = k & 15;
  return {(w >> 1) * 64 + i * 32 + acc_row(v, lane >> 5), (w & 1) * 64 + j * 32 + (lane & 31)};
}

// Stores this thread's 64 fp32 accumulators (16 float4) of split slot `slot`,
// except float4s whose rows all lie at or past `rows` (tile-local).
__device__ __forceinline__ void store_partial(float* part, int slot, const float (&v)[64], int rows) {
  float4* p = reinterpret_cast<float4*>(part) + static_cast<size_t>(slot) * 16 * 256;
#pragma unroll
  for (int q = 0; q < 16; ++q)
    if (part_pos(q, threadIdx.x).row0 < rows)
      p[q * 256 + threadIdx.x] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
}

// float4 q of thread t summed over slots slot0 + stride * s, s = 0 .. S-1, in that order.
__device__ __forceinline__ float4 sum_partials(const float* part, int slot0, int stride, int S, int q, int t) {
  const float4* p = reinterpret_cast<const float4*>(part) + q * 256 + t;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < S; ++s) {
    const float4 v = p[static_cast<size_t>(slot0 + stride * s) * 16 * 256];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  return acc;
}

// Flattened views of a wave's 2 x 2 block of 32x32 accumulators.
__device__ __forceinline__ void flatten(const f32x16_t (&acc)[2][2], float (&v)[64]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int k = 0; k < 16; ++k) v[(i * 2 + j) * 16 + k] = acc[i][j][k];
}


__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int v = 0; v < 16; ++v) z[v] = 0.f;
  return z;
}

template <bool kGather, bool kSplit>
__global__ __launch_bounds__(256, 2) void gated_up_kernel(DenseArgs a, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * 3 * kTile];
  const int R = kGather ? min(max(*a.n_rows, 0), a.M) : a.M;
  if (kGather && a.ring_min_rows > 0 && R >= a.ring_min_rows) return;  // the ring kernels take this list
  const int tiles_m = (R + kDM - 1) / kDM;
  const int nk = a.d / kDK;
  const SplitPlan plan = plan_split(kGather && a.split_k, tiles_m * tiles_n, nk);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int half = lane >> 5, col = lane & 31;
  const int lrow = tid >> 2, lpc = tid & 3;
  const uint32_t so[2] = {lds_off(lrow, lpc), lds_off(lrow + 64, lpc)};
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};

  for (int item = blockIdx.x; item < plan.items; item += gridDim.x) {
    const DenseTile dt = dense_tile(item, plan, tiles_m, tiles_n);
    const int sp = dt.sp, m0 = dt.m0, n0 = dt.n0;
    const int kb = sp * nk / plan.S, ke = (sp + 1) * nk / plan.S;  // this split's K chunks
    const uint16_t *pa[2], *pg[2], *pu[2];
    bool va[2], vb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = m0 + lrow + 64 * i;
      int src = (r < R) ? (kGather ? a.rows[r] : r) : -1;
      va[i] = src >= 0 && src < a.M;  // list entries outside [0, M) read as zero rows
      src = va[i] ? src : 0;
      pa[i] = a.x + static_cast<size_t>(src) * a.d + lpc * 8;
      const int c = n0 + lrow + 64 * i;
      vb[i] = c < a.F;
      pg[i] = a.Wg + static_cast<size_t>(vb[i] ? c : 0) * a.d + lpc * 8;
      pu[i] = a.WuT + static_cast<size_t>(vb[i] ? c : 0) * a.d + lpc * 8;
    }
    u32x4_t ra[2], rg[2], ru[2];
    auto gload = [&](int k0) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        ra[i] = va[i] ? gload16(pa[i] + k0) : zero4;
        rg[i] = vb[i] ? gload16(pg[i] + k0) : zero4;
        ru[i] = vb[i] ? gload16(pu[i] + k0) : zero4;
      }
    };
    auto sstore = [&](int st) {
      uint8_t* base = smem + st * 3 * kTile;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        lds_store16(base, so[i], ra[i]);
        lds_store16(base + kTile, so[i], rg[i]);
        lds_store16(base + 2 * kTile, so[i], ru[i]);
      }
    };

    f32x16_t ag[2][2], au[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) ag[i][j] = au[i][j] = zero16();

    gload(kb * kDK);
    sstore(0);
    __syncthreads();
    for (int kt = kb; kt < ke; ++kt) {
      const int st = (kt - kb) & 1;
      if (kt + 1 < ke) gload((kt + 1) * kDK);
      const uint8_t* As = smem + st * 3 * kTile;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4_t af[2], gf[2], uf[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          af[i] = lds_frag(As, wm * 64 + i * 32, ks, lane);
          gf[i] = lds_frag(As + kTile, wn * 64 + i * 32, ks, lane);
          uf[i] = lds_frag(As + 2 * kTile, wn * 64 + i * 32, ks, lane);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            ag[i][j] = mfma_32x32x16(af[i], gf[j], ag[i][j]);
            au[i][j] = mfma_32x32x16(af[i], uf[j], au[i][j]);
          }
      }
      if (kt + 1 < ke) sstore(st ^ 1);
      __syncthreads();
    }

    if (plan.S > 1) {  // slots 2 * item (z) and 2 * item + 1 (u); gated_up_reduce_kernel finishes
      float v[64];
      flatten(ag, v);
      store_partial(a.part, 2 * item, v, R - m0);
      flatten(au, v);
      store_partial(a.part, 2 * item + 1, v, R - m0);
      continue;
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = n0 + wn * 64 + j * 32 + col;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = m0 + wm * 64 + i * 32 + acc_row(v, half);
          if (r < R && c < a.F) {
            const float h = fmaxf(ag[i][j][v], 0.f) * au[i][j][v];
            const uint32_t hi = f32_to_bf16_rne(h);
            const size_t o = static_cast<size_t>(r) * a.F + c;
            a.h_hi[o] = static_cast<uint16_t>(hi);
            if constexpr (kSplit) a.h_lo[o] = static_cast<uint16_t>(f32_to_bf16_rne(h - __uint_as_float(hi << 16)));
          }
        }
      }
  }
}

template <bool kGather, bool kSplit>
__global__ __launch_bounds__(256, 2) void down_kernel(DenseArgs a, int tiles_n) {
  constexpr int kNA = kSplit ? 2 : 1;
  constexpr int kStage = (kNA + 1) * kTile;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage];
  const int R = kGather ? min(max(*a.n_rows, 0), a.M) : a.M;
  if (kGather && a.ring_min_rows > 0 && R >= a.ring_min_rows) return;  // the ring kernels take this list
  const int tiles_m = (R + kDM - 1) / kDM;
  const int nk = a.F / kDK;
  const SplitPlan plan = plan_split(kGather && a.split_k, tiles_m * tiles_n, nk);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int half = lane >> 5, col = lane & 31;
  const int lrow = tid >> 2, lpc = tid & 3;
  const uint32_t so[2] = {lds_off(lrow, lpc), lds_off(lrow + 64, lpc)};
  // B (Wd) block of this thread: k rows kg*4..+3, d columns ng*4..+3
  const int ng = tid & 31, kg = tid >> 5;
  uint32_t sbo[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) sbo[q] = lds_off(ng * 4 + q, kg >> 1) + (kg & 1) * 8;
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};

  for (int item = blockIdx.x; item < plan.items; item += gridDim.x) {
    const DenseTile dt = dense_tile(item, plan, tiles_m, tiles_n);
    const int sp = dt.sp, m0 = dt.m0, n0 = dt.n0;
    const int kb = sp * nk / plan.S, ke = (sp + 1) * nk / plan.S;
    const uint16_t* pa[kNA][2];
    bool va[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = m0 + lrow + 64 * i;
      va[i] = r < R;
      const size_t o = static_cast<size_t>(va[i] ? r : 0) * a.F + lpc * 8;
      pa[0][i] = a.h_hi + o;
      if constexpr (kSplit) pa[1][i] = a.h_lo + o;
    }
    const uint16_t* pb = a.Wd + static_cast<size_t>(kg * 4) * a.d + n0 + ng * 4;

    u32x4_t ra[kNA][2];
    u32x2_t rb[4];
    auto gload = [&](int k0) {
#pragma unroll
      for (int s = 0; s < kNA; ++s)
#pragma unroll
        for (int i = 0; i < 2; ++i) ra[s][i] = va[i] ? gload16(pa[s][i] + k0) : zero4;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        rb[q] = *reinterpret_cast<const u32x2_t*>(pb + static_cast<size_t>(k0 + q) * a.d);
    };
    auto sstore = [&](int st) {
      uint8_t* base = smem + st * kStage;
#pragma unroll
      for (int s = 0; s < kNA; ++s)
#pragma unroll
        for (int i = 0; i < 2; ++i) lds_store16(base + s * kTile, so[i], ra[s][i]);
      // 4x4 transpose of 16-bit values: column q of the loaded block becomes
      // the 4 consecutive k values of output column ng*4 + q.
      uint8_t* bt = base + kNA * kTile;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int word = q >> 1;
        const int sh = (q & 1) * 16;
        const uint32_t e0 = (rb[0][word] >> sh) & 0xFFFFu, e1 = (rb[1][word] >> sh) & 0xFFFFu;
        const uint32_t e2 = (rb[2][word] >> sh) & 0xFFFFu, e3 = (rb[3][word] >> sh) & 0xFFFFu;
        u32x2_t v = {e0 | (e1 << 16), e2 | (e3 << 16)};
        *reinterpret_cast<u32x2_t*>(bt + sbo[q]) = v;
      }
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = zero16();

    gload(kb * kDK);
    sstore(0);
    __syncthreads();
    for (int kt = kb; kt < ke; ++kt) {
      const int st = (kt - kb) & 1;
      if (kt + 1 < ke) gload((kt + 1) * kDK);
      const uint8_t* base = smem + st * kStage;
      const uint8_t* Bs = base + kNA * kTile;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4_t bfr[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) bfr[j] = lds_frag(Bs, wn * 64 + j * 32, ks, lane);
#pragma unroll
        for (int s = 0; s < kNA; ++s) {
          u32x4_t af[2];
#pragma unroll
          for (int i = 0; i < 2; ++i) af[i] = lds_frag(base + s * kTile, wm * 64 + i * 32, ks, lane);
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = mfma_32x32x16(af[i], bfr[j], acc[i][j]);
        }
      }
      if (kt + 1 < ke) sstore(st ^ 1);
      __syncthreads();
    }

    if (plan.S > 1) {  // slot `item`; down_reduce_kernel finishes
      float v[64];
      flatten(acc, v);
      store_partial(a.part, item, v, R - m0);
      continue;
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = m0 + wm * 64 + i * 32 + acc_row(v, half);
        if (r < R) {
          const int dst = kGather ? a.rows[r] : r;
          if (dst >= 0 && dst < a.M) {
#pragma unroll
            for (int j = 0; j < 2; ++j) a.y[static_cast<size_t>(dst) * a.d + n0 + wn * 64 + j * 32 + col] = acc[i][j][v];
          }
        }
      }
  }
}

// Split epilogues: one work unit per (tile, float4 index q of the flattened
// accumulators); each thread adds its float4 over the S splits in split order
// and runs the product's epilogue for those 4 rows of one column.
constexpr int kReduceWGs = 2048;  // at most 127 split tiles x 16 units: one unit a workgroup

template <bool kSplit>
__global__ __launch_bounds__(256) void gated_up_reduce_kernel(DenseArgs a, int tiles_n) {
  const int R = min(max(*a.n_rows, 0), a.M);
  if (a.ring_min_rows > 0 && R >= a.ring_min_rows) return;  // the ring kernels took this list
  const int tiles_m = (R + kDM - 1) / kDM;
  const SplitPlan plan = plan_split(a.split_k, tiles_m * tiles_n, a.d / kDK);
  if (plan.S <= 1) return;
  const int t = threadIdx.x;
  for (int u = blockIdx.x; u < tiles_m * tiles_n * 16; u += gridDim.x) {
    const int tile = u >> 4, q = u & 15;
    const int m0 = (tile % tiles_m) * kDM, n0 = (tile / tiles_m) * kDN;
    const PartPos pp = part_pos(q, t);
    if (m0 + pp.row0 >= R) continue;  // never stored
    const float4 z = sum_partials(a.part, 2 * tile * plan.S, 2, plan.S, q, t);
    const float4 g = sum_partials(a.part, 2 * tile * plan.S + 1, 2, plan.S, q, t);
    const float zz[4] = {z.x, z.y, z.z, z.w}, uu[4] = {g.x, g.y, g.z, g.w};
    const int c = n0 + pp.col;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = m0 + pp.row0 + e;
      if (r < R && c < a.F) {
        const float h = fmaxf(zz[e], 0.f) * uu[e];
        const uint32_t hi = f32_to_bf16_rne(h);
        const size_t o = static_cast<size_t>(r) * a.F + c;
        a.h_hi[o] = static_cast<uint16_t>(hi);
        if constexpr (kSplit) a.h_lo[o] = static_cast<uint16_t>(f32_to_bf16_rne(h - __uint_as_float(hi << 16)));
      }
    }
  }
}

__global__ __launch_bounds__(256) void down_reduce_kernel(DenseArgs a, int tiles_n) {
  const int R = min(max(*a.n_rows, 0), a.M);
  if (a.ring_min_rows > 0 && R >= a.ring_min_rows) return;  // the ring kernels took this list
  const int tiles_m = (R + kDM - 1) / kDM;
  const SplitPlan plan = plan_split(a.split_k, tiles_m * tiles_n, a.F / kDK);
  if (plan.S <= 1) return;
  const int t = threadIdx.x;
  for (int u = blockIdx.x; u < tiles_m * tiles_n * 16; u += gridDim.x) {
    const int tile = u >> 4, q = u & 15;
    const int m0 = (tile % tiles_m) * kDM, n0 = (tile / tiles_m) * kDN;
    const PartPos pp = part_pos(q, t);
    if (m0 + pp.row0 >= R) continue;  // never stored
    const float4 v = sum_partials(a.part, tile * plan.S, 1, plan.S, q, t);
    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = m0 + pp.row0 + e;
      if (r < R) {
        const int dst = a.rows[r];
        if (dst >= 0 && dst < a.M) a.y[static_cast<size_t>(dst) * a.d + n0 + pp.col] = vv[e];
      }
    }
  }
}

template <bool kGather, bool kSplit>
hipError_t launch_pair(const DenseArgs& a, hipStream_t s) {
  const int tiles_nf = (a.F + kDN - 1) / kDN;
  const int tiles_nd = a.d / kDN;
  const int tiles_m = (a.M + kDM - 1) / kDM;  // upper bound when gathering
  int g1 = tiles_m * tiles_nf, g2 = tiles_m * tiles_nd;
  if (kGather) {
    g1 = g1 < kPersistentWGs ? g1 : kPersistentWGs;
    g2 = g2 < kPersistentWGs ? g2 : kPersistentWGs;
  }
  DenseArgs up = a, down = a;
  hipError_t e = hipSuccess;
  const bool ring = kGather && kSplit && a.ring_ws != nullptr;
  if (ring && (e = launch_ring_fallback_up(a, s)) != hipSuccess) return e;
  gated_up_kernel<kGather, kSplit><<<dim3(g1), dim3(256), 0, s>>>(up, tiles_nf);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool split = kGather && a.split_k;  // the product kernels may split K
  if (split) {
    gated_up_reduce_kernel<kSplit><<<dim3(kReduceWGs), dim3(256), 0, s>>>(up, tiles_nf);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (ring && (e = launch_ring_fallback_down(a, s)) != hipSuccess) return e;
  down_kernel<kGather, kSplit><<<dim3(g2), dim3(256), 0, s>>>(down, tiles_nd);
  e = hipGetLastError();
  if (e != hipSuccess || !split) return e;
  down_reduce_kernel<<<dim3(kReduceWGs), dim3(256), 0, s>>>(down, tiles_nd);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense(const DenseArgs& a, hipStream_t s) {
  const bool gather = a.rows != nullptr, split = a.h_lo != nullptr;
  if (gather) return split ? launch_pair<true, true>(a, s) : launch_pair<true, false>(a, s);
  return split ? launch_pair<false, true>(a, s) : launch_pair<false, false>(a, s);
}

}  // namespace twell
