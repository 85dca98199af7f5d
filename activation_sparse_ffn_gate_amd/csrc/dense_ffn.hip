// Dense gated FFN on MFMA, for gfx950: the dense baseline and the dense
// fallback of overflow rows.
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
// strides over the tiles the list needs), so no host synchronisation is needed
// and an empty list costs one short launch each.
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
  const int tiles_m = (R + kDM - 1) / kDM;
  const int ntiles = tiles_m * tiles_n;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int half = lane >> 5, col = lane & 31;
  const int lrow = tid >> 2, lpc = tid & 3;
  const uint32_t so[2] = {lds_off(lrow, lpc), lds_off(lrow + 64, lpc)};
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};

  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int m0 = (tile % tiles_m) * kDM;
    const int n0 = (tile / tiles_m) * kDN;
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

    const int nk = a.d / kDK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int st = kt & 1;
      if (kt + 1 < nk) gload((kt + 1) * kDK);
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
      if (kt + 1 < nk) sstore(st ^ 1);
      __syncthreads();
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
  const int tiles_m = (R + kDM - 1) / kDM;
  const int ntiles = tiles_m * tiles_n;

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

  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int m0 = (tile % tiles_m) * kDM;
    const int n0 = (tile / tiles_m) * kDN;
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

    const int nk = a.F / kDK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int st = kt & 1;
      if (kt + 1 < nk) gload((kt + 1) * kDK);
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
      if (kt + 1 < nk) sstore(st ^ 1);
      __syncthreads();
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
  gated_up_kernel<kGather, kSplit><<<dim3(g1), dim3(256), 0, s>>>(a, tiles_nf);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  down_kernel<kGather, kSplit><<<dim3(g2), dim3(256), 0, s>>>(a, tiles_nd);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense(const DenseArgs& a, hipStream_t s) {
  const bool gather = a.rows != nullptr, split = a.h_lo != nullptr;
  if (gather) return split ? launch_pair<true, true>(a, s) : launch_pair<true, false>(a, s);
  return split ? launch_pair<false, true>(a, s) : launch_pair<false, false>(a, s);
}

}  // namespace twell
