// Gate-only variant of the forward: dense gate and up products in one MFMA
// kernel whose epilogue packs the hidden value h = ReLU(z) * u into TwELL.
//
// This is a variant the pages do not describe. Their inference path packs the
// gate output g in the gate GEMM's epilogue and gathers one WuT row and one Wd
// row per stored unit (Telegram post on TwELL at tgviewer.app, part
// "Инференс"; aimodeling.com summary, paragraph 3). When more units are active
// the per-unit up gathers cost more than a dense up product, so here the up
// product is dense, formed from the same x tile as the gate, and only the down
// product gathers (one Wd row per stored unit, half the gathered bytes). The
// active set stays the gate's: a unit with z > 0 is stored even where h is
// zero or negative (the gate decides which units are live: Tencent Cloud
// article, section 1). Counts, slots, tile-local indices and the overflow set
// are exactly those of twell_gate_pack; only the stored value differs.
//
// Workgroup tile 128 tokens x 128 units, 4 waves as 2 x 2, each wave 64 x 64
// of z and of u (2 x 2 blocks of v_mfma_f32_32x32x16_bf16 each, 128 AGPRs),
// 32-wide K chunks in a double-buffered LDS stage holding the x, Wg and WuT
// tiles. A wave's 64 units are half a TwELL tile at T = 128 (the two waves of a
// tile add their per-token counts through LDS) or a whole tile at T = 64.
#include "gate_overflow.hpp"
#include "twell_device.hpp"
#include "twell_internal.hpp"

namespace twell {
namespace {

constexpr int kGM = 128, kGN = 128, kGK = 32;
constexpr int kGTile = kGM * kGK * 2;  // bytes of one 128 x 32 bf16 LDS tile

__device__ __forceinline__ f32x16_t zeros16() {
  f32x16_t z;
#pragma unroll
  for (int v = 0; v < 16; ++v) z[v] = 0.f;
  return z;
}

template <int kT, bool kDebug>
__global__ __launch_bounds__(256, 2) void gateup_pack_kernel(GateArgs a, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * 3 * kGTile];
  __shared__ int s_cnt[2][2][64];  // [wm][wn][token of the wave's 64]: count in the wave's 64 units
  __shared__ int s_flag;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int half = lane >> 5, col = lane & 31;
  const int lrow = tid >> 2, lpc = tid & 3;  // loader: row lrow (+64), 16-byte piece lpc of the chunk
  const uint32_t so[2] = {lds_off(lrow, lpc), lds_off(lrow + 64, lpc)};
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};

  // Each XCD (workgroups b with the same b % 8) gets a contiguous run of
  // tiles, token tiles fastest, so its tiles share Wg / WuT rows in its L2.
  const int nwg = gridDim.x, b = blockIdx.x;
  const int lin = (nwg % 8 == 0) ? (b % 8) * (nwg / 8) + (b / 8) : b;
  const int m0 = (lin % tiles_m) * kGM;
  const int n0 = (lin / tiles_m) * kGN;

  const uint16_t *pa[2], *pg[2], *pu[2];
  bool va[2], vb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = m0 + lrow + 64 * i;
    va[i] = r < a.M;
    pa[i] = a.x + static_cast<size_t>(va[i] ? r : 0) * a.d + lpc * 8;
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
    uint8_t* base = smem + st * 3 * kGTile;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      lds_store16(base, so[i], ra[i]);
      lds_store16(base + kGTile, so[i], rg[i]);
      lds_store16(base + 2 * kGTile, so[i], ru[i]);
    }
  };

  f32x16_t az[2][2], au[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) az[i][j] = au[i][j] = zeros16();

  const int nk = a.d / kGK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * kGK);
    const uint8_t* As = smem + st * 3 * kGTile;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4_t af[2], gf[2], uf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = lds_frag(As, wm * 64 + i * 32, ks, lane);
        gf[i] = lds_frag(As + kGTile, wn * 64 + i * 32, ks, lane);
        uf[i] = lds_frag(As + 2 * kGTile, wn * 64 + i * 32, ks, lane);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          az[i][j] = mfma_32x32x16(af[i], gf[j], az[i][j]);
          au[i][j] = mfma_32x32x16(af[i], uf[j], au[i][j]);
        }
    }
    if (kt + 1 < nk) sstore(st ^ 1);
    __syncthreads();
  }

  // ------------------------------------------------------------- epilogue
  // Rows and units past the matrix never count; h = ReLU(z) u in fp32.
  const int ucol0 = n0 + wn * 64;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = ucol0 + j * 32 + col;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * 64 + i * 32 + acc_row(v, half);
        const bool ok = row < a.M && c < a.F;
        const float z = ok ? az[i][j][v] : 0.f;
        const float h = fmaxf(z, 0.f) * au[i][j][v];
        if constexpr (kDebug) {
          if (ok) {
            a.z_debug[static_cast<size_t>(row) * a.F + c] = z;
            a.h_debug[static_cast<size_t>(row) * a.F + c] = h;
          }
        }
        az[i][j][v] = z;
        au[i][j][v] = h;
      }
    }

  // This wave's count of each of its 64 tokens (lane t holds token t).
  int cw = 0;
  static_for<0, 32>([&](auto I) {
    constexpr int i = decltype(I)::value / 16, v = decltype(I)::value % 16;
    const uint64_t b0 = __ballot(az[i][0][v] > 0.f), b1 = __ballot(az[i][1][v] > 0.f);
    cw = writelane<32 * i + acc_row(v, 0)>(cw, __popc(static_cast<uint32_t>(b0)) + __popc(static_cast<uint32_t>(b1)));
    cw = writelane<32 * i + acc_row(v, 1)>(cw, __popc(static_cast<uint32_t>(b0 >> 32)) +
                                                   __popc(static_cast<uint32_t>(b1 >> 32)));
  });
  s_cnt[wm][wn][lane] = cw;
  __syncthreads();
  // T = 128: the two waves of the workgroup row make one tile (wn = 0 first);
  // T = 64: each wave's units are a tile of their own.
  constexpr bool kPair = kT == 128;
  const int pre = (kPair && wn == 1) ? s_cnt[wm][0][lane] : 0;
  const int tot = kPair ? s_cnt[wm][0][lane] + s_cnt[wm][1][lane] : cw;
  const int nT = a.F / kT;
  const int tile = kPair ? n0 / kT : ucol0 / kT;
  const int C = a.C;
  int appended = 0;
  if (tile < nT) {
    const uint32_t row_slots = static_cast<uint32_t>(nT * C);
    const int ubase = kPair ? wn * 64 : 0;  // tile-local index of the wave's first unit
    static_for<0, 32>([&](auto I) {
      constexpr int i = decltype(I)::value / 16, v = decltype(I)::value % 16;
      constexpr int t_lo = 32 * i + acc_row(v, 0), t_hi = 32 * i + acc_row(v, 1);
      const uint64_t b0 = __ballot(az[i][0][v] > 0.f), b1 = __ballot(az[i][1][v] > 0.f);
      if ((b0 | b1) == 0) return;
      const uint32_t p = half ? static_cast<uint32_t>(__builtin_amdgcn_readlane(pre, t_hi))
                              : static_cast<uint32_t>(__builtin_amdgcn_readlane(pre, t_lo));
      const uint32_t row = static_cast<uint32_t>(m0 + wm * 64 + i * 32 + acc_row(v, half));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint64_t bq = j ? b1 : b0;
        if (bq == 0) continue;
        // slot: active units left of this one in the token's tile
        uint32_t rank = half ? __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bq >> 32), 0u)
                             : __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bq), 0u);
        if (j == 1) rank += half ? __popc(static_cast<uint32_t>(b0 >> 32)) : __popc(static_cast<uint32_t>(b0));
        const uint32_t slot = rank + p;
        if (az[i][j][v] > 0.f && slot < static_cast<uint32_t>(C)) {
          const uint32_t at = row * row_slots + static_cast<uint32_t>(tile * C) + slot;
          store_at(a.vals, at * 4u, au[i][j][v]);
          store_at(a.idx, at, static_cast<uint8_t>(ubase + j * 32 + col));
        }
      }
    });
    // Counts and overflow membership: the tile's first wave, lane t = token t.
    const int row = m0 + wm * 64 + lane;
    if ((!kPair || wn == 0) && row < a.M) {
      a.counts[static_cast<size_t>(row) * nT + tile] = static_cast<uint16_t>(tot);
      if (tot > C) appended = overflow_append(a, row);
    }
  }
  overflow_finalize(a, appended, &s_flag);
}

}  // namespace

hipError_t launch_gateup_pack(const GateArgs& a, hipStream_t s) {
  if (a.WuT == nullptr || (a.z_debug == nullptr) != (a.h_debug == nullptr)) return hipErrorInvalidValue;
  const int tiles_m = (a.M + kGM - 1) / kGM;
  const int tiles_n = (a.F + kGN - 1) / kGN;
  const dim3 grid(tiles_m * tiles_n), block(256);
  const bool dbg = a.z_debug != nullptr;
  if (a.T == 128) {
    if (dbg) gateup_pack_kernel<128, true><<<grid, block, 0, s>>>(a, tiles_m, tiles_n);
    else gateup_pack_kernel<128, false><<<grid, block, 0, s>>>(a, tiles_m, tiles_n);
  } else {
    if (dbg) gateup_pack_kernel<64, true><<<grid, block, 0, s>>>(a, tiles_m, tiles_n);
    else gateup_pack_kernel<64, false><<<grid, block, 0, s>>>(a, tiles_m, tiles_n);
  }
  return hipGetLastError();
}

}  // namespace twell
