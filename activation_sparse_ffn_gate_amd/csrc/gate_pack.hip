// Gate GEMM with the TwELL packing in its epilogue, for gfx950.
//
// The pages' design (aimodeling.com TwELL summary, paragraph 3; pulsen.vercel.app
// article, paragraph on tile matching; Tencent Cloud article, section 2): the
// TwELL tile width equals the gate matmul's column tile, so the kernel that
// computes a tile of z = x Wg^T can pack its non-zeros right away: no second
// launch, no synchronisation between workgroups, no dense z in memory.
//
// MI355X mapping. One workgroup (4 waves) computes a 256-token x 128-unit tile
// with v_mfma_f32_32x32x16_bf16 over LDS-staged, double-buffered 32-wide K
// chunks. Each wave owns 64 tokens x all 128 units of the tile, so every
// (token, TwELL tile) row segment of 64 or 128 units lives inside one wave.
// Packing then needs no LDS round trip: in the accumulator layout one register
// holds, across the 64 lanes, 32 consecutive units of two tokens, so a 64-bit
// ballot of (z > 0) gives both tokens' activity masks; popcounts of the masks
// give the per-tile count and each lane's slot is the popcount of the mask bits
// below it (ascending unit order). Values (fp32) and tile-local indices are
// stored only for slots < C; the per-(token, tile) count is stored unclamped.
//
// Overflow rows (some tile count > C) are appended to a deduplicated list with
// device-scope atomics. The last workgroup to finish publishes the list length
// and clears the dedup flags, so the workspace control block is zero again
// when the kernel ends and no separate clearing launch is needed.
#include "twell_device.hpp"
#include "twell_internal.hpp"

namespace twell {
namespace {

constexpr int kBM = 256;  // tokens per workgroup tile
constexpr int kBN = 128;  // hidden units per workgroup tile
constexpr int kBK = 32;   // K chunk per LDS stage
constexpr int kATileBytes = kBM * kBK * 2;
constexpr int kBTileBytes = kBN * kBK * 2;
constexpr int kStageBytes = kATileBytes + kBTileBytes;

template <int kT, bool kDebug>
__global__ __launch_bounds__(256, 2) void gate_pack_kernel(GateArgs a, int tiles_m) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStageBytes];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;

  // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
  // contiguous run of tiles (token tiles fastest) so tiles that share a block
  // of Wg rows run on the same L2.
  const int nwg = gridDim.x, b = blockIdx.x;
  const int lin = (nwg % 8 == 0) ? (b % 8) * (nwg / 8) + (b / 8) : b;
  const int m0 = (lin % tiles_m) * kBM;
  const int n0 = (lin / tiles_m) * kBN;

  // Global -> LDS staging: thread loads 16-byte piece (tid & 3) of rows
  // (tid >> 2) + 64 i of the A (x) and B (Wg) chunks.
  const int lrow = tid >> 2, lpc = tid & 3;
  const uint16_t* pa[4];
  bool va[4];
  uint32_t sa[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = m0 + lrow + 64 * i;
    va[i] = r < a.M;
    pa[i] = a.x + static_cast<size_t>(va[i] ? r : 0) * a.d + lpc * 8;
    sa[i] = lds_off(lrow + 64 * i, lpc);
  }
  const uint16_t* pb[2];
  bool vb[2];
  uint32_t sb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = n0 + lrow + 64 * i;
    vb[i] = r < a.F;
    pb[i] = a.Wg + static_cast<size_t>(vb[i] ? r : 0) * a.d + lpc * 8;
    sb[i] = lds_off(lrow + 64 * i, lpc);
  }

  u32x4_t ra[4], rb[2];
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = va[i] ? gload16(pa[i] + k0) : zero4;
#pragma unroll
    for (int i = 0; i < 2; ++i) rb[i] = vb[i] ? gload16(pb[i] + k0) : zero4;
  };
  auto sstore = [&](int stage) {
    uint8_t* As = smem + stage * kStageBytes;
    uint8_t* Bs = As + kATileBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_store16(As, sa[i], ra[i]);
#pragma unroll
    for (int i = 0; i < 2; ++i) lds_store16(Bs, sb[i], rb[i]);
  };

  f32x16_t acc[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mb][nb][v] = 0.f;

  const int nk = a.d / kBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * kBK);
    const uint8_t* As = smem + st * kStageBytes;
    const uint8_t* Bs = As + kATileBytes;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4_t af[2], bf[4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) af[mb] = lds_frag(As, w * 64 + mb * 32, ks, lane);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) bf[nb] = lds_frag(Bs, nb * 32, ks, lane);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma_32x32x16(af[mb], bf[nb], acc[mb][nb]);
    }
    if (kt + 1 < nk) sstore(st ^ 1);
    __syncthreads();
  }

  // ------------------------------------------------------------- epilogue
  const int half = lane >> 5;
  const int col = lane & 31;
  const uint32_t below = (1u << col) - 1u;
  const int nT = a.F / kT;
  constexpr int kTilesPerBlock = kBN / kT;     // 1 (T=128) or 2 (T=64)
  constexpr int kBlocksPerTile = 4 / kTilesPerBlock;  // 32-unit blocks per TwELL tile
  const int tile0 = n0 / kT;
  const int wrow0 = m0 + w * 64;
  const int C = a.C;

  if constexpr (kDebug) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wrow0 + mb * 32 + acc_row(v, half);
          const int cg = n0 + nb * 32 + col;
          if (row < a.M && cg < a.F) a.z_debug[static_cast<size_t>(row) * a.F + cg] = acc[mb][nb][v];
        }
  }

  // cnt[tt] of lane L = count of token wrow0 + L in TwELL tile tile0 + tt
  uint32_t cnt[kTilesPerBlock];
#pragma unroll
  for (int tt = 0; tt < kTilesPerBlock; ++tt) cnt[tt] = 0;

#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      uint64_t bal[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) bal[nb] = __ballot(acc[mb][nb][v] > 0.f);
      if ((bal[0] | bal[1] | bal[2] | bal[3]) == 0) continue;  // both tokens inactive here
      const int rl_lo = mb * 32 + acc_row(v, 0);  // token of lanes 0-31; lanes 32-63: +4
      const int row = wrow0 + rl_lo + 4 * half;
      uint32_t mk[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) mk[nb] = half ? static_cast<uint32_t>(bal[nb] >> 32) : static_cast<uint32_t>(bal[nb]);
#pragma unroll
      for (int tt = 0; tt < kTilesPerBlock; ++tt) {
        uint32_t c_lo = 0, c_hi = 0;
#pragma unroll
        for (int q = 0; q < kBlocksPerTile; ++q) {
          c_lo += __popc(static_cast<uint32_t>(bal[tt * kBlocksPerTile + q]));
          c_hi += __popc(static_cast<uint32_t>(bal[tt * kBlocksPerTile + q] >> 32));
        }
        if (lane == rl_lo) cnt[tt] = c_lo;
        if (lane == rl_lo + 4) cnt[tt] = c_hi;
        const int tile = tile0 + tt;
        uint32_t pre = 0;
#pragma unroll
        for (int q = 0; q < kBlocksPerTile; ++q) {
          const int nb = tt * kBlocksPerTile + q;
          const uint32_t slot = pre + __popc(mk[nb] & below);
          if (((mk[nb] >> col) & 1u) && slot < static_cast<uint32_t>(C) && row < a.M && tile < nT) {
            const size_t o = (static_cast<size_t>(row) * nT + tile) * C + slot;
            a.vals[o] = acc[mb][nb][v];
            a.idx[o] = static_cast<uint8_t>(q * 32 + col);
          }
          pre += __popc(mk[nb]);
        }
      }
    }
  }

  // Counts: lane L writes token wrow0 + L; overflow rows join the set.
  uint32_t* flags = a.ctrl + kCtrlBytes / 4;
  {
    const int row = wrow0 + lane;
    if (row < a.M) {
      bool over = false;
#pragma unroll
      for (int tt = 0; tt < kTilesPerBlock; ++tt) {
        if (tile0 + tt < nT) {
          a.counts[static_cast<size_t>(row) * nT + tile0 + tt] = static_cast<uint16_t>(cnt[tt]);
          over |= cnt[tt] > static_cast<uint32_t>(C);
        }
      }
      if (over && atomicExch(&flags[row], 1u) == 0u) {
        const uint32_t pos = atomicAdd(&a.ctrl[0], 1u);
        // pos < M whenever the control block started zeroed, as the API requires
        if (pos < static_cast<uint32_t>(a.M))
          __hip_atomic_store(&a.ovf_rows[pos], row, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }

  // The last workgroup publishes n_ovf and clears the control block.
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    const uint32_t done = atomicAdd(&a.ctrl[1], 1u);
    s_last = (done == static_cast<uint32_t>(gridDim.x) - 1u);
  }
  __syncthreads();
  if (s_last) {
    __threadfence();
    uint32_t n = __hip_atomic_load(&a.ctrl[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    n = min(n, static_cast<uint32_t>(a.M));
    for (uint32_t i = tid; i < n; i += 256) {
      const int r = __hip_atomic_load(&a.ovf_rows[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (r >= 0 && r < a.M) __hip_atomic_store(&flags[r], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid == 0) {
      *a.n_ovf = static_cast<int32_t>(n);
      __hip_atomic_store(&a.ctrl[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.ctrl[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

__global__ void set_i32_kernel(int32_t* p, int32_t v) { *p = v; }

}  // namespace

hipError_t launch_gate_pack(const GateArgs& a, hipStream_t s) {
  const int tiles_m = (a.M + kBM - 1) / kBM;
  const int tiles_n = (a.F + kBN - 1) / kBN;
  const dim3 grid(tiles_m * tiles_n), block(256);
  const bool dbg = a.z_debug != nullptr;
  if (a.T == 128) {
    if (dbg) gate_pack_kernel<128, true><<<grid, block, 0, s>>>(a, tiles_m);
    else gate_pack_kernel<128, false><<<grid, block, 0, s>>>(a, tiles_m);
  } else {
    if (dbg) gate_pack_kernel<64, true><<<grid, block, 0, s>>>(a, tiles_m);
    else gate_pack_kernel<64, false><<<grid, block, 0, s>>>(a, tiles_m);
  }
  return hipGetLastError();
}

hipError_t launch_set_i32(int32_t* p, int32_t v, hipStream_t s) {
  set_i32_kernel<<<1, 1, 0, s>>>(p, v);
  return hipGetLastError();
}

}  // namespace twell
