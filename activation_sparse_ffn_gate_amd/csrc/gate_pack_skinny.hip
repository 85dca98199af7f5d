// Gate GEMM with the TwELL packing in its epilogue, for small batches (decode).
//
// Same operation and outputs as gate_pack.hip (aimodeling.com TwELL summary,
// paragraph 3; pulsen.vercel.app article, paragraph on tile matching; Tencent
// Cloud article, section 2): z = x Wg^T, ReLU, per-(token, tile) counts,
// ascending tile-local indices and fp32 values of the first C active units,
// and the overflow list.
//
// With few tokens the 256 x 256 tiles of the large kernel leave most of the
// chip idle (F / 256 workgroups) and each workgroup streams a megabyte of Wg
// through one pipeline. Here a workgroup covers 32 tokens x 128 units (one
// TwELL tile of 128, or two of 64) with 16 waves: 4 unit groups of 32 x 4
// splits of every K chunk. K advances in 256-value chunks: every wave load
// instruction reads 1 KB contiguous (two rows' 512-byte chunk), three chunks
// are in flight in registers, and each chunk is stored to one of two LDS
// stages (512-byte rows, 16-byte pieces XOR-swizzled by row mod 16) from which
// the MFMA fragments are read. (Loading MFMA fragments straight from memory
// makes every load instruction touch 32 rows, which ran at a fifth of this
// rate.) The K splits meet through LDS in a fixed order.

// With few tokens even 128-unit workgroups are too few to stream Wg at the
// HBM rate (64 of them at F = 8192). Given room for partial sums, the gate
// then runs in two launches: workgroup (tile, q) of the first runs, for the
// four unit groups, exactly the k-steps that wave (unit group, K split q) of
// the single launch runs (a quarter of every chunk) and stores the four
// accumulators; the second is the single-launch kernel with each wave taking
// its accumulator from split q instead of a K loop, then adding the splits in
// the same order. So z, and every packed bit, is the same in both forms.
//
// Packing: per accumulator register a 64-bit ballot of z > 0 gives two tokens'
// activity over the wave's 32 units; the waves of a tile exchange per-token
// counts through LDS, so a unit's slot is the count in lower waves plus its
// rank in its own ballot. Overflow rows join the same deduplicated list as in
// the large kernel, and the last workgroup publishes n_ovf and clears the
// control block.
#include "gate_overflow.hpp"
#include "twell_device.hpp"
#include "twell_internal.hpp"

namespace twell {
namespace {

constexpr int kSN = 128;   // units per workgroup
constexpr int kKS = 4;     // K splits: waves per unit group
constexpr int kWaves = 4 * kKS;

// RB blocks of 32 tokens per workgroup; K chunk of KC values (KC / 8 pieces of
// 16 bytes per row) so that two stages of (128 + 32 RB) rows fit in LDS.
template <int RB>
struct SkinnyShape {
  static constexpr int kSM = 32 * RB;
  static constexpr int kKc = RB == 1 ? 256 : 128;
  static constexpr int kPieces = kKc / 8;
  static constexpr int kRowB = 2 * kKc;
  static constexpr int kRows = kSN + kSM;
  static constexpr int kStageB = kRows * kRowB;
  static constexpr int kLoads = kRows * kPieces / (64 * kWaves);  // 16-byte loads per thread per chunk
  static constexpr int kRedB = (kKS - 1) * 4 * 64 * 16 * RB * 4;
  static constexpr int kLdsB = (2 * kStageB > kRedB + 4 * kSM * 4 + 16) ? 2 * kStageB : kRedB + 4 * kSM * 4 + 16;
  static_assert(kRows * kPieces % (64 * kWaves) == 0, "whole loads per thread");
};

// Byte offset of 16-byte piece p of LDS row r (rows of kRowB bytes): pieces are
// XOR-swizzled with r mod 16, so the 16 rows a ds_read_b128 serves at once fall
// in 16 different bank groups.
template <int kRowB>
__device__ __forceinline__ uint32_t sk_off(int r, int p) {
  return static_cast<uint32_t>(r * kRowB + ((p ^ (r & 15)) << 4));
}

// K chunks (256 values) a split workgroup preloads: d <= 2048 splits.
constexpr int kMaxSplitChunks = 8;

template <int kT, bool kDebug, bool kAct, int RB, bool kFromParts = false>
__global__ __launch_bounds__(64 * kWaves, 1) void gate_pack_skinny_kernel(GateArgs a, int tiles_m) {
  using S = SkinnyShape<RB>;
  constexpr int kSM = S::kSM;
  // One LDS object: two K-chunk stages; after the K loop its first bytes hold
  // the K-split exchange, then the per-wave token counts and the finalize flag.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S::kLdsB];
  float(*s_red)[4][64][16 * RB] = reinterpret_cast<float(*)[4][64][16 * RB]>(smem);
  int(*s_cnt)[kSM] = reinterpret_cast<int(*)[kSM]>(smem + S::kRedB);
  int* s_last = reinterpret_cast<int*>(smem + S::kRedB + 4 * kSM * 4);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = w & 3, kh = w >> 2;  // unit group, K split
  // Tile index: workgroups are dispatched round-robin over the 8 XCDs, and
  // the tiles_m token tiles of one unit tile (consecutive indices) read the
  // same Wg rows, so with several token tiles each XCD takes a contiguous run
  // of indices and those reads meet in its L2 instead of each XCD fetching
  // them again (one token tile shares nothing: dispatch order kept).
  const int nwg = gridDim.x;
  const int tix = (tiles_m > 1 && nwg % 8 == 0) ? (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8 : blockIdx.x;
  const int m0 = (tix % tiles_m) * kSM;
  const int n0 = (tix / tiles_m) * kSN;
  const int r = lane & 31, half = lane >> 5;

  f32x16_t acc[RB];
  if constexpr (kFromParts) {
    // Launched with 4 waves (kh = 0): unit group wn's sums of the K splits,
    // added in split order as the single launch adds its waves' sums (float4s
    // of rows past M were not stored: they read as zero, those rows never count).
    const float4* src = reinterpret_cast<const float4*>(a.kpart) +
                        (static_cast<size_t>(tix) * kKS * 4 + wn) * 64 * 4 * RB + lane * 4 * RB;
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bool live = m0 + 32 * b + 8 * g + 4 * half < a.M;
        float4 v[kKS];
#pragma unroll
        for (int q = 0; q < kKS; ++q)
          v[q] = live ? src[static_cast<size_t>(q) * 4 * 64 * 4 * RB + 4 * b + g] : make_float4(0.f, 0.f, 0.f, 0.f);
        float4 t = v[0];
#pragma unroll
        for (int q = 1; q < kKS; ++q) {
          t.x += v[q].x;
          t.y += v[q].y;
          t.z += v[q].z;
          t.w += v[q].w;
        }
        acc[b][4 * g] = t.x;
        acc[b][4 * g + 1] = t.y;
        acc[b][4 * g + 2] = t.z;
        acc[b][4 * g + 3] = t.w;
      }
  } else {
  // Loads: every wave instruction reads 1 KB contiguous (whole rows' K chunk).
  // Thread tid holds pieces q = tid + 1024 i of the chunk's kRows x kPieces:
  // rows below 128 are Wg rows, the rest x rows. Rows past M or F read a valid
  // row; their results are discarded. Offsets are 32-bit (x and Wg are below
  // 2 GiB, checked by the host).
  const uint32_t row_bytes = static_cast<uint32_t>(a.d) * 2u;
  const char* xb = reinterpret_cast<const char*>(a.x);
  const char* wb = reinterpret_cast<const char*>(a.Wg);
  uint32_t goff[S::kLoads], soff[S::kLoads];
  bool isw[S::kLoads];
#pragma unroll
  for (int i = 0; i < S::kLoads; ++i) {
    const int q = tid + 64 * kWaves * i;
    const int row = q / S::kPieces, piece = q % S::kPieces;
    isw[i] = row < kSN;
    const int grow = isw[i] ? min(n0 + row, a.F - 1) : min(m0 + row - kSN, a.M - 1);
    goff[i] = static_cast<uint32_t>(grow) * row_bytes + static_cast<uint32_t>(piece) * 16u;
    soff[i] = sk_off<S::kRowB>(row, piece);
  }
  struct Regs {
    u32x4_t v[S::kLoads];
  };
  auto gload = [&](Regs& g, int ck) {
    const uint32_t k = static_cast<uint32_t>(ck) * S::kRowB;
#pragma unroll
    for (int i = 0; i < S::kLoads; ++i)
      g.v[i] = *reinterpret_cast<const u32x4_t*>((isw[i] ? wb : xb) + goff[i] + k);
  };
  auto sstore = [&](const Regs& g, int st) {
#pragma unroll
    for (int i = 0; i < S::kLoads; ++i) lds_store16(smem + st * S::kStageB, soff[i], g.v[i]);
  };

  // MFMA: wave (wn, kh) takes units wn*32 .. +31 and a quarter of the chunk's
  // kKc / 16 k-steps; step s uses piece 2s + half of its rows (A: token rows,
  // one accumulator block per 32 tokens; B: unit rows).
  constexpr int kStepsPerWave = S::kKc / 16 / kKS;
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[b][v] = 0.f;
  auto mma = [&](int st) {
    const uint8_t* base = smem + st * S::kStageB;
#pragma unroll
    for (int j = 0; j < kStepsPerWave; ++j) {
      const int p = 2 * (kh * kStepsPerWave + j) + half;
      const u32x4_t bf = lds_load16(base, sk_off<S::kRowB>(wn * 32 + r, p));
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const u32x4_t af = lds_load16(base, sk_off<S::kRowB>(kSN + 32 * b + r, p));
        acc[b] = mfma_32x32x16(af, bf, acc[b]);
      }
    }
  };

  // Three chunks in flight in registers, two LDS stages. Chunk c: wait for its
  // registers, store them to stage c % 2, barrier (every wave is past chunk
  // c - 2's reads of that stage, and chunk c is visible), issue the loads of
  // chunk c + 3, then the products. Loads past the last chunk re-read it
  // (unconditional loads keep the wait counts exact).
  const int nck = a.d / S::kKc;
  Regs g0, g1, g2;
  gload(g0, 0);
  gload(g1, min(1, nck - 1));
  gload(g2, min(2, nck - 1));
  for (int ck = 0; ck < nck; ck += 3) {
    sstore(g0, ck & 1);
    __syncthreads();
    gload(g0, min(ck + 3, nck - 1));
    mma(ck & 1);
    if (ck + 1 < nck) {  // uniform
      sstore(g1, (ck + 1) & 1);
      __syncthreads();
      gload(g1, min(ck + 4, nck - 1));
      mma((ck + 1) & 1);
    }
    if (ck + 2 < nck) {
      sstore(g2, (ck + 2) & 1);
      __syncthreads();
      gload(g2, min(ck + 5, nck - 1));
      mma((ck + 2) & 1);
    }
  }
  }
  __syncthreads();  // every wave is done with the stages

  // K splits: splits 1 .. kKS-1 hand their sums to split 0, which adds them in
  // split order.
  if (kh > 0) {
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) s_red[kh - 1][wn][lane][16 * b + v] = acc[b][v];
  }
  __syncthreads();

  const int nT = a.F / kT;
  const int C = a.C;
  constexpr int kWavesPerTile = kT / 32;     // 4 (T = 128) or 2 (T = 64)
  const int tile = (n0 + wn * 32) / kT;       // this wave's TwELL tile
  const int wt = wn % kWavesPerTile;          // its rank among the tile's waves
  int appended = 0;

  if (kh == 0) {
    if constexpr (!kFromParts) {
#pragma unroll
      for (int j = 0; j < kKS - 1; ++j)
#pragma unroll
        for (int b = 0; b < RB; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[b][v] += s_red[j][wn][lane][16 * b + v];
    }
    const int ucol = n0 + wn * 32 + r;  // this lane's unit
    const bool unit_ok = ucol < a.F;
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + 32 * b + acc_row(v, half);
        const bool ok = unit_ok && row < a.M;
        if constexpr (kDebug) {
          if (ok) a.z_debug[static_cast<size_t>(row) * a.F + ucol] = acc[b][v];
        }
        acc[b][v] = ok ? acc[b][v] : 0.f;  // rows and units past the matrix never count
      }
    // This wave's count of each token, lane t holding token t (t < kSM).
    uint64_t bal[RB][16];
    int cw = 0;
    static_for<0, 16 * RB>([&](auto I) {
      constexpr int b = decltype(I)::value / 16, v = decltype(I)::value % 16;
      bal[b][v] = __ballot(acc[b][v] > 0.f);
      cw = writelane<32 * b + acc_row(v, 0)>(cw, __popc(static_cast<uint32_t>(bal[b][v])));
      cw = writelane<32 * b + acc_row(v, 1)>(cw, __popc(static_cast<uint32_t>(bal[b][v] >> 32)));
    });
    if constexpr (kAct) {  // column activity of the wave's 32 units
      uint64_t any = 0;
#pragma unroll
      for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) any |= bal[b][v];
      const uint32_t word = static_cast<uint32_t>(any) | static_cast<uint32_t>(any >> 32);
      if (word != 0u && lane == 0) atomicOr(&a.col_active[(n0 + wn * 32) >> 5], word);
    }
    if (lane < kSM) s_cnt[wn][lane] = cw;
    __syncthreads();  // (1) counts of every wave
    // Lane t: active units of token t in the tile's lower waves, and in all of them.
    int pre = 0, tot = 0;
    const int wfirst = wn - wt;
#pragma unroll
    for (int j = 0; j < kWavesPerTile; ++j) {
      const int c = s_cnt[wfirst + j][lane % kSM];
      tot += c;
      pre += (j < wt) ? c : 0;
    }
    if (tile < nT) {
      const uint32_t row_slots = static_cast<uint32_t>(nT * C);
      const uint32_t ulocal = static_cast<uint32_t>(wt * 32 + r);  // index inside the tile
      // Uniform skips: registers whose rows all lie past M, and the spill when
      // no token of the tile overflows (the common case).
      const bool spill_any = a.spill != nullptr && __ballot(lane < kSM && tot > C) != 0;
      static_for<0, 16 * RB>([&](auto I) {
        constexpr int b = decltype(I)::value / 16, v = decltype(I)::value % 16;
        constexpr int t_lo = 32 * b + acc_row(v, 0), t_hi = 32 * b + acc_row(v, 1);
        if (m0 + t_lo >= a.M) return;  // t_lo < t_hi: both rows past M
        if (spill_any) {  // every z of a (token, tile) that overflows, active or not
          const int t_own = half ? __builtin_amdgcn_readlane(tot, t_hi) : __builtin_amdgcn_readlane(tot, t_lo);
          const int row = m0 + 32 * b + acc_row(v, half);
          if (t_own > C && row < a.M)
            a.spill[(static_cast<size_t>(row) * nT + tile) * kT + ulocal] = acc[b][v];
        }
        const uint64_t bq = bal[b][v];
        if (bq == 0) return;
        const uint32_t pre_lo = __builtin_amdgcn_readlane(pre, t_lo);
        const uint32_t pre_hi = __builtin_amdgcn_readlane(pre, t_hi);
        const uint32_t rank = half ? __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bq >> 32), 0u)
                                   : __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bq), 0u);
        const uint32_t slot = rank + (half ? pre_hi : pre_lo);
        if (acc[b][v] > 0.f && slot < static_cast<uint32_t>(C)) {
          const uint32_t row = static_cast<uint32_t>(m0 + 32 * b + acc_row(v, half));
          const uint32_t at = row * row_slots + static_cast<uint32_t>(tile * C) + slot;
          store_at(a.vals, at * 4u, acc[b][v]);
          store_at(a.idx, at, static_cast<uint8_t>(ulocal));
        }
      });
      // Counts and overflow membership: the tile's first wave, lane t = token t.
      const int row = m0 + lane;
      if (wt == 0 && lane < kSM && row < a.M) {
        a.counts[static_cast<size_t>(row) * nT + tile] = static_cast<uint16_t>(tot);
        if (tot > C) appended = overflow_append(a, row);
      }
    }
  } else {
    __syncthreads();  // (1)
  }

  overflow_finalize(a, appended, s_last);
}

// First launch of the K split (RB = 1 only): workgroup (tile, q), 4 waves,
// wave wn = unit group wn. Each chunk's quarter q (pieces 8q .. 8q + 7 of its
// 32) is staged in LDS as 128-byte rows, 16-byte pieces XOR-swizzled by
// (row / 2) mod 8 so the 16 rows a ds_read_b128 serves at once fall in 16
// bank groups; the MFMAs are those of wave (wn, kh = q) of the single launch,
// chunk by chunk in the same order.
__global__ __launch_bounds__(256) void gate_skinny_split_kernel(GateArgs a, int tiles_m) {
  using S = SkinnyShape<1>;
  constexpr int kQP = S::kPieces / kKS;  // pieces of a chunk per split: 8
  constexpr int kRowQ = kQP * 16;
  constexpr int kStageQ = S::kRows * kRowQ;
  constexpr int kLoadsQ = S::kRows * kQP / 256;  // 16-byte loads per thread per chunk
  static_assert(S::kRows * kQP % 256 == 0 && kQP == 8, "whole loads per thread");
  constexpr int kStepsPerWave = S::kKc / 16 / kKS;
  static_assert(2 * kStepsPerWave == kQP, "a wave's k-steps cover its quarter");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kStageQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wn = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = blockIdx.x % kKS;
  const int tile = blockIdx.x / kKS;
  const int m0 = (tile % tiles_m) * S::kSM;
  const int n0 = (tile / tiles_m) * kSN;
  const int r = lane & 31, half = lane >> 5;
  auto soff_of = [](int row, int pq) { return static_cast<uint32_t>(row * kRowQ + ((pq ^ ((row >> 1) & 7)) << 4)); };

  // rows below 128 are Wg rows, the rest x rows; rows past M or F read a valid row
  const uint32_t row_bytes = static_cast<uint32_t>(a.d) * 2u;
  const char* xb = reinterpret_cast<const char*>(a.x);
  const char* wb = reinterpret_cast<const char*>(a.Wg);
  uint32_t goff[kLoadsQ], soff[kLoadsQ];
  bool isw[kLoadsQ];
#pragma unroll
  for (int i = 0; i < kLoadsQ; ++i) {
    const int idx = tid + 256 * i;
    const int row = idx / kQP, pq = idx % kQP;
    isw[i] = row < kSN;
    const int grow = isw[i] ? min(n0 + row, a.F - 1) : min(m0 + row - kSN, a.M - 1);
    goff[i] = static_cast<uint32_t>(grow) * row_bytes + static_cast<uint32_t>(q * kQP + pq) * 16u;
    soff[i] = soff_of(row, pq);
  }
  struct Regs {
    u32x4_t v[kLoadsQ];
  };
  auto gload = [&](Regs& g, int ck) {
    const uint32_t k = static_cast<uint32_t>(ck) * S::kRowB;
#pragma unroll
    for (int i = 0; i < kLoadsQ; ++i)
      g.v[i] = *reinterpret_cast<const u32x4_t*>((isw[i] ? wb : xb) + goff[i] + k);
  };
  auto sstore = [&](const Regs& g, int st) {
#pragma unroll
    for (int i = 0; i < kLoadsQ; ++i) lds_store16(smem + st * kStageQ, soff[i], g.v[i]);
  };
  f32x16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  auto mma = [&](int st) {
    const uint8_t* base = smem + st * kStageQ;
#pragma unroll
    for (int j = 0; j < kStepsPerWave; ++j) {
      const int pq = 2 * j + half;  // piece 2 (q kStepsPerWave + j) + half of the chunk
      const u32x4_t bf = lds_load16(base, soff_of(wn * 32 + r, pq));
      const u32x4_t af = lds_load16(base, soff_of(kSN + r, pq));
      acc = mfma_32x32x16(af, bf, acc);
    }
  };
  // Every chunk's loads go out at once (at most kMaxSplitChunks chunks: 40
  // sixteen-byte loads a thread), so the workgroup waits for one memory round
  // trip rather than one every few chunks; chunks then pass through two LDS
  // stages in order.
  const int nck = a.d / S::kKc;
  Regs g[kMaxSplitChunks];
  static_for<0, kMaxSplitChunks>([&](auto I) { gload(g[I.value], min(I.value, nck - 1)); });
  static_for<0, kMaxSplitChunks>([&](auto I) {
    constexpr int ck = I.value;
    if (ck < nck) {  // uniform
      sstore(g[ck], ck & 1);
      __syncthreads();
      mma(ck & 1);
    }
  });
  // the accumulator, float4 g holding rows 8 g + 4 half .. +3 of the tile
  float4* dst = reinterpret_cast<float4*>(a.kpart) + ((static_cast<size_t>(tile) * kKS + q) * 4 + wn) * 64 * 4 + lane * 4;
#pragma unroll
  for (int g = 0; g < 4; ++g)
    if (m0 + 8 * g + 4 * half < a.M) dst[g] = make_float4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
}

template <int RB>
hipError_t launch_rb(const GateArgs& a, hipStream_t s) {
  const int tiles_m = (a.M + 32 * RB - 1) / (32 * RB);
  const int tiles_n = (a.F + kSN - 1) / kSN;
  const dim3 grid(tiles_m * tiles_n), block(64 * kWaves);
  const bool dbg = a.z_debug != nullptr, act = a.col_active != nullptr;
  if (RB == 1 && a.kpart != nullptr && a.kpart_bytes >= skinny_kpart_bytes(a.M, a.d, a.F) &&
      skinny_kpart_bytes(a.M, a.d, a.F) > 0) {
    gate_skinny_split_kernel<<<dim3(tiles_m * tiles_n * kKS), dim3(256), 0, s>>>(a, tiles_m);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 block4(256);  // the unit groups' first waves only (kh = 0)
    if (a.T == 128) {
      if (dbg) gate_pack_skinny_kernel<128, true, false, RB, true><<<grid, block4, 0, s>>>(a, tiles_m);
      else if (act) gate_pack_skinny_kernel<128, false, true, RB, true><<<grid, block4, 0, s>>>(a, tiles_m);
      else gate_pack_skinny_kernel<128, false, false, RB, true><<<grid, block4, 0, s>>>(a, tiles_m);
    } else {
      if (dbg) gate_pack_skinny_kernel<64, true, false, RB, true><<<grid, block4, 0, s>>>(a, tiles_m);
      else if (act) gate_pack_skinny_kernel<64, false, true, RB, true><<<grid, block4, 0, s>>>(a, tiles_m);
      else gate_pack_skinny_kernel<64, false, false, RB, true><<<grid, block4, 0, s>>>(a, tiles_m);
    }
    return hipGetLastError();
  }
  if (a.T == 128) {
    if (dbg) gate_pack_skinny_kernel<128, true, false, RB><<<grid, block, 0, s>>>(a, tiles_m);
    else if (act) gate_pack_skinny_kernel<128, false, true, RB><<<grid, block, 0, s>>>(a, tiles_m);
    else gate_pack_skinny_kernel<128, false, false, RB><<<grid, block, 0, s>>>(a, tiles_m);
  } else {
    if (dbg) gate_pack_skinny_kernel<64, true, false, RB><<<grid, block, 0, s>>>(a, tiles_m);
    else if (act) gate_pack_skinny_kernel<64, false, true, RB><<<grid, block, 0, s>>>(a, tiles_m);
    else gate_pack_skinny_kernel<64, false, false, RB><<<grid, block, 0, s>>>(a, tiles_m);
  }
  return hipGetLastError();
}

}  // namespace

size_t skinny_kpart_bytes(int64_t M, int64_t d, int64_t F) {
  if (M <= 0 || M > kSkinnyRb1MaxM || d > kMaxSplitChunks * SkinnyShape<1>::kKc) return 0;
  const int64_t tiles = ((M + 31) / 32) * ((F + kSN - 1) / kSN);
  if (tiles >= 128) return 0;  // enough workgroups already (measured: splitting 128 was slower)
  return size_t(tiles) * kKS * 4 * 64 * 16 * sizeof(float);
}

hipError_t launch_gate_pack_skinny(const GateArgs& a, hipStream_t s) {
  // 32-token tiles while they already give a few hundred workgroups' worth of
  // parallelism; 64-token tiles (half the re-reads of Wg) above.
  return a.M <= kSkinnyRb1MaxM ? launch_rb<1>(a, s) : launch_rb<2>(a, s);
}

}  // namespace twell
