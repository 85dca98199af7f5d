// Dense gated FFN on the gate kernel's LDS-DMA ring, for gfx950: the dense
// baseline (the dense matmuls the pages compare against: tgviewer.app
// Telegram post, paragraph after "Обучение"), the dense fallback of long
// overflow lists, and the gate-only variant's dense products.
//
// Both products are run as C = A B^T with A and B row-major, K contiguous,
// which is the form the gate kernel's pipeline streams: 256 x 256 output
// elements per workgroup, 4 waves each owning a 128 x 128 quarter in 16
// accumulator blocks of v_mfma_f32_32x32x16_bf16 (256 AGPRs), K in 32-wide
// chunks through a 5-stage LDS ring filled by global_load_lds four chunks
// ahead, with the same pinned order of MFMAs, fragment reads and DMAs.
//
// Gated up: A = x, and the 256 B rows of a tile are 64 Wg rows, the same 64
// units' WuT rows, then the next 64 units' Wg and WuT rows. Wave (wm, wn) then
// holds z of 64 units in its accumulator blocks 0-1 and u of the same units,
// lane for lane, in blocks 2-3, so h = ReLU(z) * u is formed in registers and
// stored as bf16 (rounded to nearest even). A tile covers 256 tokens x 128
// units and reads one x tile for both products.
//
// Down: y = h Wd, and Wd is [F, d] with d contiguous while the MFMA wants 8
// consecutive k (= F) values per lane. The call first writes Wd^T ([d, F],
// 2 F d bytes, about 8 us at the 1.5B shape) into the workspace; the product
// is then A = h, B = Wd^T. When there are fewer output tiles than CUs the K
// range is cut into S splits: split 0 stores into y, split s > 0 into partial
// s of the workspace, and a last launch adds the partials to y in split
// order (the sum order is fixed).
//
// Fallback of long overflow lists (rows that do not fit the sparse block go to
// a dense path: Telegram post, part "Обучение"; Tencent Cloud article,
// section 3): the same two products over the list's rows, read on the device
// (gated up: A rows are the listed tokens' x rows; down: y rows are scattered
// to them), with the hidden kept as a bf16 hi/lo pair and the down product run
// over K = 2F, the hi plane and then the lo plane against the same Wd^T.
// These launches return at once for a list too short to fill the chip
// without splitting K; the register-staged kernels of dense_ffn.hip take it.
//
// Gated up with the TwELL packing of h: the gate-only variant of the forward,
// which the pages do not describe. Their inference path packs the gate output
// g in the gate GEMM's epilogue and gathers one WuT row and one Wd row per
// stored unit (Telegram post on TwELL at tgviewer.app, part "Инференс";
// aimodeling.com summary, paragraph 3). When more units are active the per-
// unit up gathers cost more than a dense up product, so here the up product
// is dense, from the same x tile as the gate, and only the down product
// gathers (one Wd row per stored unit). The active set stays the gate's: a
// unit with z > 0 is stored even where h is zero or negative (the gate decides
// which units are live: Tencent Cloud article, section 1), and z is computed
// exactly as the gate kernel computes it, so counts, slots, tile-local indices
// and the overflow set are those of twell_gate_pack; only the stored value,
// h = ReLU(z) u in fp32, differs. The packing is done from the registers with
// ballots and per-token counts (the two waves of a 128-unit tile add theirs
// through LDS).
#include <algorithm>

#include "gate_overflow.hpp"
#include "twell_device.hpp"
#include "twell_internal.hpp"

namespace twell {
namespace {

constexpr int kRM = 256;  // A rows per workgroup tile
constexpr int kRN = 256;  // B rows per workgroup tile
constexpr int kRK = 32;   // K chunk per LDS stage
constexpr int kRStages = 5;
constexpr int kRAhead = kRStages - 1;
constexpr int kRTileBytes = 256 * kRK * 2;
constexpr int kRStageBytes = 2 * kRTileBytes;
constexpr int kRDma = 8;          // global_load_lds per thread per stage (4 for A, 4 for B)
constexpr int kMinChunks = 8;     // K chunks per split at least (the pipeline's prologue and drain)
constexpr int kCUs = 256;

enum RingMode { kGatedUp = 0, kDown = 1, kGatedUpPack = 2 };

struct RingArgs {
  const uint16_t* a;   // A rows [rows_a, K] (hi/lo down: the hi plane, [rows_a, kwrap])
  const uint16_t* b0;  // B rows [rows_b, K] (gated up: Wg)
  const uint16_t* b1;  // gated up: WuT; down: unused
  int rows_a, rows_b, K;
  int S;               // K splits
  int tiles_m, tiles_n;
  uint16_t* h;         // gated up: h [rows_a, rows_b] bf16 (hi/lo: the hi plane)
  uint16_t* h_lo;      // hi/lo gated up: the lo plane
  const uint16_t* a_lo;  // hi/lo down: the lo plane of A
  int kwrap;           // hi/lo down: F (A and B rows hold F elements, K = 2F)
  float* y;            // down: y [rows_a, rows_b] fp32 (split 0)
  float* part;         // down: partial s at part + (s - 1) * rows_a * rows_b
  // gathering: list i is token rows[i] (A rows of the gated up, y rows of the
  // down), i < *n_rows; nothing is done when *n_rows < min_rows
  const int32_t* rows;
  const int32_t* n_rows;
  int min_rows;
  // gated up with the TwELL packing of h (the gate-only variant): outputs,
  // control block, T and C as for the gate kernel
  GateArgs g;
};

// kGather: rows come from a device-side list (S = 1, tiles_m from its
// length); kHiLo: the hidden is kept as a bf16 pair h ~ hi + lo and the down
// product runs over K = 2F, the hi plane against Wd^T and then the lo plane.
template <int kMode, bool kGather = false, bool kHiLo = false>
__global__ __launch_bounds__(256, 1) void ring_kernel(RingArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kRStages * kRStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;
  constexpr bool kGU = kMode != kDown;  // the B rows interleave Wg and WuT
  constexpr int kTileN = kGU ? 128 : 256;  // output columns per tile

  int R = a.rows_a, tiles_m = a.tiles_m;
  if constexpr (kGather) {
    R = min(max(*a.n_rows, 0), a.rows_a);
    if (R < a.min_rows || R == 0) return;  // the register-staged kernels take this list
    tiles_m = (R + kRM - 1) / kRM;
  }
  // Work item -> (split, tile): splits vary slowest. Each XCD (workgroups
  // b with the same b % 8) takes a contiguous run of items, walked in groups
  // of 8 token tiles, so the tiles an XCD runs at once share A and B rows in
  // its L2. (Gathering, the grid is sized for the longest list and the
  // workgroups past this list's items return.)
  const int tiles = tiles_m * a.tiles_n;
  const int items = tiles * a.S, b = blockIdx.x;
  if (b >= items) return;
  const int lin = (items % 8 == 0) ? (b % 8) * (items / 8) + (b / 8) : b;
  const int sp = lin / tiles;
  const int t = lin - sp * tiles;
  constexpr int kGroupM = 8;
  const int group = t / (kGroupM * a.tiles_n);
  const int gm = min(kGroupM, tiles_m - group * kGroupM);
  const int within = t - group * kGroupM * a.tiles_n;
  const int m0 = (group * kGroupM + within % gm) * kRM;
  const int n0 = (within / gm) * kTileN;

  const int nkt = a.K / kRK;
  const int c0 = sp * nkt / a.S, c1 = (sp + 1) * nkt / a.S;
  const int nk = c1 - c0;

  // DMA addressing as in the gate kernel: wave w fills the 16-row blocks
  // 4w .. 4w+3 of each operand tile; lane l lands on row l / 4 at physical
  // piece l % 4. Rows past the matrix (or the list) read a valid row; their
  // results are discarded. A 32-bit per-lane byte offset from a wave-uniform
  // base.
  const uint32_t row_bytes = static_cast<uint32_t>(kHiLo && kMode == kDown ? a.kwrap : a.K) * 2u;
  uint32_t oa[4], ob[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (w * 4 + i) * 16 + (lane >> 2);
    const uint32_t lp = static_cast<uint32_t>((lane & 3) ^ lds_swz(row)) * 16u;
    int arow = min(m0 + row, R - 1);
    if constexpr (kGather && kGU) arow = a.rows[arow];  // x row of list entry arow
    oa[i] = static_cast<uint32_t>(arow) * row_bytes + lp;
    // gated up: B rows 64g .. 64g+63 are Wg (g even) or WuT (g odd) rows of
    // units n0 + 64 (g / 2) + 0..63, and wave w's blocks all lie in g = w
    const int brow = kGU ? n0 + (w >> 1) * 64 + i * 16 + (lane >> 2) : n0 + row;
    ob[i] = static_cast<uint32_t>(min(brow, a.rows_b - 1)) * row_bytes + lp;
  }
  const char* abase = reinterpret_cast<const char*>(a.a) + static_cast<size_t>(c0) * kRK * 2;
  const char* bbase = reinterpret_cast<const char*>((kGU && (w & 1)) ? a.b1 : a.b0) +
                      static_cast<size_t>(c0) * kRK * 2;
  auto dma = [&](int j, int buf, int k0) {
    uint8_t* st = smem + buf * kRStageBytes + w * 4 * 1024;
    if constexpr (kHiLo && kMode == kDown) {
      // chunks of the second half read the lo plane against the same Wd^T
      // columns (F % 32 == 0: no chunk straddles the two halves)
      const bool lo = k0 >= a.kwrap;
      const int kk = lo ? k0 - a.kwrap : k0;
      const char* ab = lo ? reinterpret_cast<const char*>(a.a_lo) : abase;
      if (j < 4) dma16(reinterpret_cast<const uint16_t*>(ab + kk * 2 + oa[j]), st + j * 1024);
      else dma16(reinterpret_cast<const uint16_t*>(bbase + kk * 2 + ob[j - 4]), st + kRTileBytes + (j - 4) * 1024);
    } else {
      if (j < 4) dma16(reinterpret_cast<const uint16_t*>(abase + k0 * 2 + oa[j]), st + j * 1024);
      else dma16(reinterpret_cast<const uint16_t*>(bbase + k0 * 2 + ob[j - 4]), st + kRTileBytes + (j - 4) * 1024);
    }
  };
  auto issue = [&](int buf, int k0) {
#pragma unroll
    for (int j = 0; j < kRDma; ++j) dma(j, buf, k0);
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mb][nb][v] = 0.f;

  struct Frags {
    u32x4_t a[4], b[4];
  };
  auto load_frags = [&](Frags& f, int buf, int ks) {
    const uint8_t* As = smem + buf * kRStageBytes;
    const uint8_t* Bs = As + kRTileBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f.a[i] = lds_frag(As, wm * 128 + i * 32, ks, lane);
      f.b[i] = lds_frag(Bs, wn * 128 + i * 32, ks, lane);
    }
  };
  // One k step: 16 MFMAs; a fragment read of the next step after each of the
  // first 8, one DMA of a later chunk after every other one of the last 8.
  auto step = [&](auto kDma0, const Frags& cur, Frags& nxt, int nbuf, int nks, int dbuf, int dk0) {
    constexpr int d0 = decltype(kDma0)::value;
    const uint8_t* As = smem + nbuf * kRStageBytes;
    const uint8_t* Bs = As + kRTileBytes;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int mb = i >> 2, nb = i & 3;
      acc[mb][nb] = mfma_32x32x16(cur.a[mb], cur.b[nb], acc[mb][nb]);
      if (i < 8) {
        if (i & 1) nxt.b[i >> 1] = lds_frag(Bs, wn * 128 + (i >> 1) * 32, nks, lane);
        else nxt.a[i >> 1] = lds_frag(As, wm * 128 + (i >> 1) * 32, nks, lane);
      } else if constexpr (d0 >= 0) {
        if ((i & 1) == 0) dma(d0 + ((i - 8) >> 1), dbuf, dk0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma_32x32x16(f.a[mb], f.b[nb], acc[mb][nb]);
  };
  constexpr std::integral_constant<int, -1> no_dma{};
  constexpr std::integral_constant<int, 0> dma_lo{};
  constexpr std::integral_constant<int, 4> dma_hi{};

  // The gate kernel's pipeline (nk >= kMinChunks, checked by the host).
  auto wait_chunks = [](int chunks) {
    if (chunks >= 2) waitcnt<2 * kRDma, 15>();
    else if (chunks == 1) waitcnt<kRDma, 15>();
    else waitcnt<0, 15>();
  };
  static_assert(kRAhead == 4, "the batch split below assumes chunks run four ahead");
#pragma unroll
  for (int s = 0; s < kRAhead - 1; ++s) issue(s, s * kRK);
#pragma unroll
  for (int j = 0; j < 4; ++j) dma(j, kRAhead - 1, (kRAhead - 1) * kRK);
  waitcnt<2 * kRDma + 4, 15>();
  raw_barrier();
  Frags f0, f1;
  load_frags(f0, 0, 0);
  int kt = 0;
  for (; kt < nk - kRAhead; ++kt) {
    step(dma_hi, f0, f1, kt % kRStages, 1, (kt + kRAhead - 1) % kRStages, (kt + kRAhead - 1) * kRK);
    waitcnt<2 * kRDma, 15>();
    raw_barrier();
    step(dma_lo, f1, f0, (kt + 1) % kRStages, 0, (kt + kRAhead) % kRStages, (kt + kRAhead) * kRK);
  }
  step(dma_hi, f0, f1, kt % kRStages, 1, (kt + kRAhead - 1) % kRStages, (kt + kRAhead - 1) * kRK);
  wait_chunks(nk - 2 - kt);
  raw_barrier();
  step(no_dma, f1, f0, (kt + 1) % kRStages, 0, 0, 0);
  for (++kt; kt < nk - 1; ++kt) {
    step(no_dma, f0, f1, kt % kRStages, 1, 0, 0);
    wait_chunks(nk - 2 - kt);
    raw_barrier();
    step(no_dma, f1, f0, (kt + 1) % kRStages, 0, 0, 0);
  }
  step(no_dma, f0, f1, (nk - 1) % kRStages, 1, 0, 0);
  mma(f1);

  // ------------------------------------------------------------- epilogue
  // The tile goes out through the idle ring so every global store is a whole
  // 16-byte piece of a row (a store from the accumulator layout would write
  // 2 or 4 bytes per lane).
  const int half = lane >> 5, col = lane & 31;
  waitcnt<63, 0>();
  raw_barrier();  // every wave is past its last fragment reads of the ring
  if constexpr (kMode == kGatedUp) {
    // h of the 256 x 128 tile as bf16 rows of 128 (+8 padding) units
    // (hi/lo: the lo plane, h - hi rounded to bf16, in a second region)
    constexpr int kHS = 128 + 8;
    constexpr int kPlane = 256 * kHS;
    uint16_t* hs = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 128 + mb * 32 + acc_row(v, half);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const float hv = fmaxf(acc[mb][nb][v], 0.f) * acc[mb][nb + 2][v];
          const uint32_t hi = f32_to_bf16_rne(hv);
          hs[r * kHS + wn * 64 + nb * 32 + col] = static_cast<uint16_t>(hi);
          if constexpr (kHiLo)
            hs[kPlane + r * kHS + wn * 64 + nb * 32 + col] =
                static_cast<uint16_t>(f32_to_bf16_rne(hv - __uint_as_float(hi << 16)));
        }
      }
    waitcnt<63, 0>();
    raw_barrier();
    const int F = a.rows_b;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int piece = i * 256 + tid, r = piece >> 4, p = piece & 15;
      if (m0 + r < R && n0 + p * 8 < F) {
        const size_t o = static_cast<size_t>(m0 + r) * F + n0 + p * 8;
        *reinterpret_cast<u32x4_t*>(a.h + o) = *reinterpret_cast<const u32x4_t*>(hs + r * kHS + p * 8);
        if constexpr (kHiLo)
          *reinterpret_cast<u32x4_t*>(a.h_lo + o) = *reinterpret_cast<const u32x4_t*>(hs + kPlane + r * kHS + p * 8);
      }
    }
  } else if constexpr (kMode == kDown) {
    // y in two passes of 128 rows (the waves with wm == pass write theirs),
    // fp32 rows of 256 (+8 padding) columns
    constexpr int kYS = 256 + 8;
    float* ys = reinterpret_cast<float*>(smem);
    const int d = a.rows_b;
    float* dst = sp == 0 ? a.y : a.part + static_cast<size_t>(sp - 1) * a.rows_a * d;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      if (wm == pass) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = mb * 32 + acc_row(v, half);
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) ys[r * kYS + wn * 128 + nb * 32 + col] = acc[mb][nb][v];
          }
      }
      waitcnt<63, 0>();
      raw_barrier();
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int piece = i * 256 + tid, r = piece >> 6, p = piece & 63;
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(ys + r * kYS + p * 4);
        const int row = m0 + pass * 128 + r;
        if (row < R) {
          const int out = kGather ? a.rows[row] : row;  // gathering: y row of the list entry's token
          *reinterpret_cast<f32x4_t*>(dst + static_cast<size_t>(out) * d + n0 + p * 4) = v;
        }
      }
      waitcnt<63, 0>();
      raw_barrier();  // reads done before the next pass writes
    }
  } else {
    // The gate-only variant's packing, from the registers: z decides which
    // units are stored (the gate's own active set, z computed as the gate
    // kernel computes it), h = ReLU(z) u is the stored value. Wave (wm, wn)
    // holds 128 tokens x 64 units; with T = 128 the wave pair wn = 0, 1 is one
    // tile (wn = 0 first), with T = 64 each wave's units are a tile.
    const GateArgs& g = a.g;
    const int F = a.rows_b;
    const int wrow0 = m0 + wm * 128, ucol0 = n0 + wn * 64;
    // rows and units past the matrix never count
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int c = ucol0 + nb * 32 + col;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wrow0 + mb * 32 + acc_row(v, half);
          const float z = (row < R && c < F) ? acc[mb][nb][v] : 0.f;
          acc[mb][nb][v] = z;
          acc[mb][nb + 2][v] = fmaxf(z, 0.f) * acc[mb][nb + 2][v];
        }
      }
    if (g.z_debug != nullptr) {  // bit-exact checks: every z and h of the tile
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = wrow0 + mb * 32 + acc_row(v, half), c = ucol0 + nb * 32 + col;
            if (row < R && c < F) {
              g.z_debug[static_cast<size_t>(row) * F + c] = acc[mb][nb][v];
              g.h_debug[static_cast<size_t>(row) * F + c] = acc[mb][nb + 2][v];
            }
          }
    }
    // Each token's count in this wave's 64 units: lane t holds token t (cw0)
    // and token 64 + t (cw1).
    int cw0 = 0, cw1 = 0;
    static_for<0, 64>([&](auto I) {
      constexpr int mb = decltype(I)::value / 16, v = decltype(I)::value % 16;
      constexpr int t0 = (mb & 1) * 32 + acc_row(v, 0), t1 = (mb & 1) * 32 + acc_row(v, 1);
      const uint64_t b0 = __ballot(acc[mb][0][v] > 0.f), b1 = __ballot(acc[mb][1][v] > 0.f);
      const int lo = __popc(static_cast<uint32_t>(b0)) + __popc(static_cast<uint32_t>(b1));
      const int hi = __popc(static_cast<uint32_t>(b0 >> 32)) + __popc(static_cast<uint32_t>(b1 >> 32));
      if constexpr (mb < 2) {
        cw0 = writelane<t0>(cw0, lo);
        cw0 = writelane<t1>(cw0, hi);
      } else {
        cw1 = writelane<t0>(cw1, lo);
        cw1 = writelane<t1>(cw1, hi);
      }
    });
    int* s_cnt = reinterpret_cast<int*>(smem);  // [wm][wn][128 tokens]
    int* s_flag = s_cnt + 2 * 2 * 128;
    s_cnt[(wm * 2 + wn) * 128 + lane] = cw0;
    s_cnt[(wm * 2 + wn) * 128 + 64 + lane] = cw1;
    __syncthreads();
    const bool pair = g.T == 128;
    const int* c0 = s_cnt + (wm * 2) * 128;   // the wave pair's wn = 0 counts
    const int* c1 = c0 + 128;                 // ... and wn = 1
    const int pre0 = (pair && wn == 1) ? c0[lane] : 0, pre1 = (pair && wn == 1) ? c0[64 + lane] : 0;
    const int tot0 = pair ? c0[lane] + c1[lane] : cw0, tot1 = pair ? c0[64 + lane] + c1[64 + lane] : cw1;
    const int nT = F / g.T;
    const int tile = pair ? n0 / g.T : ucol0 / g.T;
    const int C = g.C;
    int appended = 0;
    if (tile < nT) {
      const uint32_t row_slots = static_cast<uint32_t>(nT * C);
      const int ubase = pair ? wn * 64 : 0;  // tile-local index of the wave's first unit
      static_for<0, 64>([&](auto I) {
        constexpr int mb = decltype(I)::value / 16, v = decltype(I)::value % 16;
        constexpr int t_lo = (mb & 1) * 32 + acc_row(v, 0), t_hi = (mb & 1) * 32 + acc_row(v, 1);
        const uint64_t b0 = __ballot(acc[mb][0][v] > 0.f), b1 = __ballot(acc[mb][1][v] > 0.f);
        if ((b0 | b1) == 0) return;
        const int pre = mb < 2 ? pre0 : pre1;
        const uint32_t p = half ? static_cast<uint32_t>(__builtin_amdgcn_readlane(pre, t_hi))
                                : static_cast<uint32_t>(__builtin_amdgcn_readlane(pre, t_lo));
        const uint32_t row = static_cast<uint32_t>(wrow0 + mb * 32 + acc_row(v, half));
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const uint64_t bq = nb ? b1 : b0;
          if (bq == 0) continue;
          // slot: active units left of this one in the token's tile
          uint32_t rank = half ? __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bq >> 32), 0u)
                               : __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bq), 0u);
          if (nb == 1) rank += half ? __popc(static_cast<uint32_t>(b0 >> 32)) : __popc(static_cast<uint32_t>(b0));
          const uint32_t slot = rank + p;
          if (acc[mb][nb][v] > 0.f && slot < static_cast<uint32_t>(C)) {
            const uint32_t at = row * row_slots + static_cast<uint32_t>(tile * C) + slot;
            store_at(g.vals, at * 4u, acc[mb][nb + 2][v]);
            store_at(g.idx, at, static_cast<uint8_t>(ubase + nb * 32 + col));
          }
        }
      });
      // counts and overflow membership: the tile's first wave, lane t =
      // tokens t and 64 + t of the wave's rows
      if (!pair || wn == 0) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int row = wrow0 + hh * 64 + lane, tot = hh ? tot1 : tot0;
          if (row < R) {
            g.counts[static_cast<size_t>(row) * nT + tile] = static_cast<uint16_t>(tot);
            if (tot > C) appended |= overflow_append(g, row);
          }
        }
      }
    }
    overflow_finalize(g, appended, s_flag);
  }
}

// dst [cols, rows] = src [rows, cols]^T for bf16, 64 x 64 tiles through LDS
// (rows and cols multiples of 64). Thread t loads 8 columns of the row pair
// 2 (t / 8), 2 (t / 8) + 1 and writes each column's two values as one 32-bit
// word of the transposed tile, so a 16-byte read there is 8 consecutive rows
// of one column.
// With n_rows set, nothing is done when *n_rows < min_rows.
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ src,
                                                        uint16_t* __restrict__ dst, int rows, int cols,
                                                        const int32_t* n_rows, int min_rows) {
  if (n_rows != nullptr && *n_rows < min_rows) return;
  constexpr int kTS = 32 + 4;  // 32-bit words per transposed row (16-byte aligned)
  __shared__ __attribute__((aligned(16))) uint32_t tt[64 * kTS];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  {
    const int rp = tid >> 3, q = tid & 7;
    const u32x4_t lo = gload16(src + static_cast<size_t>(r0 + 2 * rp) * cols + c0 + q * 8);
    const u32x4_t hi = gload16(src + static_cast<size_t>(r0 + 2 * rp + 1) * cols + c0 + q * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tt[(q * 8 + 2 * e) * kTS + rp] = (lo[e] & 0xFFFFu) | (hi[e] << 16);
      tt[(q * 8 + 2 * e + 1) * kTS + rp] = (lo[e] >> 16) | (hi[e] & 0xFFFF0000u);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = tid + 256 * i, c = p >> 3, g = p & 7;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&tt[c * kTS + g * 4]);
    *reinterpret_cast<u32x4_t*>(dst + static_cast<size_t>(c0 + c) * rows + r0 + g * 8) = v;
  }
}

// y += partial 1, then partial 2, ... (S - 1 partials of n floats; n % 4 == 0).
// Four float4 per thread, all loaded before any is stored.
__global__ __launch_bounds__(256) void add_partials_kernel(float* __restrict__ y, const float* __restrict__ part,
                                                           int64_t n, int S) {
  const int64_t n4 = n / 4;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * 1024 + threadIdx.x;
  float4 v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t i = i0 + 256 * j;
    v[j] = i < n4 ? reinterpret_cast<const float4*>(y)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int s = 1; s < S; ++s) {
    const float4* ps = reinterpret_cast<const float4*>(part + static_cast<size_t>(s - 1) * n);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t i = i0 + 256 * j;
      if (i < n4) {
        const float4 p = ps[i];
        v[j].x += p.x;
        v[j].y += p.y;
        v[j].z += p.z;
        v[j].w += p.w;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t i = i0 + 256 * j;
    if (i < n4) reinterpret_cast<float4*>(y)[i] = v[j];
  }
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

int dense_ring_splits(int64_t M, int64_t d, int64_t F) {
  const int64_t tiles = ceil_div(M, kRM) * (d / kRN);
  const int64_t by_k = (F / kRK) / kMinChunks;
  int64_t S = tiles >= kCUs ? 1 : kCUs / tiles;
  S = std::min<int64_t>(S, by_k);
  return static_cast<int>(std::max<int64_t>(S, 1));
}

bool dense_ring_supports(int64_t M, int64_t d, int64_t F) {
  const int64_t lim = int64_t(1) << 31;  // 32-bit per-lane byte offsets
  return M >= 1 && d % kRN == 0 && d / kRK >= kMinChunks && F % 64 == 0 && F / kRK >= kMinChunks &&
         M * d * 2 < lim && F * d * 2 < lim && M * F * 2 < lim;
}

size_t dense_ring_bytes(int64_t M, int64_t d, int64_t F) {
  const size_t wdt = align256(size_t(F) * size_t(d) * 2);
  return wdt + align256(size_t(dense_ring_splits(M, d, F) - 1) * size_t(M) * size_t(d) * 4);
}

hipError_t launch_dense_ring(const DenseArgs& da, void* ring_ws, hipStream_t s) {
  const int M = da.M, d = da.d, F = da.F;
  uint16_t* wdt = static_cast<uint16_t*>(ring_ws);
  float* part = reinterpret_cast<float*>(static_cast<uint8_t*>(ring_ws) + align256(size_t(F) * size_t(d) * 2));

  transpose_kernel<<<dim3(F / 64, d / 64), dim3(256), 0, s>>>(da.Wd, wdt, F, d, nullptr, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  RingArgs up{};
  up.a = da.x;
  up.b0 = da.Wg;
  up.b1 = da.WuT;
  up.rows_a = M;
  up.rows_b = F;
  up.K = d;
  up.S = 1;
  up.tiles_m = static_cast<int>(ceil_div(M, kRM));
  up.tiles_n = static_cast<int>(ceil_div(F, 128));
  up.h = da.h_hi;
  ring_kernel<kGatedUp><<<dim3(up.tiles_m * up.tiles_n), dim3(256), 0, s>>>(up);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  RingArgs dn{};
  dn.a = da.h_hi;
  dn.b0 = wdt;
  dn.b1 = wdt;
  dn.rows_a = M;
  dn.rows_b = d;
  dn.K = F;
  dn.S = dense_ring_splits(M, d, F);
  dn.tiles_m = up.tiles_m;
  dn.tiles_n = d / kRN;
  dn.y = da.y;
  dn.part = part;
  ring_kernel<kDown><<<dim3(dn.tiles_m * dn.tiles_n * dn.S), dim3(256), 0, s>>>(dn);
  e = hipGetLastError();
  if (e != hipSuccess || dn.S == 1) return e;
  const int64_t n = int64_t(M) * d;
  add_partials_kernel<<<dim3(static_cast<unsigned>(ceil_div(n / 4, 1024))), dim3(256), 0, s>>>(da.y, part, n, dn.S);
  return hipGetLastError();
}

// ------------------------------------------------------------------ fallback
int dense_ring_fallback_min_rows(int64_t d) {
  const int64_t across = d / kRN;  // down tiles across d
  const int64_t tiles_m = (kCUs + across - 1) / across;
  return static_cast<int>((tiles_m - 1) * kRM + 1);
}

bool dense_ring_fallback_possible(int64_t M, int64_t d, int64_t F) {
  return dense_ring_supports(M, d, F) && M >= dense_ring_fallback_min_rows(d);
}

size_t dense_ring_fallback_bytes(int64_t d, int64_t F) { return align256(size_t(F) * size_t(d) * 2); }

hipError_t launch_ring_fallback_up(const DenseArgs& da, hipStream_t s) {
  const int M = da.M, d = da.d, F = da.F;
  uint16_t* wdt = static_cast<uint16_t*>(da.ring_ws);
  transpose_kernel<<<dim3(F / 64, d / 64), dim3(256), 0, s>>>(da.Wd, wdt, F, d, da.n_rows, da.ring_min_rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  RingArgs up{};
  up.a = da.x;
  up.b0 = da.Wg;
  up.b1 = da.WuT;
  up.rows_a = M;
  up.rows_b = F;
  up.K = d;
  up.S = 1;
  up.tiles_m = static_cast<int>(ceil_div(M, kRM));
  up.tiles_n = static_cast<int>(ceil_div(F, 128));
  up.h = da.h_hi;
  up.h_lo = da.h_lo;
  up.rows = da.rows;
  up.n_rows = da.n_rows;
  up.min_rows = da.ring_min_rows;
  ring_kernel<kGatedUp, true, true><<<dim3(up.tiles_m * up.tiles_n), dim3(256), 0, s>>>(up);
  return hipGetLastError();
}

hipError_t launch_ring_fallback_down(const DenseArgs& da, hipStream_t s) {
  const int M = da.M, d = da.d, F = da.F;
  const uint16_t* wdt = static_cast<const uint16_t*>(da.ring_ws);
  RingArgs dn{};
  dn.a = da.h_hi;
  dn.a_lo = da.h_lo;
  dn.kwrap = F;
  dn.b0 = wdt;
  dn.b1 = wdt;
  dn.rows_a = M;
  dn.rows_b = d;
  dn.K = 2 * F;
  dn.S = 1;
  dn.tiles_m = static_cast<int>(ceil_div(M, kRM));
  dn.tiles_n = d / kRN;
  dn.y = da.y;
  dn.rows = da.rows;
  dn.n_rows = da.n_rows;
  dn.min_rows = da.ring_min_rows;
  ring_kernel<kDown, true, true><<<dim3(dn.tiles_m * dn.tiles_n), dim3(256), 0, s>>>(dn);
  return hipGetLastError();
}

// ---------------------------------------------------------- gate-only variant
hipError_t launch_gateup_pack(const GateArgs& a, hipStream_t s) {
  if (a.WuT == nullptr || (a.z_debug == nullptr) != (a.h_debug == nullptr)) return hipErrorInvalidValue;
  if (a.d % kRN != 0 || a.d / kRK < kMinChunks) return hipErrorInvalidValue;
  RingArgs up{};
  up.a = a.x;
  up.b0 = a.Wg;
  up.b1 = a.WuT;
  up.rows_a = a.M;
  up.rows_b = a.F;
  up.K = a.d;
  up.S = 1;
  up.tiles_m = static_cast<int>(ceil_div(a.M, kRM));
  up.tiles_n = static_cast<int>(ceil_div(a.F, 128));
  up.g = a;
  ring_kernel<kGatedUpPack><<<dim3(up.tiles_m * up.tiles_n), dim3(256), 0, s>>>(up);
  return hipGetLastError();
}

}  // namespace twell
