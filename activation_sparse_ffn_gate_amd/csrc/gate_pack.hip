// Gate GEMM with the TwELL packing in its epilogue, for gfx950.
//
// The pages' design (aimodeling.com TwELL summary, paragraph 3; pulsen.vercel.app
// article, paragraph on tile matching; Tencent Cloud article, section 2): the
// TwELL tile width equals the gate matmul's column tile, so the kernel that
// computes a tile of z = x Wg^T can pack its non-zeros right away: no second
// launch, no synchronisation between workgroups, no dense z in memory.
//
// MI355X mapping. One workgroup (4 waves, one per SIMD) computes a 256-token x
// 256-unit tile with v_mfma_f32_32x32x16_bf16; each wave owns a 128 x 128
// quarter (16 accumulator blocks, kept in the AGPRs). K advances in 32-wide
// chunks through a 5-stage LDS ring filled by gfx950's global_load_lds (16
// bytes per lane straight into LDS, no register staging), issued four chunks
// ahead so HBM/MALL latency hides behind the MFMAs. Small batches use
// gate_pack_skinny.hip instead (see launch_gate_pack).
//
// Packing. The finished tile is staged through the idle LDS ring, 128 token
// rows at a time: the two waves that own those rows write their
// accumulators, then every thread takes one (token, 128 units) segment and
// builds its activity mask with plain compares (unit c at bit c), so the
// per-tile count is a popcount and the stored slots are the first C set bits
// in ascending unit order, each found with a count-trailing-zeros. Only slots
// < C are stored (fp32 value, tile-local index); the count is stored
// unclamped. The training instance also copies all T z of each overflowing
// (token, tile) into a spill record. The column-activity instance packs
// nothing: per 32-unit block it ORs the ballots of z > 0 over its tokens.
//
// Overflow rows (some tile count > C) are appended to a deduplicated list with
// device-scope atomics. The last workgroup to finish publishes the list length
// and clears the dedup flags, so the control block is zero again when the
// kernel ends and no separate clearing launch is needed.
#include "gate_overflow.hpp"
#include "twell_device.hpp"
#include "twell_internal.hpp"

namespace twell {
namespace {

constexpr int kBM = 256;     // tokens per workgroup tile
constexpr int kBN = 256;     // hidden units per workgroup tile
constexpr int kBK = 32;      // K chunk per LDS stage
constexpr int kStages = 5;   // LDS ring depth (5 x 32 KB = all 160 KB of LDS)
constexpr int kAhead = kStages - 1;  // chunks in flight ahead of the one computed
constexpr int kTileBytes = 256 * kBK * 2;  // one operand tile of a stage (16 KB)
constexpr int kStageBytes = 2 * kTileBytes;
constexpr int kDmaPerStage = 8;  // global_load_lds per thread per stage (4 for A, 4 for B)

// m * 2 + (z > 0): the compare sets VCC per lane (strict: +0, -0 and NaN
// give 0) and an add with carry-in shifts that bit in.
__device__ __forceinline__ uint32_t shift_in_active(uint32_t m, float z) {
  asm("v_cmp_lt_f32_e32 vcc, 0, %1\n\tv_addc_co_u32_e32 %0, vcc, %0, %0, vcc" : "+v"(m) : "v"(z) : "vcc");
  return m;
}

template <int kT, bool kDebug, bool kAct, bool kSpill = false>
__global__ __launch_bounds__(256, 1) void gate_pack_kernel(GateArgs a, int tiles_m, int tiles_n) {
  // One LDS object only: with a second one the compiler attaches alias scopes
  // to LDS accesses and then makes every LDS read wait for all outstanding
  // DMA, which would drain the pipeline below.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = w >> 1, wn = w & 1;

  // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
  // contiguous run of tile indices, and walk tiles in groups of 8 token tiles
  // (unit tiles within a group), so the tiles an XCD runs at once form a
  // compact block that shares x and Wg slices in its L2.
  const int nwg = gridDim.x, b = blockIdx.x;
  const int lin = (nwg % 8 == 0) ? (b % 8) * (nwg / 8) + (b / 8) : b;
  constexpr int kGroupM = 8;
  const int group = lin / (kGroupM * tiles_n);
  const int gm = min(kGroupM, tiles_m - group * kGroupM);  // token tiles in this group
  const int within = lin - group * kGroupM * tiles_n;
  const int m0 = (group * kGroupM + within % gm) * kBM;
  const int n0 = (within / gm) * kBN;

  // DMA addressing. A stage tile is 256 rows x 64 bytes; wave w fills the
  // 16-row blocks 4w .. 4w+3 of each operand. In a block, lane l lands on row
  // l / 4 at physical piece l % 4, which holds logical piece
  // (l % 4) ^ lds_swz(row) of the swizzled layout (see lds_off). Rows past M
  // or F read a valid row instead: their results are discarded. Addresses are
  // a wave-uniform base plus a 32-bit per-lane byte offset (x and Wg are
  // below 2 GiB, checked by the host).
  uint32_t oa[4], ob[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (w * 4 + i) * 16 + (lane >> 2);
    const uint32_t lp = static_cast<uint32_t>((lane & 3) ^ lds_swz(row)) * 16u;
    oa[i] = static_cast<uint32_t>(min(m0 + row, a.M - 1)) * static_cast<uint32_t>(a.d * 2) + lp;
    ob[i] = static_cast<uint32_t>(min(n0 + row, a.F - 1)) * static_cast<uint32_t>(a.d * 2) + lp;
  }
  const char* xbase = reinterpret_cast<const char*>(a.x);
  const char* wbase = reinterpret_cast<const char*>(a.Wg);
  // DMA j (0..7) of the batch filling buffer `buf` with chunk k0: j < 4 are
  // the wave's A blocks, j >= 4 its B blocks.
  auto dma = [&](int j, int buf, int k0) {
    uint8_t* st = smem + buf * kStageBytes + w * 4 * 1024;
    if (j < 4) dma16(reinterpret_cast<const uint16_t*>(xbase + k0 * 2 + oa[j]), st + j * 1024);
    else dma16(reinterpret_cast<const uint16_t*>(wbase + k0 * 2 + ob[j - 4]), st + kTileBytes + (j - 4) * 1024);
  };
  auto issue = [&](int buf, int k0) {
#pragma unroll
    for (int j = 0; j < kDmaPerStage; ++j) dma(j, buf, k0);
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mb][nb][v] = 0.f;

  // MFMA operands of one 16-wide k step: 4 A and 4 B fragments.
  struct Frags {
    u32x4_t a[4], b[4];
  };
  auto load_frags = [&](Frags& f, int buf, int ks) {
    const uint8_t* As = smem + buf * kStageBytes;
    const uint8_t* Bs = As + kTileBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f.a[i] = lds_frag(As, wm * 128 + i * 32, ks, lane);
      f.b[i] = lds_frag(Bs, wn * 128 + i * 32, ks, lane);
    }
  };
  // One k step: the 16 MFMAs of `cur`; after each of the first 8 one fragment
  // read of the next step (into `nxt`, buffer nbuf, half nks); after every
  // other one of the last 8, one DMA (kDma0 .. kDma0 + 3, when kDma0 >= 0) of
  // the batch for chunk dk0 into buffer dbuf. The order is pinned so the
  // matrix pipe never waits behind an issue block, and each chunk's 32 DMAs
  // per CU are spread over the whole chunk rather than queued at once.
  auto step = [&](auto kDma0, const Frags& cur, Frags& nxt, int nbuf, int nks, int dbuf, int dk0) {
    constexpr int d0 = decltype(kDma0)::value;
    const uint8_t* As = smem + nbuf * kStageBytes;
    const uint8_t* Bs = As + kTileBytes;
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
  constexpr std::integral_constant<int, 0> dma_lo{};  // DMAs 0-3 of a batch
  constexpr std::integral_constant<int, 4> dma_hi{};  // DMAs 4-7 of a batch

  // Pipeline (nk >= 8 since d >= 256). Chunk kt's two k steps run from
  // registers f0 / f1 while the next step's fragments load. Halfway through
  // chunk kt every thread waits until its DMA of chunk kt + 1 has landed
  // (chunks kt + 2 and kt + 3 may stay in flight); the barrier then publishes
  // chunk kt + 1 and guarantees all waves are done with chunk kt - 1, whose
  // buffer chunk kt + kAhead reuses: its DMAs 0-3 go out after this barrier,
  // 4-7 in the first half of the next chunk (before the next wait). Fragment
  // reads never need waiting on at the barrier: the MFMAs that consumed them
  // already waited.
  const int nk = a.d / kBK;
  // vmcnt allowing `chunks` later whole chunks (kDmaPerStage each) in flight
  auto wait_chunks = [](int chunks) {
    if (chunks >= 2) waitcnt<2 * kDmaPerStage, 15>();
    else if (chunks == 1) waitcnt<kDmaPerStage, 15>();
    else waitcnt<0, 15>();
  };
  static_assert(kAhead == 4, "the batch split below assumes chunks run four ahead");
#pragma unroll
  for (int s = 0; s < kAhead - 1; ++s) issue(s, s * kBK);
#pragma unroll
  for (int j = 0; j < 4; ++j) dma(j, kAhead - 1, (kAhead - 1) * kBK);  // chunk 3, first half
  waitcnt<2 * kDmaPerStage + 4, 15>();  // chunk 0 landed
  raw_barrier();
  Frags f0, f1;
  load_frags(f0, 0, 0);
  int kt = 0;
  for (; kt < nk - kAhead; ++kt) {  // steady state
    step(dma_hi, f0, f1, kt % kStages, 1, (kt + kAhead - 1) % kStages, (kt + kAhead - 1) * kBK);
    waitcnt<2 * kDmaPerStage, 15>();
    raw_barrier();
    step(dma_lo, f1, f0, (kt + 1) % kStages, 0, (kt + kAhead) % kStages, (kt + kAhead) * kBK);
  }
  // first drain iteration still completes the last chunk's batch
  step(dma_hi, f0, f1, kt % kStages, 1, (kt + kAhead - 1) % kStages, (kt + kAhead - 1) * kBK);
  wait_chunks(nk - 2 - kt);
  raw_barrier();
  step(no_dma, f1, f0, (kt + 1) % kStages, 0, 0, 0);
  for (++kt; kt < nk - 1; ++kt) {
    step(no_dma, f0, f1, kt % kStages, 1, 0, 0);
    wait_chunks(nk - 2 - kt);
    raw_barrier();
    step(no_dma, f1, f0, (kt + 1) % kStages, 0, 0, 0);
  }
  step(no_dma, f0, f1, (nk - 1) % kStages, 1, 0, 0);
  mma(f1);

  // ------------------------------------------------------------- epilogue
  const int half = lane >> 5;
  const int col = lane & 31;
  const int nT = a.F / kT;
  constexpr int kTilesPerWave = 128 / kT;            // 1 (T=128) or 2 (T=64)
  constexpr int kBlocksPerTile = 4 / kTilesPerWave;  // 32-unit blocks per TwELL tile
  const int wcol0 = n0 + wn * 128;
  const int tile0 = wcol0 / kT;
  const int wrow0 = m0 + wm * 128;
  const int C = a.C;
  const uint32_t row_slots = static_cast<uint32_t>(nT * C);  // slots per token

  if constexpr (kDebug) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wrow0 + mb * 32 + acc_row(v, half);
          const int cg = wcol0 + nb * 32 + col;
          if (row < a.M && cg < a.F) a.z_debug[static_cast<size_t>(row) * a.F + cg] = acc[mb][nb][v];
        }
  }

  // Tokens past M (only in the last row of tiles) must not count or pack.
  if (wrow0 + 128 > a.M) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const bool ok = wrow0 + mb * 32 + acc_row(v, half) < a.M;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb][v] = ok ? acc[mb][nb][v] : 0.f;
      }
  }

  if constexpr (kAct) {
    // Column activity only (its packing would be thrown away): per 32-unit
    // block the OR over the wave's tokens of the ballots of z > 0, one atomic
    // OR per block. No packing, so no overflow set and no finalize.
    uint64_t act[4] = {0, 0, 0, 0};
    static_for<0, 64>([&](auto g) {
      constexpr int mb = decltype(g)::value / 16, v = decltype(g)::value % 16;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) act[nb] |= __ballot(acc[mb][nb][v] > 0.f);
    });
    // both halves of a ballot hold the same 32 units, for two tokens; blocks
    // past the last tile are skipped
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const uint32_t word = static_cast<uint32_t>(act[nb]) | static_cast<uint32_t>(act[nb] >> 32);
      if (tile0 + nb / kBlocksPerTile < nT && word != 0u && lane == 0)
        atomicOr(&a.col_active[(wcol0 >> 5) + nb], word);
    }
    return;
  } else {
    // Packing through LDS. The ring is idle after the K loop; each of two
    // passes holds the 128 token rows of one half of the tile (row-major, rows
    // padded by 4 floats so the column reads below fall in distinct banks).
    // Every thread then packs one (token, 128 units) on its own: a 128-bit
    // activity mask from plain compares, its popcounts, and the first C
    // active units in ascending order. No cross-lane or scalar step.
    constexpr int kZS = kBN + 4;
    constexpr int kTilesPerThread = 128 / kT;
    constexpr int kWordsPerTile = kT / 32;
    float* zs = reinterpret_cast<float*>(smem);
    // the low 32 bits of an LDS object's generic address are its LDS offset
    const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));
    const int t = threadIdx.x;
    const int r_loc = t & 127, th = t >> 7;
    int appended = 0;
    waitcnt<63, 0>();
    raw_barrier();  // every wave is past its last fragment reads of the ring
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      if (wm == pass) {
        // ds_write_b32 straight from the accumulator registers, at immediate
        // offsets from two bases (rows 0-63 and 64-127 of the pass), so no
        // copies and no address arithmetic per value.
        const uint32_t b0 = lds_base + static_cast<uint32_t>((acc_row(0, half) * kZS + wn * 128 + col) * 4);
        const uint32_t b1 = b0 + 64u * kZS * 4u;
        static_for<0, 256>([&](auto I) {
          constexpr int mb = I.value / 64, nb = (I.value / 16) % 4, v = I.value % 16;
          constexpr int off = (((mb & 1) * 32 + 8 * (v / 4) + (v % 4)) * kZS + nb * 32) * 4;
          static_assert(off < 65536, "ds offset");
          const uint32_t base = mb < 2 ? b0 : b1;
          const float val = acc[mb][nb][v];
          asm volatile("ds_write_b32 %0, %1 offset:%2" ::"v"(base), "a"(val), "i"(off) : "memory");
        });
      }
      waitcnt<63, 0>();
      raw_barrier();  // the pass's rows are in LDS
      const float* zr = zs + r_loc * kZS + th * 128;
      uint32_t m[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // shift-in from the highest unit down: unit c ends at bit c
        uint32_t mw = 0;
#pragma unroll
        for (int q = 7; q >= 0; --q) {
          const float4 z4 = *reinterpret_cast<const float4*>(zr + w * 32 + 4 * q);
          mw = shift_in_active(mw, z4.w);
          mw = shift_in_active(mw, z4.z);
          mw = shift_in_active(mw, z4.y);
          mw = shift_in_active(mw, z4.x);
        }
        m[w] = mw;
      }
      const int token = m0 + pass * 128 + r_loc;
#pragma unroll
      for (int k = 0; k < kTilesPerThread; ++k) {
        const int tile = (n0 + th * 128) / kT + k;
        const bool valid = token < a.M && tile < nT;
        int cnt = 0;
#pragma unroll
        for (int w = 0; w < kWordsPerTile; ++w) cnt += __popc(m[k * kWordsPerTile + w]);
        if constexpr (kSpill) {
          // Every z of an overflowing (token, tile) goes to a spill record. The
          // wave takes its records with one atomic; lanes number theirs by
          // rank. The slot map names the record even past the list's
          // capacity, so readers see that it was not stored.
          const bool ov = valid && cnt > C;
          const uint64_t bal = __ballot(ov);
          if (bal != 0u) {  // wave-uniform
            const int first = __builtin_ctzll(bal);
            int rec0 = 0;
            if (lane == first) rec0 = atomicAdd(reinterpret_cast<int*>(a.ctrl + 2), __popcll(bal));
            rec0 = __builtin_amdgcn_readlane(rec0, first);
            if (ov) {
              const int rec = rec0 + static_cast<int>(mask_rank(bal));
              a.rec_slot[static_cast<size_t>(token) * nT + tile] = rec;
              if (rec < a.rec_cap) {
                float4* rz = reinterpret_cast<float4*>(a.rec_z + static_cast<size_t>(rec) * kT);
                const float4* src = reinterpret_cast<const float4*>(zr + k * kT);
#pragma unroll
                for (int q = 0; q < kT / 4; ++q) rz[q] = src[q];
              }
            }
          }
        }
        if (valid) {
          a.counts[static_cast<size_t>(token) * nT + tile] = static_cast<uint16_t>(cnt);
          if (cnt > C) appended |= overflow_append(a, token);
          const uint32_t base = static_cast<uint32_t>(token) * row_slots + static_cast<uint32_t>(tile * C);
          int slot = 0;
#pragma unroll
          for (int w = 0; w < kWordsPerTile; ++w) {
            uint32_t mask = m[k * kWordsPerTile + w];
            while (mask != 0u && slot < C) {
              const int b = __builtin_ctz(mask);
              const int c = w * 32 + b;  // tile-local unit
              store_at(a.vals, (base + slot) * 4u, zr[k * kT + c]);
              store_at(a.idx, base + slot, static_cast<uint8_t>(c));
              ++slot;
              mask &= mask - 1u;
            }
          }
        }
      }
      waitcnt<63, 0>();
      raw_barrier();  // every thread is done reading before the next pass writes
    }
    // Only overflow-list appends take the release fence: nothing in this
    // kernel reads the spill records (the launch boundary publishes them),
    // and the record counter is an atomic whose returned value every wave
    // has used before the workgroup arrives, so the last arrival reads it
    // whole. (Fencing every spilling wave cost 40% of the layer's gate time
    // on the heavy-tailed layer: each fence writes back the XCD's L2.)
    overflow_finalize(a, appended, reinterpret_cast<int*>(smem));
  }
}

__global__ void set_i32_kernel(int32_t* p, int32_t v) { *p = v; }

}  // namespace

hipError_t launch_gate_pack(const GateArgs& a, hipStream_t s) {
  const bool rec = a.rec_z != nullptr;  // spill records: the large kernel at every M
  if (a.M <= kSkinnyMaxM && !rec) return launch_gate_pack_skinny(a, s);
  if (a.spill != nullptr) return hipErrorInvalidValue;  // only the small-batch kernel spills whole rows
  const int tiles_m = (a.M + kBM - 1) / kBM;
  const int tiles_n = (a.F + kBN - 1) / kBN;
  const dim3 grid(tiles_m * tiles_n), block(256);
  const bool dbg = a.z_debug != nullptr, act = a.col_active != nullptr;
  if (rec) {
    if (act || a.rec_slot == nullptr || a.rec_n == nullptr) return hipErrorInvalidValue;
    if (a.T == 128) {
      if (dbg) gate_pack_kernel<128, true, false, true><<<grid, block, 0, s>>>(a, tiles_m, tiles_n);
      else gate_pack_kernel<128, false, false, true><<<grid, block, 0, s>>>(a, tiles_m, tiles_n);
    } else {
      if (dbg) gate_pack_kernel<64, true, false, true><<<grid, block, 0, s>>>(a, tiles_m, tiles_n);
      else gate_pack_kernel<64, false, false, true><<<grid, block, 0, s>>>(a, tiles_m, tiles_n);
    }
    return hipGetLastError();
  }
  if (a.T == 128) {
    if (dbg) gate_pack_kernel<128, true, false><<<grid, block, 0, s>>>(a, tiles_m, tiles_n);
    else if (act) gate_pack_kernel<128, false, true><<<grid, block, 0, s>>>(a, tiles_m, tiles_n);
    else gate_pack_kernel<128, false, false><<<grid, block, 0, s>>>(a, tiles_m, tiles_n);
  } else {
    if (dbg) gate_pack_kernel<64, true, false><<<grid, block, 0, s>>>(a, tiles_m, tiles_n);
    else if (act) gate_pack_kernel<64, false, true><<<grid, block, 0, s>>>(a, tiles_m, tiles_n);
    else gate_pack_kernel<64, false, false><<<grid, block, 0, s>>>(a, tiles_m, tiles_n);
  }
  return hipGetLastError();
}

hipError_t launch_set_i32(int32_t* p, int32_t v, hipStream_t s) {
  set_i32_kernel<<<1, 1, 0, s>>>(p, v);
  return hipGetLastError();
}

}  // namespace twell
