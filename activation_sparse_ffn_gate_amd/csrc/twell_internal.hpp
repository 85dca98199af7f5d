// Host-side launch helpers of libtwell (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace twell {

// Control block of the gate kernel's overflow set: one 64-bit word whose low
// half (ctrl[0]) counts rows appended this call and high half (ctrl[1])
// workgroups finished, then one dedup flag per row, then kDenseCounters
// arrival counters (the few-row fused kernel's per-row ordered sums). Zero
// between calls.
constexpr size_t kCtrlBytes = 256;

inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

struct GateArgs {
  const uint16_t* x;
  const uint16_t* Wg;
  int M, d, F, T, C;
  float* vals;
  uint8_t* idx;
  uint16_t* counts;
  int32_t* ovf_rows;
  int32_t* n_ovf;
  uint32_t* ctrl;   // kCtrlBytes, then flags[M]
  float* z_debug;   // nullable
  uint32_t* col_active;  // nullable: bit j % 32 of word j / 32 ORed with "some row has z_j > 0"
  float* spill;          // nullable, small-batch kernel only: [M, F/T, T] raw z of every (row, tile) with count > C
  // Gate-only variant (gateup_pack): the up weights, and an optional [M, F]
  // dump of the hidden values h = ReLU(z) u (z goes to z_debug).
  const uint16_t* WuT = nullptr;
  float* h_debug = nullptr;
  // Training gate (large kernel only): every z of each (row, tile) whose count
  // exceeds C goes to a record of a list of rec_cap records of T floats;
  // rec_slot[row][tile] receives its record, rec_n the records needed (the
  // counter lives in ctrl word 2 and is cleared by the last workgroup).
  float* rec_z = nullptr;
  int32_t* rec_slot = nullptr;
  int32_t* rec_n = nullptr;
  int rec_cap = 0;
  // Small-batch kernel: room for the K split across workgroups (nullable:
  // single launch); kpart_bytes must cover skinny_kpart_bytes(M, d, F).
  float* kpart = nullptr;
  size_t kpart_bytes = 0;
};

struct FusedArgs {
  const uint16_t* x;
  const uint16_t* WuT;
  const uint16_t* Wd;
  const float* vals;
  const uint8_t* idx;
  const uint16_t* counts;
  int M, d, F, T, C;
  float* y;
  const float* spill;  // nullable: rows with a tile count > C are done from it (else left to the fallback)
  // Workgroup-per-row form: long rows cut into up to `splits` parts, partial y
  // rows in part [splits, M, d], per-row arrival counters (zero, left zero).
  int splits = 1;
  float* part = nullptr;
  uint32_t* counters = nullptr;
};

// Dense gated FFN over a list of rows (all rows, or the overflow rows).
struct DenseArgs {
  const uint16_t* x;
  const uint16_t* Wg;
  const uint16_t* WuT;
  const uint16_t* Wd;
  int M, d, F;
  const int32_t* rows;    // nullptr: rows 0..M-1
  const int32_t* n_rows;  // device count of `rows` (when rows != nullptr)
  uint16_t* h_hi;         // [M, F] bf16 hidden (or its high part)
  uint16_t* h_lo;         // [M, F] low part; nullptr: plain bf16 hidden
  float* y;
  // Split-K of the gathering kernels: partial tiles, added up by a reduce
  // launch after each product.
  float* part;            // kDenseSplitSlots partial tiles of 64 KB
  bool split_k;           // the gathering kernels may split K
  // Gathering with a hi/lo hidden only: when the device-side row count
  // reaches ring_min_rows the ring kernels run the list instead (ring_ws
  // receives Wd^T); nullptr / 0: the register-staged kernels always do.
  void* ring_ws = nullptr;
  int ring_min_rows = 0;
};

// Partial-tile slots of the split-K fallback: 2 per work item of the gated-up
// kernel (z and u), 1 per item of the down kernel; at most 256 items.
constexpr int kDenseSplitSlots = 512;
constexpr size_t kDenseSplitBytes = size_t(kDenseSplitSlots) * 64 * 1024;
constexpr int kDenseCounters = 256;

// Up + down projections split into kSlices column slices of d, one per XCD.
constexpr int kSlices = 8;

struct SlicedArgs {
  const uint16_t* x;
  const uint16_t* WuT;
  const uint16_t* Wd;
  const float* vals;
  const uint8_t* idx;
  const uint16_t* counts;
  int M, d, F, T, C;
  float* part;       // [kSlices, M, (F / T) * C] partial up-projections
  int2* list;        // [M, (F / T) * C] each row's (unit, gate value bits) in (tile, slot) order
  int32_t* row_len;  // [M] number of stored units, -1 for an overflow row
  float* y;
};

// Byte offsets of the sliced kernels' buffers inside their workspace region.
struct SlicedLayout {
  size_t part, list, row_len, total;
};

hipError_t launch_gate_pack(const GateArgs& a, hipStream_t s);
// Batches up to this many tokens take the small-batch gate kernel.
constexpr int kSkinnyMaxM = 256;
constexpr int kSkinnyRb1MaxM = 128;  // up to here 32-token tiles, then 64-token tiles
hipError_t launch_gate_pack_skinny(const GateArgs& a, hipStream_t s);
// Bytes of K-split partial sums the small-batch gate uses for M rows when it
// splits K across workgroups (0: it does not split at this shape).
size_t skinny_kpart_bytes(int64_t M, int64_t d, int64_t F);
hipError_t launch_sliced_updown(const SlicedArgs& a, hipStream_t s);
// d and F the sliced kernels take (lane splits exist, weights below 2 GiB).
bool sliced_supports(int64_t d, int64_t F);
SlicedLayout sliced_layout(int64_t M, int64_t F, int T, int C);
constexpr int kFewRows = 256;  // up to here: the fused form with a workgroup per token, also in the forward
// Hybrid training format from a complete TwELL packing (C == T).
struct HybridArgs {
  const float* vals;
  const uint8_t* idx;
  const uint16_t* counts;
  int M, F, T, C, K, R;
  int32_t* h_idx;     // [M, K] global units, ascending; a reserve row's slot 0 holds its reserve slot
  float* h_vals;      // [M, K]
  int32_t* h_count;   // [M]
  int32_t* res_rows;  // [R]
  float* res_vals;    // [R, F]
  int32_t* n_res;     // [1]
  // C < T: the spill records of the overflowing tiles (GateArgs::rec_*)
  const float* rec_z = nullptr;
  const int32_t* rec_slot = nullptr;
  int rec_cap = 0;
};
hipError_t launch_hybrid_pack(const HybridArgs& a, hipStream_t s);

// Sparse backward over the hybrid format; entry list and sort buffers in a workspace.
struct BackwardArgs {
  const uint16_t *x, *Wg, *WuT, *Wd, *dy;
  const int32_t* h_idx;
  const float* h_vals;
  const int32_t* h_count;
  const int32_t* res_rows;
  const float* res_vals;
  const int32_t* n_res;
  int M, d, F, K, R;
  int64_t E_max;  // entry capacity: M K + R F
  float *dx, *dWg, *dWu, *dWd;
  int32_t* row_off;    // [M + 1]
  int32_t* hist;       // [sort blocks, F] entry counts, then first positions
  int32_t* unit_tot;   // [F]
  int32_t* unit_base;  // [F + 1]
  int32_t *e_unit, *e_row, *perm;  // [E_max]
  float *e_h, *e_dz, *e_du;        // [E_max]
  int32_t* res_prefix;  // [R + 1]: first work item of each reserve row (its runs follow)
  float* res_part;      // [R, kResMaxRuns, d]: each run's partial dx row
};
constexpr int kBackwardMaxF = 16384;  // the entry placement keeps one counter per unit in LDS (64 KB)
constexpr int kResMaxRuns = 16;       // runs a reserve row's units are cut into at most
bool backward_supports_d(int d);
int backward_sort_blocks(int64_t M);
hipError_t launch_backward(const BackwardArgs& a, hipStream_t s);

// Row gather: out[i] = W[src[i]] for 0 <= src[i] < F, else a zero row.
hipError_t launch_gather_rows(const uint16_t* W, int F, int d, const int32_t* src, int n, uint16_t* out,
                              hipStream_t s);

hipError_t launch_fused_updown(const FusedArgs& a, hipStream_t s);
// Gate-only variant: dense gate and up products with the packing of h in the
// epilogue (vals hold h), then the down product from that packing.
hipError_t launch_gateup_pack(const GateArgs& a, hipStream_t s);
hipError_t launch_hidden_down(const SlicedArgs& a, hipStream_t s);
// Register-staged dense kernels: gathering (rows != nullptr) for the
// fallback, which also enqueues the ring kernels when ring_ws is set.
hipError_t launch_dense(const DenseArgs& a, hipStream_t s);

// Dense baseline on the gate kernel's LDS-DMA ring (rows 0..M-1, bf16 h):
// whether the shape fits its 32-bit offsets, the K splits of its down
// product, and the workspace it needs (Wd^T, then the partials of splits 1..).
bool dense_ring_supports(int64_t M, int64_t d, int64_t F);
int dense_ring_splits(int64_t M, int64_t d, int64_t F);
size_t dense_ring_bytes(int64_t M, int64_t d, int64_t F);
hipError_t launch_dense_ring(const DenseArgs& a, void* ring_ws, hipStream_t s);

// The fallback's ring path, for lists long enough to fill the chip without
// splitting K (at least dense_ring_fallback_min_rows(d) rows, a count the
// kernels read on the device): whether a batch of M rows can reach it, the
// workspace it needs (Wd^T), and its two launch steps, each returning at once
// for a shorter list (transpose + gated up with a hi/lo hidden; down over
// K = 2F, the hi and then the lo plane, with y rows scattered to the list's
// tokens).
int dense_ring_fallback_min_rows(int64_t d);
bool dense_ring_fallback_possible(int64_t M, int64_t d, int64_t F);
size_t dense_ring_fallback_bytes(int64_t d, int64_t F);
hipError_t launch_ring_fallback_up(const DenseArgs& a, hipStream_t s);
hipError_t launch_ring_fallback_down(const DenseArgs& a, hipStream_t s);
hipError_t launch_set_i32(int32_t* p, int32_t v, hipStream_t s);

bool fused_supports_d(int d);

}  // namespace twell
