// extern "C" entry points of libtwell.so: argument checks, workspace layout
// and launch order. Declared and documented in include/twell.h.
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "../../include/twell.h"
#include "twell_internal.hpp"

using twell::align256;

namespace {

constexpr int64_t kMaxM = int64_t(1) << 30;
constexpr int64_t kMaxF = int64_t(1) << 24;

struct Layout {
  size_t vals = 0, idx = 0, counts = 0, ovf_rows = 0, n_ovf = 0, h_hi = 0, h_lo = 0, part = 0;
  size_t split = 0;  // the split-K fallback's partial tiles
  size_t ring = 0;   // the dense baseline's Wd^T and split partials
  size_t total = 0;
};

// Header, one flag per row, then the few-row fused kernel's arrival counters.
size_t ctrl_flags_bytes(int64_t M) { return twell::kCtrlBytes + align256(size_t(M) * 4); }
size_t ctrl_bytes(int64_t M) { return ctrl_flags_bytes(M) + align256(twell::kDenseCounters * 4); }
uint32_t* row_counters(void* ctrl, int64_t M) {
  return reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ctrl) + ctrl_flags_bytes(M));
}

// Offsets inside the workspace of each operation (all 256-byte aligned).
Layout layout(int32_t op, int64_t M, int64_t d, int64_t F, int32_t T, int32_t C) {
  Layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t m = size_t(M), f = size_t(F);
  const size_t nT = (T > 0) ? f / size_t(T) : 0;
  switch (op) {
    case TWELL_OP_GATE_PACK:
      break;
    case TWELL_OP_COLUMN_ACTIVITY:  // a packing that is thrown away
      L.vals = take(m * nT * size_t(C) * 4);
      L.idx = take(m * nT * size_t(C));
      L.counts = take(m * nT * 2);
      L.ovf_rows = take(m * 4);
      L.n_ovf = take(4);
      break;
    case TWELL_OP_FFN_FORWARD:
      L.vals = take(m * nT * size_t(C) * 4);
      L.idx = take(m * nT * size_t(C));
      L.counts = take(m * nT * 2);
      L.ovf_rows = take(m * 4);
      L.n_ovf = take(4);
      // The up/down kernels and the fallback run concurrently (two streams),
      // so each has its own region: the sliced kernels' partials, then the
      // fallback's hidden pair and partial tiles.
      L.part = take(twell::sliced_layout(M, F, T, C).total);
      L.h_hi = take(m * f * 2);
      L.h_lo = take(m * f * 2);
      L.split = take(twell::kDenseSplitBytes);
      // a long overflow list runs on the ring kernels, which read Wd^T
      if (twell::dense_ring_fallback_possible(M, d, F)) L.ring = take(twell::dense_ring_fallback_bytes(d, F));
      break;
    case TWELL_OP_SLICED_UPDOWN:
      L.part = take(twell::sliced_layout(M, F, T, C).total);
      break;
    case TWELL_OP_FFN_FORWARD_GATEUP:  // packing of h, then the fallback's region
      L.vals = take(m * nT * size_t(C) * 4);
      L.idx = take(m * nT * size_t(C));
      L.counts = take(m * nT * 2);
      L.ovf_rows = take(m * 4);
      L.n_ovf = take(4);
      L.h_hi = take(m * f * 2);
      L.h_lo = take(m * f * 2);
      L.split = take(twell::kDenseSplitBytes);
      if (twell::dense_ring_fallback_possible(M, d, F)) L.ring = take(twell::dense_ring_fallback_bytes(d, F));
      break;
    case TWELL_OP_DENSE_FFN:
      L.h_hi = take(m * f * 2);
      if (twell::dense_ring_supports(M, d, F)) L.ring = take(twell::dense_ring_bytes(M, d, F));
      break;
    case TWELL_OP_DENSE_FALLBACK:
      L.h_hi = take(m * f * 2);
      L.h_lo = take(m * f * 2);
      L.split = take(twell::kDenseSplitBytes);
      if (twell::dense_ring_fallback_possible(M, d, F)) L.ring = take(twell::dense_ring_fallback_bytes(d, F));
      break;
    default:
      return L;
  }
  L.total = off;
  return L;
}

int check_dims(int64_t M, int64_t d, int64_t F) {
  if (M < 0 || d <= 0 || F <= 0) return TWELL_E_INVALID_ARG;
  if (M > kMaxM || F > kMaxF) return TWELL_E_INVALID_ARG;
  if (d % 256 != 0 || d > 8192 || !twell::fused_supports_d(int(d))) return TWELL_E_UNSUPPORTED;
  return TWELL_OK;
}

int check_tc(int64_t F, int32_t T, int32_t C) {
  if (T != 64 && T != 128) return TWELL_E_UNSUPPORTED;
  if (F % T != 0) return TWELL_E_UNSUPPORTED;
  if (C < 1 || C > T) return TWELL_E_UNSUPPORTED;
  return TWELL_OK;
}

// The gate kernels address x, Wg and the packed values with 32-bit byte offsets.
int check_gate_offsets(int64_t M, int64_t d, int64_t F, int32_t T, int32_t C) {
  const int64_t lim = int64_t(1) << 31;
  if (M * d * 2 >= lim || F * d * 2 >= lim || M * (F / T) * int64_t(C) * 4 >= lim) return TWELL_E_UNSUPPORTED;
  return TWELL_OK;
}

int check_ws(int32_t op, int64_t M, int64_t d, int64_t F, int32_t T, int32_t C, void* ws, size_t ws_bytes) {
  const Layout L = layout(op, M, d, F, T, C);
  if (L.total == 0) return TWELL_OK;
  if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0 || ws_bytes < L.total)
    return TWELL_E_WORKSPACE;
  return TWELL_OK;
}

int check_ctrl(int64_t M, void* ctrl, size_t n) {
  if (ctrl == nullptr || (reinterpret_cast<uintptr_t>(ctrl) & 255u) != 0 || n < ctrl_bytes(M))
    return TWELL_E_WORKSPACE;
  return TWELL_OK;
}

// With M == 0 the row arrays are empty and may be NULL; n_ovf is still written.
bool packed_ok(const twell_packed* p, int64_t M) {
  return p && p->n_ovf && (M == 0 || (p->vals && p->idx && p->counts && p->ovf_rows));
}

int hip_status(hipError_t e) { return e == hipSuccess ? TWELL_OK : TWELL_E_HIP; }

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off);
}

twell_packed packed_in_ws(void* ws, const Layout& L) {
  twell_packed p;
  p.vals = at<float>(ws, L.vals);
  p.idx = at<uint8_t>(ws, L.idx);
  p.counts = at<uint16_t>(ws, L.counts);
  p.ovf_rows = at<int32_t>(ws, L.ovf_rows);
  p.n_ovf = at<int32_t>(ws, L.n_ovf);
  return p;
}

int gate_pack_impl(const uint16_t* x, const uint16_t* Wg, int64_t M, int64_t d, int64_t F, int32_t T,
                   int32_t C, const twell_packed* out, float* z_debug, uint32_t* ctrl,
                   hipStream_t s, uint32_t* col_active = nullptr, float* spill = nullptr,
                   float* kpart = nullptr, size_t kpart_bytes = 0) {
  if (M == 0) return hip_status(twell::launch_set_i32(out->n_ovf, 0, s));
  twell::GateArgs a;
  a.x = x;
  a.Wg = Wg;
  a.M = int(M);
  a.d = int(d);
  a.F = int(F);
  a.T = T;
  a.C = C;
  a.vals = out->vals;
  a.idx = out->idx;
  a.counts = out->counts;
  a.ovf_rows = out->ovf_rows;
  a.n_ovf = out->n_ovf;
  a.ctrl = ctrl;
  a.z_debug = z_debug;
  a.col_active = col_active;
  a.spill = spill;
  a.kpart = kpart;
  a.kpart_bytes = kpart_bytes;
  return hip_status(twell::launch_gate_pack(a, s));
}

twell::FusedArgs fused_args(const uint16_t* x, const uint16_t* WuT, const uint16_t* Wd, const twell_packed* in,
                            int64_t M, int64_t d, int64_t F, int32_t T, int32_t C, float* y) {
  twell::FusedArgs a;
  a.x = x;
  a.WuT = WuT;
  a.Wd = Wd;
  a.vals = in->vals;
  a.idx = in->idx;
  a.counts = in->counts;
  a.M = int(M);
  a.d = int(d);
  a.F = int(F);
  a.T = T;
  a.C = C;
  a.y = y;
  a.spill = nullptr;
  return a;
}

int fused_impl(const uint16_t* x, const uint16_t* WuT, const uint16_t* Wd, const twell_packed* in,
               int64_t M, int64_t d, int64_t F, int32_t T, int32_t C, float* y, hipStream_t s) {
  if (M == 0) return TWELL_OK;
  return hip_status(twell::launch_fused_updown(fused_args(x, WuT, Wd, in, M, d, F, T, C, y), s));
}

// `region` is the sliced kernels' workspace region (twell::sliced_layout).
int sliced_impl(const uint16_t* x, const uint16_t* WuT, const uint16_t* Wd, const twell_packed* in,
                int64_t M, int64_t d, int64_t F, int32_t T, int32_t C, void* region, float* y,
                hipStream_t s) {
  if (M == 0) return TWELL_OK;
  const twell::SlicedLayout sl = twell::sliced_layout(M, F, T, C);
  twell::SlicedArgs a;
  a.x = x;
  a.WuT = WuT;
  a.Wd = Wd;
  a.vals = in->vals;
  a.idx = in->idx;
  a.counts = in->counts;
  a.M = int(M);
  a.d = int(d);
  a.F = int(F);
  a.T = T;
  a.C = C;
  a.part = at<float>(region, sl.part);
  a.list = at<int2>(region, sl.list);
  a.row_len = at<int32_t>(region, sl.row_len);
  a.y = y;
  return hip_status(twell::launch_sliced_updown(a, s));
}

// The fallback's Wd^T region when a list of M rows can reach its ring kernels.
void* ring_region(void* ws, const Layout& L, int64_t M, int64_t d, int64_t F) {
  return twell::dense_ring_fallback_possible(M, d, F) ? static_cast<void*>(static_cast<uint8_t*>(ws) + L.ring)
                                                      : nullptr;
}

int dense_impl(const uint16_t* x, const uint16_t* Wg, const uint16_t* WuT, const uint16_t* Wd,
               int64_t M, int64_t d, int64_t F, const int32_t* rows, const int32_t* n_rows,
               uint16_t* h_hi, uint16_t* h_lo, float* y, float* split_part, bool split_k, hipStream_t s,
               void* ring_ws = nullptr) {
  if (M == 0) return TWELL_OK;
  twell::DenseArgs a;
  a.x = x;
  a.Wg = Wg;
  a.WuT = WuT;
  a.Wd = Wd;
  a.M = int(M);
  a.d = int(d);
  a.F = int(F);
  a.rows = rows;
  a.n_rows = n_rows;
  a.h_hi = h_hi;
  a.h_lo = h_lo;
  a.y = y;
  a.part = split_part;
  a.split_k = split_k;
  a.ring_ws = ring_ws;
  a.ring_min_rows = ring_ws != nullptr ? twell::dense_ring_fallback_min_rows(d) : 0;
  return hip_status(twell::launch_dense(a, s));
}

// Gate-only variant: dense gate and up products with h packed in TwELL.
int gateup_impl(const uint16_t* x, const uint16_t* Wg, const uint16_t* WuT, int64_t M, int64_t d, int64_t F,
                int32_t T, int32_t C, const twell_packed* out, float* z_debug, float* h_debug, uint32_t* ctrl,
                hipStream_t s) {
  if (M == 0) return hip_status(twell::launch_set_i32(out->n_ovf, 0, s));
  twell::GateArgs a;
  a.x = x;
  a.Wg = Wg;
  a.M = int(M);
  a.d = int(d);
  a.F = int(F);
  a.T = T;
  a.C = C;
  a.vals = out->vals;
  a.idx = out->idx;
  a.counts = out->counts;
  a.ovf_rows = out->ovf_rows;
  a.n_ovf = out->n_ovf;
  a.ctrl = ctrl;
  a.z_debug = z_debug;
  a.col_active = nullptr;
  a.spill = nullptr;
  a.WuT = WuT;
  a.h_debug = h_debug;
  return hip_status(twell::launch_gateup_pack(a, s));
}

int hidden_down_impl(const uint16_t* Wd, const twell_packed* in, int64_t M, int64_t d, int64_t F, int32_t T,
                     int32_t C, float* y, hipStream_t s) {
  if (M == 0) return TWELL_OK;
  twell::SlicedArgs a{};
  a.Wd = Wd;
  a.vals = in->vals;
  a.idx = in->idx;
  a.counts = in->counts;
  a.M = int(M);
  a.d = int(d);
  a.F = int(F);
  a.T = T;
  a.C = C;
  a.y = y;
  return hip_status(twell::launch_hidden_down(a, s));
}

// The forward up to twell::kFewRows rows: the small-batch gate spills the z
// of every overflowing (row, tile) into `spill`, and the fused kernel (a
// workgroup per row) does overflow rows from it: two launches in all. Long
// rows are cut over several workgroups, with their partial rows in `part`
// (splits * M * d floats) and one arrival counter per row after the control
// block's flags.
int splits_for(int64_t M) { return int(std::min<int64_t>(16, std::max<int64_t>(1, 512 / M))); }

// Optional events recorded on the stream right before the gate's launches
// and right after them (twell_ffn_forward_timed); null: none.
struct GateEvents {
  hipEvent_t begin = nullptr, end = nullptr;
};

int record(hipEvent_t e, hipStream_t s) {
  return (e == nullptr || hipEventRecord(e, s) == hipSuccess) ? TWELL_OK : TWELL_E_HIP;
}

int few_rows_forward(const uint16_t* x, const uint16_t* Wg, const uint16_t* WuT, const uint16_t* Wd, int64_t M,
                     int64_t d, int64_t F, int32_t T, int32_t C, float* y, void* ctrl, const twell_packed& p,
                     float* spill, float* part, size_t part_bytes, hipStream_t s, GateEvents ev = {}) {
  // The gate's K-split partial sums (if it splits) are consumed before the
  // fused kernel writes its partial rows to the same region.
  int st = record(ev.begin, s);
  if (st == TWELL_OK)
    st = gate_pack_impl(x, Wg, M, d, F, T, C, &p, nullptr, static_cast<uint32_t*>(ctrl), s, nullptr, spill, part,
                        part_bytes);
  if (st == TWELL_OK) st = record(ev.end, s);
  if (st != TWELL_OK) return st;
  twell::FusedArgs a = fused_args(x, WuT, Wd, &p, M, d, F, T, C, y);
  a.spill = spill;
  a.splits = splits_for(M);
  a.part = part;
  a.counters = row_counters(ctrl, M);
  return hip_status(twell::launch_fused_updown(a, s));
}

// ------------------------------------------------ allocation-free forward
// One static device buffer per GPU for twell_ffn_forward_static: the control
// block (sized for the most rows that entry takes), then the packing, the
// spill and the partial rows of the call. It starts zeroed when the code
// object is loaded; the control block in it is left zeroed by every call, as
// for a caller-owned one. Host code never names the array in an argument:
// it uses the address hipGetSymbolAddress returned on that device.
constexpr size_t kStaticScratch = TWELL_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kStaticScratch];

struct StaticLayout {
  size_t ctrl = 0, vals = 0, idx = 0, counts = 0, ovf_rows = 0, n_ovf = 0, spill = 0, part = 0, total = 0;
};

StaticLayout static_layout(int64_t M, int64_t d, int64_t F, int32_t T, int32_t C) {
  StaticLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t m = size_t(M), nT = size_t(F / T);
  L.ctrl = take(ctrl_bytes(twell::kFewRows));
  L.vals = take(m * nT * size_t(C) * 4);
  L.idx = take(m * nT * size_t(C));
  L.counts = take(m * nT * 2);
  L.ovf_rows = take(m * 4);
  L.n_ovf = take(4);
  L.spill = take(m * size_t(F) * 4);
  L.part = take(std::max(size_t(splits_for(std::max<int64_t>(M, 1))) * m * size_t(d) * 4,
                         twell::skinny_kpart_bytes(M, d, F)));
  L.total = off;
  return L;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

int stream_device(hipStream_t s, int* dev);

// Device address of `scratch` on the stream's device, taken once per device
// with that device current.
int static_scratch(hipStream_t s, uint8_t** out) {
  int dev = -1;
  if (stream_device(s, &dev) != TWELL_OK) return TWELL_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return TWELL_E_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return TWELL_E_HIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || ptr == nullptr) return TWELL_E_HIP;
    g_scratch[dev] = ptr;
  }
  *out = static_cast<uint8_t*>(g_scratch[dev]);
  return TWELL_OK;
}

// ------------------------------------------------ fallback side stream
// Above the few-row range the dense fallback of overflow rows does not depend
// on the up/down kernels (they write disjoint rows of y and use disjoint
// workspace regions), so it runs on a second stream of the caller's device,
// forked after the gate and joined before the call returns (stream order of
// the caller's stream is kept). With no overflow row its two launches end at
// once and hide behind the up/down kernels; with overflow rows the two paths
// overlap. One non-blocking stream at the default priority and two events per
// device, created on the first forward on that device and kept for the
// process; the fork and join of one call are issued under a lock, so calls
// from several host threads pair their events correctly (their fallbacks then
// run one after the other on the side stream).
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];

int stream_device(hipStream_t s, int* dev) {
  if ((s ? hipStreamGetDevice(s, dev) : hipGetDevice(dev)) != hipSuccess) return TWELL_E_HIP;
  return (*dev >= 0 && *dev < kMaxDevices) ? TWELL_OK : TWELL_E_HIP;
}

// Creates the side stream and events of device `dev` if needed; call with
// g_side_mu held.
int side_stream_locked(int dev, SideStream** out) {
  SideStream& ss = g_side[dev];
  if (ss.s == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return TWELL_E_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return TWELL_E_HIP;
    SideStream n;
    bool ok = hipStreamCreateWithFlags(&n.s, hipStreamNonBlocking) == hipSuccess;
    ok = ok && hipEventCreateWithFlags(&n.fork, hipEventDisableTiming) == hipSuccess;
    ok = ok && hipEventCreateWithFlags(&n.join, hipEventDisableTiming) == hipSuccess;
    if (cur != dev) (void)hipSetDevice(cur);
    if (!ok) {
      if (n.join) (void)hipEventDestroy(n.join);
      if (n.fork) (void)hipEventDestroy(n.fork);
      if (n.s) (void)hipStreamDestroy(n.s);
      return TWELL_E_HIP;
    }
    ss = n;
  }
  *out = &ss;
  return TWELL_OK;
}

// Workspace of twell_ffn_backward: row offsets, the counting sort's per-block
// counts and unit offsets, and the entry list (unit, row, h, dz, du) with its
// unit-major order.
struct BwdLayout {
  size_t row_off = 0, hist = 0, unit_tot = 0, unit_base = 0, e_unit = 0, e_row = 0, perm = 0;
  size_t e_h = 0, e_dz = 0, e_du = 0, res_prefix = 0, res_part = 0, total = 0;
  int64_t E_max = 0;
};

int check_bwd(int64_t M, int64_t d, int64_t F, int32_t K, int64_t R) {
  if (M < 0 || d <= 0 || F <= 0 || K < 1 || R < 0 || R > M) return TWELL_E_INVALID_ARG;
  if (M > kMaxM || F > kMaxF) return TWELL_E_INVALID_ARG;
  if (!twell::backward_supports_d(int(d)) || F > twell::kBackwardMaxF) return TWELL_E_UNSUPPORTED;
  if (M * int64_t(K) + R * F >= (int64_t(1) << 31)) return TWELL_E_UNSUPPORTED;
  return TWELL_OK;
}

BwdLayout bwd_layout(int64_t M, int64_t d, int64_t F, int32_t K, int64_t R) {
  BwdLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  L.E_max = M * int64_t(K) + R * F;
  const size_t e4 = size_t(L.E_max) * 4;
  L.row_off = take(size_t(M + 1) * 4);
  // per-block counts and unit totals are one region (cleared together)
  L.hist = take(size_t(twell::backward_sort_blocks(M) + 1) * size_t(F) * 4);
  L.unit_tot = L.hist + size_t(twell::backward_sort_blocks(M)) * size_t(F) * 4;
  L.unit_base = take(size_t(F + 1) * 4);
  L.e_unit = take(e4);
  L.e_row = take(e4);
  L.perm = take(e4);
  L.e_h = take(e4);
  L.e_dz = take(e4);
  L.e_du = take(e4);
  L.res_prefix = take(size_t(R + 1) * 4);
  L.res_part = take(size_t(R) * twell::kResMaxRuns * size_t(d) * 4);
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

int twell_hybrid_pack(const twell_packed* in, const twell_spill* spill, int64_t M, int64_t F, int32_t T,
                      int32_t C, int32_t K, int64_t R, const twell_hybrid* out, void* stream) {
  if (!in || !out || !out->n_res) return TWELL_E_INVALID_ARG;
  if (M < 0 || M > kMaxM || F <= 0 || F > kMaxF || K < 1 || R < 0 || R > M) return TWELL_E_INVALID_ARG;
  int st = check_tc(F, T, C);
  if (st != TWELL_OK) return st;
  // below C = T the tiles that overflow come from the spill list
  if (C != T && (!spill || !spill->z || !spill->slot || spill->cap < 0 || spill->cap * T >= (int64_t(1) << 31)))
    return TWELL_E_INVALID_ARG;
  if (M != 0 && (!in->vals || !in->idx || !in->counts || !out->idx || !out->vals || !out->count))
    return TWELL_E_INVALID_ARG;
  if (R != 0 && (!out->res_rows || !out->res_vals)) return TWELL_E_INVALID_ARG;
  twell::HybridArgs a;
  a.vals = in->vals;
  a.idx = in->idx;
  a.counts = in->counts;
  a.M = int(M);
  a.F = int(F);
  a.T = T;
  a.C = C;
  a.K = K;
  a.R = int(R);
  a.h_idx = out->idx;
  a.h_vals = out->vals;
  a.h_count = out->count;
  a.res_rows = out->res_rows;
  a.res_vals = out->res_vals;
  a.n_res = out->n_res;
  if (C != T) {
    a.rec_z = spill->z;
    a.rec_slot = spill->slot;
    a.rec_cap = int(spill->cap);
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (M == 0) return hip_status(twell::launch_set_i32(out->n_res, 0, s));
  return hip_status(twell::launch_hybrid_pack(a, s));
}

int twell_gate_pack_spill(const uint16_t* x, const uint16_t* Wg, int64_t M, int64_t d, int64_t F, int32_t T,
                          int32_t C, const twell_packed* out, const twell_spill* spill, float* z_debug,
                          void* ctrl, size_t ctrl_bytes_, void* stream) {
  if ((M != 0 && !x) || !Wg || !packed_ok(out, M) || !spill || !spill->n_spill) return TWELL_E_INVALID_ARG;
  if (M != 0 && (!spill->slot || !spill->z)) return TWELL_E_INVALID_ARG;
  if (spill->cap < 0 || spill->cap * T >= (int64_t(1) << 31)) return TWELL_E_INVALID_ARG;
  int st = check_dims(M, d, F);
  if (st == TWELL_OK) st = check_tc(F, T, C);
  if (st == TWELL_OK) st = check_gate_offsets(M, d, F, T, C);
  if (st == TWELL_OK) st = check_ctrl(M, ctrl, ctrl_bytes_);
  if (st != TWELL_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (M == 0) {
    st = hip_status(twell::launch_set_i32(out->n_ovf, 0, s));
    return st != TWELL_OK ? st : hip_status(twell::launch_set_i32(spill->n_spill, 0, s));
  }
  twell::GateArgs a;
  a.x = x;
  a.Wg = Wg;
  a.M = int(M);
  a.d = int(d);
  a.F = int(F);
  a.T = T;
  a.C = C;
  a.vals = out->vals;
  a.idx = out->idx;
  a.counts = out->counts;
  a.ovf_rows = out->ovf_rows;
  a.n_ovf = out->n_ovf;
  a.ctrl = static_cast<uint32_t*>(ctrl);
  a.z_debug = z_debug;
  a.col_active = nullptr;
  a.spill = nullptr;
  a.rec_z = spill->z;
  a.rec_slot = spill->slot;
  a.rec_n = spill->n_spill;
  a.rec_cap = int(spill->cap);
  return hip_status(twell::launch_gate_pack(a, s));
}

size_t twell_backward_workspace_bytes(int64_t M, int64_t d, int64_t F, int32_t K, int64_t R) {
  if (check_bwd(M, d, F, K, R) != TWELL_OK) return 0;
  return bwd_layout(M, d, F, K, R).total;
}

int twell_ffn_backward(const uint16_t* x, const uint16_t* Wg, const uint16_t* WuT, const uint16_t* Wd,
                       const uint16_t* dy, const twell_hybrid* hy, int64_t M, int64_t d, int64_t F,
                       int32_t K, int64_t R, float* dx, float* dWg, float* dWuT, float* dWd,
                       void* workspace, size_t ws_bytes, void* stream) {
  if (!Wg || !WuT || !Wd || !hy || !hy->n_res || !dWg || !dWuT || !dWd) return TWELL_E_INVALID_ARG;
  if (M != 0 && (!x || !dy || !dx || !hy->idx || !hy->vals || !hy->count)) return TWELL_E_INVALID_ARG;
  if (R != 0 && (!hy->res_vals || !hy->res_rows)) return TWELL_E_INVALID_ARG;
  int st = check_bwd(M, d, F, K, R);
  if (st != TWELL_OK) return st;
  const BwdLayout L = bwd_layout(M, d, F, K, R);
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || ws_bytes < L.total)
    return TWELL_E_WORKSPACE;
  twell::BackwardArgs a;
  a.x = x;
  a.Wg = Wg;
  a.WuT = WuT;
  a.Wd = Wd;
  a.dy = dy;
  a.h_idx = hy->idx;
  a.h_vals = hy->vals;
  a.h_count = hy->count;
  a.res_rows = hy->res_rows;
  a.res_vals = hy->res_vals;
  a.n_res = hy->n_res;
  a.M = int(M);
  a.d = int(d);
  a.F = int(F);
  a.K = K;
  a.R = int(R);
  a.E_max = L.E_max;
  a.dx = dx;
  a.dWg = dWg;
  a.dWu = dWuT;
  a.dWd = dWd;
  a.row_off = at<int32_t>(workspace, L.row_off);
  a.hist = at<int32_t>(workspace, L.hist);
  a.unit_tot = at<int32_t>(workspace, L.unit_tot);
  a.unit_base = at<int32_t>(workspace, L.unit_base);
  a.e_unit = at<int32_t>(workspace, L.e_unit);
  a.e_row = at<int32_t>(workspace, L.e_row);
  a.perm = at<int32_t>(workspace, L.perm);
  a.e_h = at<float>(workspace, L.e_h);
  a.e_dz = at<float>(workspace, L.e_dz);
  a.e_du = at<float>(workspace, L.e_du);
  a.res_prefix = at<int32_t>(workspace, L.res_prefix);
  a.res_part = at<float>(workspace, L.res_part);
  return hip_status(twell::launch_backward(a, static_cast<hipStream_t>(stream)));
}

int twell_gate_pack(const uint16_t* x, const uint16_t* Wg, int64_t M, int64_t d, int64_t F,
                    int32_t T, int32_t C, const twell_packed* out, float* z_debug, void* ctrl,
                    size_t ctrl_bytes_, void* stream) {
  if ((M != 0 && !x) || !Wg || !packed_ok(out, M)) return TWELL_E_INVALID_ARG;
  int st = check_dims(M, d, F);
  if (st == TWELL_OK) st = check_tc(F, T, C);
  if (st == TWELL_OK) st = check_gate_offsets(M, d, F, T, C);
  if (st == TWELL_OK) st = check_ctrl(M, ctrl, ctrl_bytes_);
  if (st != TWELL_OK) return st;
  return gate_pack_impl(x, Wg, M, d, F, T, C, out, z_debug, static_cast<uint32_t*>(ctrl),
                        static_cast<hipStream_t>(stream));
}

int twell_fused_updown(const uint16_t* x, const uint16_t* WuT, const uint16_t* Wd,
                       const twell_packed* in, int64_t M, int64_t d, int64_t F, int32_t T,
                       int32_t C, float* y, void* stream) {
  if (!WuT || !Wd || !in) return TWELL_E_INVALID_ARG;
  if (M != 0 && (!x || !y || !in->vals || !in->idx || !in->counts)) return TWELL_E_INVALID_ARG;
  int st = check_dims(M, d, F);
  if (st == TWELL_OK) st = check_tc(F, T, C);
  if (st != TWELL_OK) return st;
  return fused_impl(x, WuT, Wd, in, M, d, F, T, C, y, static_cast<hipStream_t>(stream));
}

int twell_sliced_updown(const uint16_t* x, const uint16_t* WuT, const uint16_t* Wd,
                        const twell_packed* in, int64_t M, int64_t d, int64_t F, int32_t T,
                        int32_t C, float* y, void* workspace, size_t ws_bytes, void* stream) {
  if (!WuT || !Wd || !in) return TWELL_E_INVALID_ARG;
  if (M != 0 && (!x || !y || !in->vals || !in->idx || !in->counts)) return TWELL_E_INVALID_ARG;
  int st = check_dims(M, d, F);
  if (st == TWELL_OK) st = check_tc(F, T, C);
  if (st == TWELL_OK && !twell::sliced_supports(d, F)) st = TWELL_E_UNSUPPORTED;
  if (st == TWELL_OK) st = check_ws(TWELL_OP_SLICED_UPDOWN, M, d, F, T, C, workspace, ws_bytes);
  if (st != TWELL_OK) return st;
  const Layout L = layout(TWELL_OP_SLICED_UPDOWN, M, d, F, T, C);
  return sliced_impl(x, WuT, Wd, in, M, d, F, T, C, at<uint8_t>(workspace, L.part), y,
                     static_cast<hipStream_t>(stream));
}

int twell_dense_fallback(const uint16_t* x, const uint16_t* Wg, const uint16_t* WuT,
                         const uint16_t* Wd, const twell_packed* in, int64_t M, int64_t d,
                         int64_t F, float* y, void* ctrl, size_t ctrl_bytes_, void* workspace,
                         size_t ws_bytes, void* stream) {
  if (!Wg || !WuT || !Wd || !in || !in->n_ovf) return TWELL_E_INVALID_ARG;
  if (M != 0 && (!x || !y || !in->ovf_rows)) return TWELL_E_INVALID_ARG;
  int st = check_dims(M, d, F);
  if (st == TWELL_OK && F % 64 != 0) st = TWELL_E_UNSUPPORTED;
  if (st == TWELL_OK) st = check_ctrl(M, ctrl, ctrl_bytes_);
  if (st == TWELL_OK) st = check_ws(TWELL_OP_DENSE_FALLBACK, M, d, F, 0, 0, workspace, ws_bytes);
  if (st != TWELL_OK) return st;
  const Layout L = layout(TWELL_OP_DENSE_FALLBACK, M, d, F, 0, 0);
  return dense_impl(x, Wg, WuT, Wd, M, d, F, in->ovf_rows, in->n_ovf, at<uint16_t>(workspace, L.h_hi),
                    at<uint16_t>(workspace, L.h_lo), y, at<float>(workspace, L.split),
                    true, static_cast<hipStream_t>(stream), ring_region(workspace, L, M, d, F));
}

static int ffn_forward_impl(const uint16_t* x, const uint16_t* Wg, const uint16_t* WuT, const uint16_t* Wd,
                            int64_t M, int64_t d, int64_t F, int32_t T, int32_t C, float* y, void* ctrl,
                            size_t ctrl_bytes_, void* workspace, size_t ws_bytes, void* stream, GateEvents ev) {
  if (!Wg || !WuT || !Wd || (M != 0 && (!x || !y))) return TWELL_E_INVALID_ARG;
  int st = check_dims(M, d, F);
  if (st == TWELL_OK) st = check_tc(F, T, C);
  if (st == TWELL_OK) st = check_gate_offsets(M, d, F, T, C);
  if (st == TWELL_OK) st = check_ctrl(M, ctrl, ctrl_bytes_);
  if (st == TWELL_OK) st = check_ws(TWELL_OP_FFN_FORWARD, M, d, F, T, C, workspace, ws_bytes);
  if (st != TWELL_OK) return st;
  if (M == 0) return TWELL_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const Layout L = layout(TWELL_OP_FFN_FORWARD, M, d, F, T, C);
  const twell_packed p = packed_in_ws(workspace, L);
  if (M <= twell::kFewRows) {
    // The spill (M F floats) takes the fallback's hidden pair (2 M F bf16) and
    // the partial rows (at most 512 rows of d floats) its split-K region; both
    // are idle on this path.
    return few_rows_forward(x, Wg, WuT, Wd, M, d, F, T, C, y, ctrl, p, at<float>(workspace, L.h_hi),
                            at<float>(workspace, L.split), twell::kDenseSplitBytes, s, ev);
  }
  int dev = -1;
  if (stream_device(s, &dev) != TWELL_OK) return TWELL_E_HIP;
  std::lock_guard<std::mutex> lock(g_side_mu);
  SideStream* ss = nullptr;
  st = side_stream_locked(dev, &ss);  // before anything is enqueued
  if (st != TWELL_OK) return st;
  st = record(ev.begin, s);
  if (st == TWELL_OK) st = gate_pack_impl(x, Wg, M, d, F, T, C, &p, nullptr, static_cast<uint32_t*>(ctrl), s);
  if (st == TWELL_OK) st = record(ev.end, s);
  if (st != TWELL_OK) return st;
  // fork: the fallback of the overflow rows on the side stream
  if (hipEventRecord(ss->fork, s) != hipSuccess || hipStreamWaitEvent(ss->s, ss->fork, 0) != hipSuccess)
    return TWELL_E_HIP;
  const int st_fb = dense_impl(x, Wg, WuT, Wd, M, d, F, p.ovf_rows, p.n_ovf, at<uint16_t>(workspace, L.h_hi),
                               at<uint16_t>(workspace, L.h_lo), y, at<float>(workspace, L.split),
                               true, ss->s, ring_region(workspace, L, M, d, F));
  // join before anything else can be reported, so the caller's stream never
  // runs ahead of work already on the side stream
  const bool joined = hipEventRecord(ss->join, ss->s) == hipSuccess;
  if (twell::sliced_supports(d, F))
    st = sliced_impl(x, WuT, Wd, &p, M, d, F, T, C, at<uint8_t>(workspace, L.part), y, s);
  else
    st = fused_impl(x, WuT, Wd, &p, M, d, F, T, C, y, s);
  if (!joined || hipStreamWaitEvent(s, ss->join, 0) != hipSuccess) return TWELL_E_HIP;
  return st != TWELL_OK ? st : st_fb;
}

int twell_ffn_forward(const uint16_t* x, const uint16_t* Wg, const uint16_t* WuT,
                      const uint16_t* Wd, int64_t M, int64_t d, int64_t F, int32_t T, int32_t C,
                      float* y, void* ctrl, size_t ctrl_bytes_, void* workspace, size_t ws_bytes,
                      void* stream) {
  return ffn_forward_impl(x, Wg, WuT, Wd, M, d, F, T, C, y, ctrl, ctrl_bytes_, workspace, ws_bytes, stream, {});
}

int twell_ffn_forward_timed(const uint16_t* x, const uint16_t* Wg, const uint16_t* WuT, const uint16_t* Wd,
                            int64_t M, int64_t d, int64_t F, int32_t T, int32_t C, float* y, void* ctrl,
                            size_t ctrl_bytes_, void* workspace, size_t ws_bytes, void* gate_begin,
                            void* gate_end, void* stream) {
  if (!gate_begin || !gate_end) return TWELL_E_INVALID_ARG;
  GateEvents ev;
  ev.begin = static_cast<hipEvent_t>(gate_begin);
  ev.end = static_cast<hipEvent_t>(gate_end);
  return ffn_forward_impl(x, Wg, WuT, Wd, M, d, F, T, C, y, ctrl, ctrl_bytes_, workspace, ws_bytes, stream, ev);
}

int twell_ffn_forward_static(const uint16_t* x, const uint16_t* Wg, const uint16_t* WuT, const uint16_t* Wd,
                             int64_t M, int64_t d, int64_t F, int32_t T, int32_t C, float* y, void* stream) {
  if (!Wg || !WuT || !Wd || (M != 0 && (!x || !y))) return TWELL_E_INVALID_ARG;
  int st = check_dims(M, d, F);
  if (st == TWELL_OK) st = check_tc(F, T, C);
  if (st == TWELL_OK) st = check_gate_offsets(M, d, F, T, C);
  if (st == TWELL_OK && M > twell::kFewRows) st = TWELL_E_UNSUPPORTED;
  if (st != TWELL_OK) return st;
  const StaticLayout L = static_layout(M, d, F, T, C);
  if (L.total > kStaticScratch) return TWELL_E_SCRATCH;
  if (M == 0) return TWELL_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* base = nullptr;
  st = static_scratch(s, &base);
  if (st != TWELL_OK) return st;
  twell_packed p;
  p.vals = reinterpret_cast<float*>(base + L.vals);
  p.idx = base + L.idx;
  p.counts = reinterpret_cast<uint16_t*>(base + L.counts);
  p.ovf_rows = reinterpret_cast<int32_t*>(base + L.ovf_rows);
  p.n_ovf = reinterpret_cast<int32_t*>(base + L.n_ovf);
  return few_rows_forward(x, Wg, WuT, Wd, M, d, F, T, C, y, base + L.ctrl, p,
                          reinterpret_cast<float*>(base + L.spill), reinterpret_cast<float*>(base + L.part),
                          L.total - L.part, s);
}

int twell_gateup_pack(const uint16_t* x, const uint16_t* Wg, const uint16_t* WuT, int64_t M, int64_t d,
                      int64_t F, int32_t T, int32_t C, const twell_packed* out, float* z_debug, float* h_debug,
                      void* ctrl, size_t ctrl_bytes_, void* stream) {
  if ((M != 0 && !x) || !Wg || !WuT || !packed_ok(out, M)) return TWELL_E_INVALID_ARG;
  if ((z_debug == nullptr) != (h_debug == nullptr)) return TWELL_E_INVALID_ARG;
  int st = check_dims(M, d, F);
  if (st == TWELL_OK) st = check_tc(F, T, C);
  if (st == TWELL_OK) st = check_gate_offsets(M, d, F, T, C);
  if (st == TWELL_OK) st = check_ctrl(M, ctrl, ctrl_bytes_);
  if (st != TWELL_OK) return st;
  return gateup_impl(x, Wg, WuT, M, d, F, T, C, out, z_debug, h_debug, static_cast<uint32_t*>(ctrl),
                     static_cast<hipStream_t>(stream));
}

int twell_hidden_down(const uint16_t* Wd, const twell_packed* in, int64_t M, int64_t d, int64_t F, int32_t T,
                      int32_t C, float* y, void* stream) {
  if (!Wd || !in) return TWELL_E_INVALID_ARG;
  if (M != 0 && (!y || !in->vals || !in->idx || !in->counts)) return TWELL_E_INVALID_ARG;
  int st = check_dims(M, d, F);
  if (st == TWELL_OK) st = check_tc(F, T, C);
  if (st == TWELL_OK && !twell::sliced_supports(d, F)) st = TWELL_E_UNSUPPORTED;
  if (st != TWELL_OK) return st;
  return hidden_down_impl(Wd, in, M, d, F, T, C, y, static_cast<hipStream_t>(stream));
}

int twell_ffn_forward_gateup(const uint16_t* x, const uint16_t* Wg, const uint16_t* WuT, const uint16_t* Wd,
                             int64_t M, int64_t d, int64_t F, int32_t T, int32_t C, float* y, void* ctrl,
                             size_t ctrl_bytes_, void* workspace, size_t ws_bytes, void* stream) {
  if (!Wg || !WuT || !Wd || (M != 0 && (!x || !y))) return TWELL_E_INVALID_ARG;
  int st = check_dims(M, d, F);
  if (st == TWELL_OK) st = check_tc(F, T, C);
  if (st == TWELL_OK) st = check_gate_offsets(M, d, F, T, C);
  if (st == TWELL_OK && !twell::sliced_supports(d, F)) st = TWELL_E_UNSUPPORTED;
  if (st == TWELL_OK) st = check_ctrl(M, ctrl, ctrl_bytes_);
  if (st == TWELL_OK) st = check_ws(TWELL_OP_FFN_FORWARD_GATEUP, M, d, F, T, C, workspace, ws_bytes);
  if (st != TWELL_OK) return st;
  if (M == 0) return TWELL_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const Layout L = layout(TWELL_OP_FFN_FORWARD_GATEUP, M, d, F, T, C);
  const twell_packed p = packed_in_ws(workspace, L);
  int dev = -1;
  if (stream_device(s, &dev) != TWELL_OK) return TWELL_E_HIP;
  std::lock_guard<std::mutex> lock(g_side_mu);
  SideStream* ss = nullptr;
  st = side_stream_locked(dev, &ss);
  if (st != TWELL_OK) return st;
  st = gateup_impl(x, Wg, WuT, M, d, F, T, C, &p, nullptr, nullptr, static_cast<uint32_t*>(ctrl), s);
  if (st != TWELL_OK) return st;
  if (hipEventRecord(ss->fork, s) != hipSuccess || hipStreamWaitEvent(ss->s, ss->fork, 0) != hipSuccess)
    return TWELL_E_HIP;
  const int st_fb = dense_impl(x, Wg, WuT, Wd, M, d, F, p.ovf_rows, p.n_ovf, at<uint16_t>(workspace, L.h_hi),
                               at<uint16_t>(workspace, L.h_lo), y, at<float>(workspace, L.split),
                               true, ss->s, ring_region(workspace, L, M, d, F));
  const bool joined = hipEventRecord(ss->join, ss->s) == hipSuccess;
  st = hidden_down_impl(Wd, &p, M, d, F, T, C, y, s);
  if (!joined || hipStreamWaitEvent(s, ss->join, 0) != hipSuccess) return TWELL_E_HIP;
  return st != TWELL_OK ? st : st_fb;
}

int twell_dense_ffn_forward(const uint16_t* x, const uint16_t* Wg, const uint16_t* WuT,
                            const uint16_t* Wd, int64_t M, int64_t d, int64_t F, float* y,
                            void* workspace, size_t ws_bytes, void* stream) {
  if (!Wg || !WuT || !Wd || (M != 0 && (!x || !y))) return TWELL_E_INVALID_ARG;
  int st = check_dims(M, d, F);
  if (st == TWELL_OK && F % 64 != 0) st = TWELL_E_UNSUPPORTED;
  if (st == TWELL_OK) st = check_ws(TWELL_OP_DENSE_FFN, M, d, F, 0, 0, workspace, ws_bytes);
  if (st != TWELL_OK) return st;
  const Layout L = layout(TWELL_OP_DENSE_FFN, M, d, F, 0, 0);
  if (M != 0 && twell::dense_ring_supports(M, d, F)) {
    twell::DenseArgs a{};
    a.x = x;
    a.Wg = Wg;
    a.WuT = WuT;
    a.Wd = Wd;
    a.M = int(M);
    a.d = int(d);
    a.F = int(F);
    a.h_hi = at<uint16_t>(workspace, L.h_hi);
    a.y = y;
    return hip_status(twell::launch_dense_ring(a, at<uint8_t>(workspace, L.ring), static_cast<hipStream_t>(stream)));
  }
  return dense_impl(x, Wg, WuT, Wd, M, d, F, nullptr, nullptr, at<uint16_t>(workspace, L.h_hi),
                    nullptr, y, nullptr, false, static_cast<hipStream_t>(stream));
}

int twell_column_activity(const uint16_t* x, const uint16_t* Wg, int64_t M, int64_t d, int64_t F,
                          int32_t T, int32_t C, uint32_t* active_bits, void* ctrl, size_t ctrl_bytes_,
                          void* workspace, size_t ws_bytes, void* stream) {
  if ((M != 0 && !x) || !Wg || !active_bits) return TWELL_E_INVALID_ARG;
  int st = check_dims(M, d, F);
  if (st == TWELL_OK) st = check_tc(F, T, C);
  if (st == TWELL_OK) st = check_gate_offsets(M, d, F, T, C);
  if (st == TWELL_OK) st = check_ctrl(M, ctrl, ctrl_bytes_);
  if (st == TWELL_OK) st = check_ws(TWELL_OP_COLUMN_ACTIVITY, M, d, F, T, C, workspace, ws_bytes);
  if (st != TWELL_OK) return st;
  if (M == 0) return TWELL_OK;
  const twell_packed p = packed_in_ws(workspace, layout(TWELL_OP_COLUMN_ACTIVITY, M, d, F, T, C));
  return gate_pack_impl(x, Wg, M, d, F, T, C, &p, nullptr, static_cast<uint32_t*>(ctrl),
                        static_cast<hipStream_t>(stream), active_bits);
}

int twell_live_layout(const uint32_t* active_bits, int64_t F, int32_t T, int32_t* src, int64_t cap,
                      int64_t* width) {
  if (!active_bits || !width || F <= 0 || F > kMaxF || T < 1) return TWELL_E_INVALID_ARG;
  int64_t live = 0;
  for (int64_t j = 0; j < F; ++j) live += (active_bits[j >> 5] >> (j & 31)) & 1u;
  const int64_t w = std::max<int64_t>(T, (live + T - 1) / T * T);
  *width = w;
  if (src == nullptr) return TWELL_OK;
  if (cap < w) return TWELL_E_INVALID_ARG;
  int64_t i = 0;
  for (int64_t j = 0; j < F; ++j)
    if ((active_bits[j >> 5] >> (j & 31)) & 1u) src[i++] = static_cast<int32_t>(j);
  for (; i < w; ++i) src[i] = -1;
  return TWELL_OK;
}

int twell_gather_rows(const uint16_t* W, int64_t F, int64_t d, const int32_t* src, int64_t n,
                      uint16_t* out, void* stream) {
  if (n < 0) return TWELL_E_INVALID_ARG;
  if (n == 0) return TWELL_OK;
  if (!W || !src || !out) return TWELL_E_INVALID_ARG;
  int st = check_dims(1, d, F);
  if (st != TWELL_OK) return st;
  if (n > kMaxF) return TWELL_E_INVALID_ARG;
  return hip_status(twell::launch_gather_rows(W, int(F), int(d), src, int(n), out,
                                              static_cast<hipStream_t>(stream)));
}

size_t twell_workspace_bytes(int32_t op, int64_t M, int64_t d, int64_t F, int32_t T, int32_t C) {
  if (check_dims(M, d, F) != TWELL_OK) return 0;
  if (op == TWELL_OP_GATE_PACK || op == TWELL_OP_FFN_FORWARD || op == TWELL_OP_SLICED_UPDOWN ||
      op == TWELL_OP_COLUMN_ACTIVITY || op == TWELL_OP_FFN_FORWARD_GATEUP) {
    if (check_tc(F, T, C) != TWELL_OK) return 0;
    if ((op == TWELL_OP_SLICED_UPDOWN || op == TWELL_OP_FFN_FORWARD_GATEUP) && !twell::sliced_supports(d, F))
      return 0;
  } else if (op == TWELL_OP_DENSE_FFN || op == TWELL_OP_DENSE_FALLBACK) {
    if (F % 64 != 0) return 0;
    T = 0;
    C = 0;
  } else {
    return 0;
  }
  return layout(op, M, d, F, T, C).total;
}

size_t twell_ctrl_bytes(int64_t M) {
  if (M < 0 || M > kMaxM) return 0;
  return ctrl_bytes(M);
}

int twell_packed_view(void* workspace, size_t ws_bytes, int64_t M, int64_t d, int64_t F,
                      int32_t T, int32_t C, twell_packed* out) {
  if (!out) return TWELL_E_INVALID_ARG;
  int st = check_dims(M, d, F);
  if (st == TWELL_OK) st = check_tc(F, T, C);
  if (st == TWELL_OK) st = check_ws(TWELL_OP_FFN_FORWARD, M, d, F, T, C, workspace, ws_bytes);
  if (st != TWELL_OK) return st;
  *out = packed_in_ws(workspace, layout(TWELL_OP_FFN_FORWARD, M, d, F, T, C));
  return TWELL_OK;
}

const char* twell_status_string(int32_t status) {
  switch (status) {
    case TWELL_OK: return "ok";
    case TWELL_E_INVALID_ARG: return "invalid argument (null pointer or bad dimension)";
    case TWELL_E_UNSUPPORTED: return "unsupported shape (T, C, F % T or d)";
    case TWELL_E_WORKSPACE: return "workspace missing, misaligned or too small";
    case TWELL_E_HIP: return "HIP launch failed";
    case TWELL_E_SCRATCH: return "shape needs more scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

int32_t twell_abi_version(void) { return TWELL_ABI_VERSION; }

}  // extern "C"
