/* twell.h — C ABI of libtwell.so: TwELL sparse gated-FFN forward on MI355X (gfx950).
 *
 * The layer computed is the ReLU-gated FFN
 *     y = (ReLU(x Wg^T) ⊙ (x Wu^T)) Wd
 * (a Llama-style gated FFN with its SiLU gate replaced by ReLU: Tencent Cloud
 * article "一文读懂 NVIDIA 与 Sakana AI 联手打造的稀疏 LLM 黑科技", section 1;
 * aimodeling.com TwELL news summary, paragraph 4). When the gate is mostly
 * zero, the gate GEMM packs its non-zeros per column tile into TwELL in its
 * epilogue and a fused kernel does the up and down projections over the packed
 * non-zeros only (Telegram post on TwELL at tgviewer.app, parts "Вот тут и
 * решает TwELL" and "Инференс"; aimodeling.com summary, paragraph 3).
 *
 * Conventions for every entry point
 *  - bf16 tensors are passed as raw uint16_t bit patterns.
 *  - Every array argument is a DEVICE pointer to row-major, contiguous memory
 *    allocated and owned by the caller. The library never allocates or frees
 *    device memory. What it keeps per GPU for the process: the static buffer
 *    of twell_ffn_forward_static, and a side stream with two events that
 *    twell_ffn_forward creates on its first call on that GPU (above 256 rows).
 *  - Weights are all [F, d] row-major, row j belonging to hidden unit j:
 *      Wg  = gate_proj.weight, WuT = up_proj.weight,
 *      Wd  = down_proj.weight transposed (row j = the d outputs unit j feeds).
 *    So every per-unit gather of the fused kernel reads one contiguous row.
 *  - x is [M, d] bf16; y is [M, d] fp32.
 *  - All work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *    void*; NULL = the default stream). Errors found on the host are returned
 *    before anything is enqueued; execution errors surface at the caller's
 *    stream synchronisation. No exception crosses the ABI.
 *  - Shape limits: 0 <= M <= 2^30 and 0 < F <= 2^24 (larger values return
 *    TWELL_E_INVALID_ARG); d % 256 == 0 and 256 <= d <= 8192;
 *    F % T == 0; T in {64, 128}; 1 <= C <= T. Calls that run the
 *    gate (twell_gate_pack, twell_column_activity, twell_ffn_forward) also
 *    need M d 2, F d 2 and M (F / T) C 4 below 2^31 bytes (32-bit offsets);
 *    larger shapes return TWELL_E_UNSUPPORTED (split the batch).
 *  - Workspace: a caller-owned device scratch buffer of at least
 *    twell_workspace_bytes(op, ...) bytes, 256-byte aligned, contents
 *    irrelevant. One workspace must not be used by two calls that may run
 *    concurrently.
 *  - Control block (twell_gate_pack, twell_dense_fallback, twell_ffn_forward):
 *    a caller-owned device buffer of at least twell_ctrl_bytes(M) bytes,
 *    256-byte aligned, used only for this purpose. It must be zero-filled
 *    before its first use; every call leaves it zero-filled again when it
 *    completes (stream order), so one buffer sized for the largest M serves
 *    every later call. It holds the overflow-set counters, one deduplication
 *    flag per row and the arrival counters of the few-row forward's split
 *    rows (twell_dense_fallback checks it but no longer writes it: its split
 *    products are added by reduce launches).
 *    Calls sharing a control block must not run concurrently.
 *  - With M == 0 nothing is computed; x and y may then be NULL.
 */
#ifndef TWELL_H_
#define TWELL_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TWELL_ABI_VERSION 7

/* Status codes. */
#define TWELL_OK 0
#define TWELL_E_INVALID_ARG (-1) /* null pointer, negative or zero dimension, M too large */
#define TWELL_E_UNSUPPORTED (-2) /* F % T != 0, T not in {64,128}, C out of [1,T], d not supported */
#define TWELL_E_WORKSPACE (-3)   /* workspace or control block null, misaligned or too small */
#define TWELL_E_HIP (-4)         /* a HIP launch failed (hipGetLastError) */
#define TWELL_E_SCRATCH (-5)     /* twell_ffn_forward_static: shape past its static buffer */

/* Operations for twell_workspace_bytes. */
#define TWELL_OP_GATE_PACK 0
#define TWELL_OP_FFN_FORWARD 1
#define TWELL_OP_DENSE_FFN 2
#define TWELL_OP_DENSE_FALLBACK 3
#define TWELL_OP_SLICED_UPDOWN 4
#define TWELL_OP_COLUMN_ACTIVITY 5
#define TWELL_OP_FFN_FORWARD_GATEUP 6

/* TwELL packing of ReLU(x Wg^T) with tile width T and capacity C
 * (the format: tgviewer.app Telegram post, part "Вот тут и решает TwELL";
 * Tencent Cloud article, section 2). nT = F / T tiles per row.
 *   vals   [M, nT, C] fp32  gate value ReLU(z) of the s-th active unit of tile t
 *   idx    [M, nT, C] u8    its tile-local column (0..T-1), strictly ascending in s
 *   counts [M, nT]    u16   number of active units (z > 0) in the tile, NOT clamped
 *   ovf_rows [M]      i32   rows with some counts[r][t] > C, order unspecified
 *   n_ovf  [1]        i32   number of valid entries of ovf_rows
 * Only slots s < min(counts, C) are written; other slots are left untouched.
 * Overflow rows still hold the first C active units of every tile. */
typedef struct twell_packed {
  float* vals;
  uint8_t* idx;
  uint16_t* counts;
  int32_t* ovf_rows;
  int32_t* n_ovf;
} twell_packed;

/* Gate GEMM with the TwELL packing in its epilogue (aimodeling.com summary,
 * paragraph 3; pulsen.vercel.app article, paragraph on tile matching; Tencent
 * Cloud article, section 2): z = x Wg^T in fp32 from bf16 MFMA products, then
 * ReLU and the per-tile packing of `out`, in one launch and without writing z.
 * z_debug: optional [M, F] fp32; when non-NULL every pre-activation z is also
 * stored (for bit-exact checks of the packing), otherwise pass NULL.
 * ctrl: control block of >= twell_ctrl_bytes(M) bytes (see above). */
int twell_gate_pack(const uint16_t* x, const uint16_t* Wg, int64_t M, int64_t d, int64_t F,
                    int32_t T, int32_t C, const twell_packed* out, float* z_debug,
                    void* ctrl, size_t ctrl_bytes, void* stream);

/* Fused up+down projection over a TwELL packing (tgviewer.app Telegram post,
 * part "Инференс"; aimodeling.com summary, paragraph 3): for every row that is
 * not an overflow row, y[r] = sum over stored units j of
 * g_j * (x[r] . WuT[j]) * Wd[j], with fp32 accumulation. The hidden vector is
 * never written to memory. Rows with some count > C are NOT written (the dense
 * fallback owns them). `in` is what twell_gate_pack produced with the same
 * M, F, T, C. */
int twell_fused_updown(const uint16_t* x, const uint16_t* WuT, const uint16_t* Wd,
                       const twell_packed* in, int64_t M, int64_t d, int64_t F, int32_t T,
                       int32_t C, float* y, void* stream);

/* The operation of twell_fused_updown, computed for MI355X's 8 XCDs: the d
 * columns are cut into 8 slices and the workgroups of XCD k gather only slice k
 * of WuT and Wd, F * d / 8 bf16 per matrix, which stays in that XCD's L2
 * (which rows are gathered and what is summed are as in the pages' inference
 * kernel: tgviewer.app Telegram post, part "Инференс"; aimodeling.com summary,
 * paragraph 3). Three launches: the first turns each row's TwELL tiles into
 * one contiguous list of (unit, gate value) entries in (tile, slot) order and
 * its length (-1 for an overflow row); the second stores, per listed unit and
 * slice, g_j * (x_r . WuT[j]) over that slice's columns; the third sums the 8
 * partials of each unit in slice order and accumulates h_j * Wd[j] over its
 * slice. Same contract for y as twell_fused_updown (overflow rows untouched).
 * workspace: >= twell_workspace_bytes(TWELL_OP_SLICED_UPDOWN, ...)
 * = 8 M (F / T) C fp32 partials, M (F / T) C 8-byte list entries and M
 * lengths, each rounded up to 256 bytes.
 * d must be one of 256, 512, 768, 1024, 1280, 1536, 1792, 2048, 2560, 3072,
 * 3584, 4096, 5120, 6144, 7168, 8192 (d / 64 = 2^a * b with b in {1, 3, 5, 7})
 * and F * d * 2 < 2^31 (each weight matrix below 2 GiB), otherwise
 * TWELL_E_UNSUPPORTED. */
int twell_sliced_updown(const uint16_t* x, const uint16_t* WuT, const uint16_t* Wd,
                        const twell_packed* in, int64_t M, int64_t d, int64_t F, int32_t T,
                        int32_t C, float* y, void* workspace, size_t ws_bytes, void* stream);

/* Dense fallback for the overflow rows of a packing (rows that do not fit the
 * sparse block go to a dense path: tgviewer.app Telegram post, part
 * "Обучение"; Tencent Cloud article, section 3). For the *in->n_ovf rows listed
 * in in->ovf_rows it computes y[r] = (ReLU(x_r Wg^T) ⊙ x_r WuT^T) Wd with bf16
 * MFMA products, fp32 accumulation and the hidden vector carried as a bf16
 * hi/lo pair. n_ovf is read on the device (no host synchronisation); other rows
 * of y are untouched. When the list is short the K loops are split over more
 * workgroups, and a reduce launch after each product adds their partial
 * tiles in a fixed order (deterministic). When M is large enough for the list
 * to fill the device without splitting (256 output tiles of its down product:
 * 7937 rows at d = 2048), the call also enqueues kernels that take a list of
 * that length instead (the workspace then also receives Wd^T); which ones do
 * the work is decided on the device from n_ovf, and the results are the same
 * bits whichever entry (this one, twell_ffn_forward, the gate-only forward)
 * ran the fallback.
 * ctrl: >= twell_ctrl_bytes(M) (see above);
 * workspace: >= twell_workspace_bytes(TWELL_OP_DENSE_FALLBACK, ...). */
int twell_dense_fallback(const uint16_t* x, const uint16_t* Wg, const uint16_t* WuT,
                         const uint16_t* Wd, const twell_packed* in, int64_t M, int64_t d,
                         int64_t F, float* y, void* ctrl, size_t ctrl_bytes, void* workspace,
                         size_t ws_bytes, void* stream);

/* The whole sparse forward of the layer: the gate kernel that leaves its
 * non-zeros in TwELL, then the kernel that does the up and down projections
 * from that packing without a dense hidden matrix (the two inference kernels:
 * tgviewer.app Telegram post, part "Инференс"; aimodeling.com summary,
 * paragraph 3; the gate epilogue feeding a fused up/down pipeline: Tencent
 * Cloud article, section 2), plus the dense path for rows that overflow the
 * packing (Telegram post, part "Обучение"; Tencent Cloud article, section 3).
 * No host synchronisation, the packing kept in the workspace (see
 * twell_packed_view); y [M, d] fp32 is fully written.
 * Above 256 rows: twell_gate_pack, then twell_sliced_updown (twell_fused_updown
 * for the d that the sliced form does not support) on `stream` and, at the
 * same time, twell_dense_fallback on a side stream of the same GPU (forked
 * after the gate, joined into `stream` before the call returns, so work the
 * caller enqueues on `stream` afterwards sees the whole y). The side stream
 * and its two events are created on the first such call on a GPU (call it
 * once outside HIP graph capture first) and serialise the fallbacks of
 * concurrent callers on that GPU.
 * Up to 256 rows: the gate also keeps every z of each (row, tile) whose count
 * exceeds C in the workspace, and the fused kernel does overflow rows from it
 * (their whole active set, still only gathers): two launches, no fallback;
 * for a few tokens (fewer than 128 gate tiles of 32 tokens x 128 units,
 * d <= 2048) the gate splits its K over workgroups in a first launch, with
 * the same sums in the same order, so the packing is bit-identical to
 * twell_gate_pack's.
 * ctrl: >= twell_ctrl_bytes(M); workspace: >= twell_workspace_bytes(TWELL_OP_FFN_FORWARD, ...). */
int twell_ffn_forward(const uint16_t* x, const uint16_t* Wg, const uint16_t* WuT,
                      const uint16_t* Wd, int64_t M, int64_t d, int64_t F, int32_t T, int32_t C,
                      float* y, void* ctrl, size_t ctrl_bytes, void* workspace, size_t ws_bytes,
                      void* stream);

/* twell_ffn_forward, plus two caller-created HIP events (hipEvent_t passed as
 * void*, created with timing enabled, owned by the caller) recorded on
 * `stream` right before the gate's launches and right after them (at most 256
 * rows: the K-split and packing launches of the small-batch gate), so that
 * hipEventElapsedTime gives the gate's time inside the forward, next to the
 * up/down kernels it alternates with. Same kernels, arguments and result as
 * twell_ffn_forward; M = 0 records nothing. Both events non-null, else
 * TWELL_E_INVALID_ARG; a failed record gives TWELL_E_HIP. */
int twell_ffn_forward_timed(const uint16_t* x, const uint16_t* Wg, const uint16_t* WuT,
                            const uint16_t* Wd, int64_t M, int64_t d, int64_t F, int32_t T,
                            int32_t C, float* y, void* ctrl, size_t ctrl_bytes, void* workspace,
                            size_t ws_bytes, void* gate_begin, void* gate_end, void* stream);

/* Allocation-free form of twell_ffn_forward, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops that forbid
 * hipMalloc): no workspace or control block is passed. Up to 256 rows (the
 * decode and batched-decode range), the same kernels and the same result, bit
 * for bit, as twell_ffn_forward; y [M, d] fp32 is fully written.
 * Scratch: one static device buffer of TWELL_STATIC_SCRATCH_BYTES per GPU,
 * held from the library's first use on that GPU until the process ends. It
 * holds a control block sized for 256 rows, the packing (M (F/T) C 5 +
 * M (F/T) 2 + 4 M bytes), the z of overflowing tiles (M F 4 bytes) and the
 * partial rows of long rows (min(16, 512 / M) M d 4 bytes) or, where larger,
 * the gate's K-split partial sums (up to 128 rows, while fewer than 256 tiles
 * of 32 rows x 128 units: 64 KB a tile), each rounded up to 256 bytes. Every call on one GPU uses the same buffer: calls that may
 * overlap on a GPU (several streams or threads) race, and the caller must
 * order them. Returns TWELL_E_UNSUPPORTED for M > 256, TWELL_E_SCRATCH when
 * the shape needs more than the buffer, TWELL_E_HIP when the buffer's device
 * address cannot be taken; argument rules otherwise as twell_ffn_forward. */
#define TWELL_STATIC_SCRATCH_BYTES (32u << 20)
int twell_ffn_forward_static(const uint16_t* x, const uint16_t* Wg, const uint16_t* WuT,
                             const uint16_t* Wd, int64_t M, int64_t d, int64_t F, int32_t T,
                             int32_t C, float* y, void* stream);

/* Dense MFMA gated-FFN baseline (the comparator the pages measure against:
 * dense matmuls, tgviewer.app Telegram post, paragraph after "Обучение"):
 * h = ReLU(x Wg^T) ⊙ (x WuT^T) rounded to bf16 and written to the workspace,
 * then y = h Wd in fp32. The workspace also receives a transposed copy of Wd
 * and, when the down product's K range is split across workgroups, the
 * partial outputs that are added to y in split order (fixed order: two calls
 * give the same bits). workspace: >= twell_workspace_bytes(TWELL_OP_DENSE_FFN, ...). */
int twell_dense_ffn_forward(const uint16_t* x, const uint16_t* Wg, const uint16_t* WuT,
                            const uint16_t* Wd, int64_t M, int64_t d, int64_t F, float* y,
                            void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------ gate-only variant
 * A variant of the forward that the pages do not describe, for densities
 * where gathering one WuT row per stored unit costs more than a dense up
 * product: the gate and up products are dense (one MFMA kernel reading one x
 * tile for both) and the TwELL packing holds the hidden value
 * h = ReLU(z) * u; only the down product gathers, one Wd row per stored unit.
 * The active set is still the gate's (z > 0; the gate decides which units
 * are live: Tencent Cloud article, section 1), so counts, slots, tile-local
 * indices and the overflow set are those twell_gate_pack gives; a stored h
 * may be zero or negative. Overflow rows take the dense fallback. */

/* Dense gate and up products with h packed in its epilogue: `out` as for
 * twell_gate_pack except that vals hold h (fp32, from fp32 z and u).
 * z_debug, h_debug: both NULL, or both [M, F] fp32 receiving every z and
 * every h = ReLU(z) u (for bit-exact checks of the packing).
 * ctrl: >= twell_ctrl_bytes(M). */
int twell_gateup_pack(const uint16_t* x, const uint16_t* Wg, const uint16_t* WuT, int64_t M, int64_t d,
                      int64_t F, int32_t T, int32_t C, const twell_packed* out, float* z_debug,
                      float* h_debug, void* ctrl, size_t ctrl_bytes, void* stream);

/* Down product from a packing of h (twell_gateup_pack): for every row that is
 * not an overflow row, y[r] = sum over stored units j of h_j * Wd[j] in fp32;
 * overflow rows of y are not written. Gathers d / 8 columns of Wd per XCD,
 * as twell_sliced_updown does; d and F as for that call. */
int twell_hidden_down(const uint16_t* Wd, const twell_packed* in, int64_t M, int64_t d, int64_t F,
                      int32_t T, int32_t C, float* y, void* stream);

/* The whole gate-only forward: twell_gateup_pack, then twell_hidden_down on
 * `stream` and the dense fallback of overflow rows on the side stream (as in
 * twell_ffn_forward); y [M, d] fp32 fully written. The packing sits at the
 * start of the workspace, where twell_packed_view finds it given a workspace
 * of twell_workspace_bytes(TWELL_OP_FFN_FORWARD, ...) bytes.
 * ctrl: >= twell_ctrl_bytes(M); workspace: >=
 * twell_workspace_bytes(TWELL_OP_FFN_FORWARD_GATEUP, ...). */
int twell_ffn_forward_gateup(const uint16_t* x, const uint16_t* Wg, const uint16_t* WuT,
                             const uint16_t* Wd, int64_t M, int64_t d, int64_t F, int32_t T,
                             int32_t C, float* y, void* ctrl, size_t ctrl_bytes, void* workspace,
                             size_t ws_bytes, void* stream);

/* Dead gate units (pulsen.vercel.app article, dead-neuron paragraph: at the
 * recommended L1 coefficient over 30% of the units are never active; Tencent
 * Cloud article, section 6). A unit that no token activates adds exact zeros
 * to every output row, so dropping its rows from Wg, WuT and Wd leaves y
 * unchanged for inputs that keep it inactive, and shrinks the gate product.
 * The three calls below find such units over calibration batches and build
 * the compacted layer; twell_ffn_forward then runs on it unchanged (F = the
 * compacted width). */

/* Gate GEMM of x with the activity of every unit recorded: bit (j % 32) of
 * active_bits[j / 32] is ORed with 1 when z_j = x_r . Wg_j > 0 for some row r
 * (the packing's activity test, in the same fp32 arithmetic). active_bits:
 * device [ceil(F / 32)] uint32, zeroed by the caller before the first batch;
 * calls accumulate, so several batches give the union. ctrl: >=
 * twell_ctrl_bytes(M); workspace: >= twell_workspace_bytes(TWELL_OP_COLUMN_ACTIVITY,
 * ...), holds a packing that is discarded. */
int twell_column_activity(const uint16_t* x, const uint16_t* Wg, int64_t M, int64_t d, int64_t F,
                          int32_t T, int32_t C, uint32_t* active_bits, void* ctrl, size_t ctrl_bytes,
                          void* workspace, size_t ws_bytes, void* stream);

/* HOST function (no GPU work): the compacted layout from activity bits. The
 * active units in ascending order, then -1 (a zero row) up to the next
 * multiple of T; at least T entries. active_bits: host [ceil(F / 32)] as
 * written by twell_column_activity; T >= 1. *width receives the compacted
 * width; src: host [cap] int32 receives the source unit of each compacted
 * unit, or NULL to query the width only. TWELL_E_INVALID_ARG when cap <
 * width (nothing is written to src then). */
int twell_live_layout(const uint32_t* active_bits, int64_t F, int32_t T, int32_t* src, int64_t cap,
                      int64_t* width);

/* out[i] = W[src[i]] for i < n, a zero row where src[i] < 0 or src[i] >= F.
 * W: device [F, d] bf16; src: device [n] int32; out: device [n, d] bf16, not
 * overlapping W. d as for the other calls. One call per weight matrix builds
 * the compacted Wg, WuT and Wd from one src. */
int twell_gather_rows(const uint16_t* W, int64_t F, int64_t d, const int32_t* src, int64_t n,
                      uint16_t* out, void* stream);

/* ------------------------------------------------------------ training
 * Hybrid training format (tgviewer.app Telegram post, part "Обучение";
 * Tencent Cloud article, section 3): each row of ReLU(x Wg^T) is either one
 * sparse block of width K (the same for every row) holding the row's active
 * units, or, with more than K active units, a dense row in a reserve of R
 * rows. With it the backward pass below multiplies no two dense matrices.
 *   idx      [M, K] int32 global unit of slot s, ascending, s < count; for a
 *                   reserve row slot 0 holds its reserve slot instead
 *   vals     [M, K] fp32  g = ReLU(z) of that unit
 *   count    [M]    int32 active units of the row (> K: the row is in the reserve)
 *   res_rows [R]    int32 rows held densely, order unspecified, first *n_res valid
 *   res_vals [R, F] fp32  their dense g rows
 *   n_res    [1]    int32 rows that needed the reserve; when it exceeds R the
 *                   reserve is incomplete and a backward over it is not valid */
typedef struct twell_hybrid {
  int32_t* idx;
  float* vals;
  int32_t* count;
  int32_t* res_rows;
  float* res_vals;
  int32_t* n_res;
} twell_hybrid;

/* Spill list of the training gate: every pre-activation z of each (row,
 * tile) whose count exceeds C, so that a packing of small capacity C still
 * loses no active unit (the hybrid format needs them all) without the
 * M * F * 5 bytes of a C = T packing.
 *   z       [cap, T] fp32  record k: the T values z of one (row, tile)
 *   slot    [M, F/T] int32 record of (row, tile) where counts[row][tile] > C;
 *                          other entries are not written
 *   n_spill [1]      int32 records needed; when it exceeds cap the records
 *                          past cap were not stored and the list is incomplete
 *   cap              records z holds (0 <= cap < 2^31 / T); z and slot are
 *                    non-NULL whenever M > 0 */
typedef struct twell_spill {
  float* z;
  int32_t* slot;
  int32_t* n_spill;
  int64_t cap;
} twell_spill;

/* The gate of the training path: twell_gate_pack's output (any C), plus the
 * spill list of the tiles that overflow C. The kernel is twell_gate_pack's
 * large-batch one at every M (above 256 rows its packing and z are the same
 * bits). z_debug: optional [M, F] fp32 receiving every z, as in
 * twell_gate_pack. ctrl: >= twell_ctrl_bytes(M). */
int twell_gate_pack_spill(const uint16_t* x, const uint16_t* Wg, int64_t M, int64_t d, int64_t F,
                          int32_t T, int32_t C, const twell_packed* out, const twell_spill* spill,
                          float* z_debug, void* ctrl, size_t ctrl_bytes, void* stream);

/* The hybrid format from a TwELL packing and, for C < T, the spill list of
 * the same call of twell_gate_pack_spill (tiles over C are read from their
 * records); with C == T no tile overflows and spill may be NULL. K >= 1;
 * 0 <= R <= M. The format is valid when *n_res <= R and, with a spill list,
 * *n_spill <= its cap. */
int twell_hybrid_pack(const twell_packed* in, const twell_spill* spill, int64_t M, int64_t F, int32_t T,
                      int32_t C, int32_t K, int64_t R, const twell_hybrid* out, void* stream);

/* Workspace bytes of twell_ffn_backward (0 for invalid arguments). */
size_t twell_backward_workspace_bytes(int64_t M, int64_t d, int64_t F, int32_t K, int64_t R);

/* Gradients of y = (ReLU(x Wg^T) ⊙ x WuT^T) Wd for upstream gradient dy
 * (bf16 [M, d]), over the hybrid format `hy` of this x (twell_hybrid_pack):
 * dx [M, d], dWg, dWuT, dWd [F, d], all fp32 and overwritten. Only active
 * units enter (their dZ, dU and h are the only non-zeros): per token, row
 * gathers of WuT, Wd and Wg; per unit, gathers of the x and dy rows of its
 * tokens in token order. Sums have a fixed order (deterministic).
 * d: multiples of 512 up to 8192, or odd multiples of 256 below 4096;
 * F <= 16384; M K + R F < 2^31. workspace >= twell_backward_workspace_bytes(...). */
int twell_ffn_backward(const uint16_t* x, const uint16_t* Wg, const uint16_t* WuT, const uint16_t* Wd,
                       const uint16_t* dy, const twell_hybrid* hy, int64_t M, int64_t d, int64_t F,
                       int32_t K, int64_t R, float* dx, float* dWg, float* dWuT, float* dWd,
                       void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes an operation needs (0 for invalid arguments). T and C are
 * ignored for TWELL_OP_DENSE_FFN and TWELL_OP_DENSE_FALLBACK;
 * TWELL_OP_GATE_PACK needs none (0 is a valid size for it). */
size_t twell_workspace_bytes(int32_t op, int64_t M, int64_t d, int64_t F, int32_t T, int32_t C);

/* Control-block bytes for up to M rows (0 for M < 0 or M too large). */
size_t twell_ctrl_bytes(int64_t M);

/* Where twell_ffn_forward keeps its packing inside `workspace` (host-side
 * pointer arithmetic only; nothing is enqueued). Valid after that call has
 * completed on its stream. */
int twell_packed_view(void* workspace, size_t ws_bytes, int64_t M, int64_t d, int64_t F,
                      int32_t T, int32_t C, twell_packed* out);

/* Static string for a status code; never NULL. */
const char* twell_status_string(int32_t status);

/* TWELL_ABI_VERSION of the built library. */
int32_t twell_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TWELL_H_ */
