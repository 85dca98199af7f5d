"""Plain, slow, fp64 CPU oracle of the TwELL sparse gated-FFN forward.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.

Sources (cited by page title and section; the pages print no code and no
worked numeric example):

* [aimodeling] "TwELL: Sakana AI and NVIDIA ... sparse LLM inference 20% faster"
  (aimodeling.com news summary), paragraphs 1, 3 and 4.
* [tgviewer] Telegram post on TwELL (tgviewer.app, ai_machinelearning_big_data),
  parts "Вот тут и решает TwELL" (the format), "Инференс" (fused kernel) and
  "Обучение" (hybrid format).
* [pulsen] "Sakana AI og NVIDIA introduserer TwELL" (pulsen.vercel.app), the
  paragraphs on tile matching and on the sparsification recipe.
* [tencent] "一文读懂 NVIDIA 与 Sakana AI 联手打造的稀疏 LLM 黑科技"
  (developer.cloud.tencent.com.cn), sections 1, 2 and 3.

Every function states the passage it follows. Where the pages leave a step
open, the reading taken is stated next to it. Precision: bf16 inputs are
widened exactly to fp64; all products of two bf16 numbers are exact in fp64.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import scipy.sparse as sps


# --------------------------------------------------------------------------- inputs
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly.

    A bf16 number is the upper half of an IEEE-754 binary32 number, so placing
    the 16 bits in the high half of a 32-bit word gives the same value, which
    widens to binary64 without rounding.
    """
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ dense definition
def gate_preactivations(x: np.ndarray, Wg: np.ndarray, rows=None) -> np.ndarray:
    """Z = x Wg^T in fp64, shape [M, F] (or [len(rows), F]).

    The gate projection of a Llama-style gated FFN, whose sign pattern decides
    which hidden units are live ([tencent] section 1). Wg is stored [F, d] with
    row j belonging to hidden unit j.
    """
    X = decode_bf16(x if rows is None else x[rows])
    return X @ decode_bf16(Wg).T


def dense_gated_ffn(x, Wg, WuT, Wd, rows=None, chunk: int = 512) -> np.ndarray:
    """y = (ReLU(x Wg^T) ⊙ (x WuT^T)) Wd in fp64.

    The ReLU-gated FFN: a Llama-style gated FFN ([tencent] section 1) whose
    SiLU gate is replaced by ReLU ([aimodeling] paragraph 4; [pulsen], recipe
    paragraph). Reading: no biases. WuT is up_proj.weight ([F, d]); Wd is
    down_proj.weight transposed ([F, d], row j = the output row of unit j).
    """
    r_all = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
    G = decode_bf16(Wg)
    U = decode_bf16(WuT)
    D = decode_bf16(Wd)
    out = np.empty((len(r_all), D.shape[1]), dtype=np.float64)
    for s in range(0, len(r_all), chunk):
        X = decode_bf16(x[r_all[s:s + chunk]])
        Z = X @ G.T
        H = np.maximum(Z, 0.0) * (X @ U.T)
        out[s:s + chunk] = H @ D
    return out


# ---------------------------------------------------------------------- TwELL format
@dataclass
class TwellPacking:
    """Tile-wise ELL of the gate output, per (row r, tile t).

    counts[r, t]     number of active units in columns [t*T, (t+1)*T) (not clamped)
    idx[r, t, s]     tile-local column of the s-th active unit, ascending in s
    vals[r, t, s]    its gate value ReLU(z) (same dtype as the packed input)
    ovf              sorted rows with some counts[r, t] > C
    Slots s >= min(counts[r, t], C) hold 0 here (they are unspecified on the GPU).
    """

    counts: np.ndarray  # uint16 [M, F/T]
    idx: np.ndarray  # uint8  [M, F/T, C]
    vals: np.ndarray  # float  [M, F/T, C]
    ovf: np.ndarray  # int64 sorted
    T: int
    C: int

    @property
    def n_tiles(self) -> int:
        return self.counts.shape[1]


def pack_twell(Z: np.ndarray, T: int, C: int) -> TwellPacking:
    """Pack ReLU(Z) into TwELL with tile width T and C slots per (row, tile).

    The format ([tgviewer] "Вот тут и решает TwELL"; [tencent] section 2;
    [aimodeling] paragraph 3): the columns of the gate activation are cut into
    horizontal tiles of width T; inside each tile only the non-zero values and
    their tile-local indices are kept, ELL style, with no row-global packing.

    Readings where the pages are silent:
    * a unit is active iff its pre-activation is strictly positive, so ReLU(0),
      -0 and NaN are not stored; the value stored is the ReLU output itself;
    * slots follow ascending column order inside the tile (the s-th stored unit
      is the one with s active units to its left in the tile);
    * the count is not clamped to C; a row whose count exceeds C in any tile is
      an overflow row ([tgviewer] "Обучение" and [tencent] section 3 describe
      rows that do not fit the sparse block falling back to a dense buffer).
    """
    Z = np.asarray(Z)
    M, F = Z.shape
    if F % T:
        raise ValueError("F must be a multiple of T")
    nT = F // T
    tiles = Z.reshape(M, nT, T)
    active = tiles > 0
    counts = active.sum(axis=2)
    # number of active units strictly left of each column inside its tile
    left = np.cumsum(active, axis=2, dtype=np.int32) - active
    keep = active & (left < C)
    r, t, c = np.nonzero(keep)
    s = left[r, t, c]
    idx = np.zeros((M, nT, C), dtype=np.uint8)
    vals = np.zeros((M, nT, C), dtype=Z.dtype)
    idx[r, t, s] = c
    vals[r, t, s] = tiles[r, t, c]
    return TwellPacking(counts.astype(np.uint16), idx, vals, overflow_rows(counts, C), T, C)


def overflow_rows(counts: np.ndarray, C: int) -> np.ndarray:
    """Rows that do not fit: some tile holds more than C active units.

    Reading of the row-level dense fallback ([tgviewer] "Обучение";
    [tencent] section 3) applied to inference: one tile over capacity sends the
    whole row to the dense path.
    """
    counts = np.asarray(counts)
    if counts.size == 0:
        return np.zeros(0, dtype=np.int64)
    return np.flatnonzero(counts.max(axis=1) > C).astype(np.int64)


def unpack_twell(p: TwellPacking, F: int) -> np.ndarray:
    """Dense [M, F] gate output rebuilt from the stored slots.

    Exact ReLU(Z) for rows outside p.ovf; for overflow rows only the first C
    active units of each tile are present.
    """
    M = p.counts.shape[0]
    G = np.zeros((M, F), dtype=p.vals.dtype)
    used = np.minimum(p.counts.astype(np.int64), p.C)
    r, t, s = np.nonzero(np.arange(p.C)[None, None, :] < used[:, :, None])
    G[r, t * p.T + p.idx[r, t, s].astype(np.int64)] = p.vals[r, t, s]
    return G


# ---------------------------------------------------------------- sparse evaluation
def _sum_over_terms(x, WuT, Wd, r, j, g, M, chunk=1 << 15):
    """y = sum over listed terms (r, j, g) of g * (x_r . WuT_j) * Wd_j, fp64."""
    U = decode_bf16(WuT)
    h = np.empty(len(r), dtype=np.float64)
    for s in range(0, len(r), chunk):
        X = decode_bf16(x[r[s:s + chunk]])
        h[s:s + chunk] = np.einsum("nk,nk->n", X, U[j[s:s + chunk]])
    h *= np.asarray(g, dtype=np.float64)
    H = sps.csr_matrix((h, (r, j)), shape=(M, U.shape[0]))
    return np.asarray(H @ decode_bf16(Wd))


def ffn_from_twell(p: TwellPacking, x, Wg, WuT, Wd) -> np.ndarray:
    """The sparse forward read from a TwELL packing, fp64.

    [tgviewer] "Инференс"; [aimodeling] paragraph 3; [tencent] section 2: the
    fused kernel walks the stored non-zeros, fetches only the rows of Wu and Wd
    those units need, forms each unit's up-projection dot product and adds its
    contribution to the output; the hidden matrix is never formed. Overflow rows
    take the dense definition (reading of the dense fallback).
    """
    M = p.counts.shape[0]
    sparse_rows = np.ones(M, dtype=bool)
    sparse_rows[p.ovf] = False
    used = np.minimum(p.counts.astype(np.int64), p.C)
    r, t, s = np.nonzero((np.arange(p.C)[None, None, :] < used[:, :, None]) & sparse_rows[:, None, None])
    j = t * p.T + p.idx[r, t, s].astype(np.int64)
    y = _sum_over_terms(x, WuT, Wd, r, j, p.vals[r, t, s], M)
    if len(p.ovf):
        y[p.ovf] = dense_gated_ffn(x, Wg, WuT, Wd, rows=p.ovf)
    return y


def ffn_from_active_set(x, WuT, Wd, Z: np.ndarray) -> np.ndarray:
    """The gated FFN evaluated only on its non-zero terms, fp64.

    Same sum as dense_gated_ffn with the terms whose gate is exactly zero left
    out; since those terms are exact zeros this is the definition itself
    ([tgviewer] "Инференс": skipping zeros loses nothing). Z is the fp64
    pre-activation; every unit with Z > 0 contributes, with no capacity limit.
    """
    r, j = np.nonzero(Z > 0)
    return _sum_over_terms(x, WuT, Wd, r, j, Z[r, j], Z.shape[0])


# --------------------------------------------------------- gate-only variant
# A variant of the inference path that is not on the pages: the gate and up
# products are formed densely together, the packing stores the hidden value
# h = ReLU(z) * u instead of g, and the down product gathers only the Wd rows
# of stored units. The active set stays the gate's ([tencent] section 1: the
# gate decides which units are live), so a unit with z > 0 is stored even when
# its h is zero or negative. Rows that overflow a tile take the dense path, as
# in the main forward ([tgviewer] "Обучение"; [tencent] section 3).
def up_projections(x: np.ndarray, WuT: np.ndarray, rows=None) -> np.ndarray:
    """U = x WuT^T in fp64, shape [M, F] (the up projection of every unit)."""
    X = decode_bf16(x if rows is None else x[rows])
    return X @ decode_bf16(WuT).T


def pack_twell_hidden(Z: np.ndarray, H: np.ndarray, T: int, C: int) -> TwellPacking:
    """TwELL packing of the hidden values H at the units the gate activates.

    Counts, slots, tile-local indices and the overflow set are those of
    pack_twell(Z, T, C) (active iff Z > 0, ascending column order, counts not
    clamped); the value kept in a slot is H at that unit instead of ReLU(Z).
    """
    Z, H = np.asarray(Z), np.asarray(H)
    if Z.shape != H.shape:
        raise ValueError("Z and H must have the same shape")
    p = pack_twell(Z, T, C)
    M = Z.shape[0]
    used = np.arange(C)[None, None, :] < np.minimum(p.counts.astype(np.int64), C)[:, :, None]
    r, t, s = np.nonzero(used)
    vals = np.zeros((M, p.n_tiles, C), dtype=H.dtype)
    vals[r, t, s] = H.reshape(M, p.n_tiles, T)[r, t, p.idx[r, t, s].astype(np.int64)]
    return TwellPacking(p.counts, p.idx, vals, p.ovf, T, C)


def ffn_from_hidden_packing(p: TwellPacking, x, Wg, WuT, Wd) -> np.ndarray:
    """y from a packing of hidden values, fp64: for a row that fits,
    y_r = sum over its stored units j of h_j * Wd[j]; overflow rows take the
    dense definition."""
    M = p.counts.shape[0]
    D = decode_bf16(Wd)
    fits = np.ones(M, dtype=bool)
    fits[p.ovf] = False
    used = np.minimum(p.counts.astype(np.int64), p.C)
    r, t, s = np.nonzero((np.arange(p.C)[None, None, :] < used[:, :, None]) & fits[:, None, None])
    j = t * p.T + p.idx[r, t, s].astype(np.int64)
    Hs = sps.csr_matrix((p.vals[r, t, s].astype(np.float64), (r, j)), shape=(M, D.shape[0]))
    y = np.asarray(Hs @ D)
    if len(p.ovf):
        y[p.ovf] = dense_gated_ffn(x, Wg, WuT, Wd, rows=p.ovf)
    return y


def column_rms(Z: np.ndarray) -> np.ndarray:
    """Root-mean-square of each column of Z over all rows (tokens)."""
    Z = np.asarray(Z, dtype=np.float64)
    return np.sqrt(np.mean(Z * Z, axis=0))


# ------------------------------------------------------------- dead gate units
# [pulsen], dead-neuron paragraph: at the recommended L1 coefficient more than
# 30% of the gate units end up never active; [tencent] section 6: too strong a
# regularisation leaves such dead neurons. The pages re-initialise them during
# training. At inference the plain consequence is taken: a unit that no token
# activates contributes exact zeros to every output row, so its rows can be
# dropped from Wg, WuT and Wd without changing y, and the gate product shrinks.


def column_activity(Z: np.ndarray) -> np.ndarray:
    """Units active for at least one token: any over rows of Z[r, j] > 0.

    Same strict activity test as the packing (+0, -0 and NaN are inactive).
    """
    return np.asarray(np.asarray(Z) > 0).any(axis=0)


def live_layout(active: np.ndarray, T: int) -> np.ndarray:
    """Source column of each column of the compacted layer.

    The active columns in ascending order, then -1 (a zero row, never active:
    its pre-activation is exactly 0) up to the next multiple of T, so the
    compacted width stays whole TwELL tiles; at least one tile.
    """
    live = np.flatnonzero(np.asarray(active, dtype=bool))
    width = max(T, -(-len(live) // T) * T)
    src = np.full(width, -1, dtype=np.int64)
    src[: len(live)] = live
    return src


def compact_rows(W: np.ndarray, src: np.ndarray) -> np.ndarray:
    """Rows W[src[i]] (bf16 bits), and a zero row where src[i] < 0."""
    W = np.asarray(W)
    out = np.zeros((len(src),) + W.shape[1:], dtype=W.dtype)
    for i, s in enumerate(np.asarray(src)):
        if s >= 0:
            out[i] = W[s]
    return out


# ------------------------------------------------- training: hybrid format, backward
# [tgviewer] part "Обучение" and [tencent] section 3: for training every row of
# the gate output is either compressed into one sparse block whose width is the
# same for all rows ("globally aligned"), or, when it holds too many active
# units, kept as a dense row in a reserve; with it the backward pass needs no
# product of two dense matrices. Readings: the sparse block holds the row's
# active units (z > 0, the packing's test) in ascending column order with their
# gate values g = ReLU(z), width K for every row; a row with more than K active
# units goes to the reserve whole, as its dense g row.


@dataclass
class HybridFormat:
    idx: np.ndarray  # [M, K] int64 global unit of slot s (-1 past the count or for reserve rows)
    vals: np.ndarray  # [M, K] float32 g of that unit (0 where idx is -1)
    count: np.ndarray  # [M] int64 active units of the row (any size; > K for reserve rows)
    res_rows: np.ndarray  # [R] int64 rows held densely, ascending
    res_vals: np.ndarray  # [R, F] float32 their dense g rows


def hybrid_pack(Z: np.ndarray, K: int) -> HybridFormat:
    """Rows of ReLU(Z) (fp32 bits kept) in the hybrid training format."""
    Z = np.asarray(Z, dtype=np.float32)
    M, F = Z.shape
    idx = np.full((M, K), -1, dtype=np.int64)
    vals = np.zeros((M, K), dtype=np.float32)
    count = np.zeros(M, dtype=np.int64)
    res = []
    for r in range(M):
        cols = [j for j in range(F) if Z[r, j] > 0]
        count[r] = len(cols)
        if len(cols) > K:
            res.append(r)
            continue
        for s, j in enumerate(cols):
            idx[r, s] = j
            vals[r, s] = Z[r, j]
    res_rows = np.array(res, dtype=np.int64)
    res_vals = np.where(Z[res_rows] > 0, Z[res_rows], np.float32(0)).astype(np.float32)
    return HybridFormat(idx, vals, count, res_rows, res_vals.reshape(len(res_rows), F))


def _ffn_forward_f64(X, Wg, WuT, Wd):
    Z = X @ Wg.T
    G = np.maximum(Z, 0.0)
    U = X @ WuT.T
    return Z, G, U, (G * U) @ Wd


def _ffn_backward_f64(X, Wg, WuT, Wd, dY):
    """Gradients of y = (ReLU(x Wg^T) ⊙ x WuT^T) Wd by the chain rule, fp64:
    dH = dY Wd^T, dZ = dH ⊙ U ⊙ [Z > 0], dU = dH ⊙ G,
    dX = dZ Wg + dU WuT, dWg = dZ^T X, dWuT = dU^T X, dWd = H^T dY
    (ReLU'(0) taken as 0, matching the strict activity test)."""
    Z, G, U, _ = _ffn_forward_f64(X, Wg, WuT, Wd)
    dH = dY @ Wd.T
    dZ = dH * U * (Z > 0)
    dU = dH * G
    return dZ @ Wg + dU @ WuT, dZ.T @ X, dU.T @ X, (G * U).T @ dY


def _f64(a):
    """bf16 bits (uint16) decoded exactly; floating arrays taken as they are."""
    a = np.asarray(a)
    return decode_bf16(a) if a.dtype == np.uint16 else a.astype(np.float64)


def ffn_backward(x, Wg, WuT, Wd, dy):
    """(dx, dWg, dWuT, dWd) of the gated FFN for upstream gradient dy, fp64,
    from bf16 bits (dy too) or from floating arrays. Dense definition; dWuT
    is the gradient of WuT (row j = unit j), matching the weights' [F, d]
    layout."""
    return _ffn_backward_f64(*(_f64(a) for a in (x, Wg, WuT, Wd, dy)))


def ffn_backward_from_hybrid(hy: HybridFormat, x, Wg, WuT, Wd, dy):
    """The same gradients evaluated only on the active units listed by the
    hybrid format (sparse rows) and the reserve rows' dense g rows, fp64.

    Every term left out has g = 0 and z <= 0, so its dZ, dU and H are exact
    zeros; this is the definition itself, summed over the non-zero terms.
    """
    X, Wg_, WuT_, Wd_, dY = (_f64(a) for a in (x, Wg, WuT, Wd, dy))
    M, d = X.shape
    F = Wg_.shape[0]
    dX = np.zeros((M, d))
    dWg = np.zeros((F, d))
    dWu = np.zeros((F, d))
    dWd = np.zeros((F, d))
    res = {int(r): i for i, r in enumerate(hy.res_rows)}
    for r in range(M):
        if r in res:
            g_row = hy.res_vals[res[r]].astype(np.float64)
            units = np.flatnonzero(g_row > 0)
            g = g_row[units]
        else:
            n = int(hy.count[r])
            units = hy.idx[r, :n]
            g = hy.vals[r, :n].astype(np.float64)
        if len(units) == 0:
            continue
        u = WuT_[units] @ X[r]
        dh = Wd_[units] @ dY[r]
        dz = dh * u
        du = dh * g
        dX[r] = dz @ Wg_[units] + du @ WuT_[units]
        dWg[units] += np.outer(dz, X[r])
        dWu[units] += np.outer(du, X[r])
        dWd[units] += np.outer(g * u, dY[r])
    return dX, dWg, dWu, dWd
