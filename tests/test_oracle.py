"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each pin is a function of an oracle namespace so that the same pins can be run
against deliberately broken copies of the oracle (planted on the CPU, below):
every planted mistake must make at least one pin fail.

What pins what:
* decode_bf16            IEEE-754 bit patterns with known values.
* dense_gated_ffn        a hand-worked example with closed-form output (inputs,
                         values and derivation in tests/golden/); exact
                         integer brute force (Python ints, no floating point);
                         the identity ReLU(z) - ReLU(-z) = z, which turns the
                         difference of two FFN outputs into a bilinear form
                         evaluated by one einsum; the all-active and all-dead
                         degenerate densities.
* pack_twell             the hand-worked example; scipy's CSR of ReLU(Z), which
                         lists each row's non-zeros in ascending column order
                         and is sliced per tile in plain loops; T = F reduces
                         TwELL to row-wise ELL, i.e. CSR rows; strictness of
                         the activity test on +0, -0, NaN, subnormals.
* overflow_rows          boundary count == C (fits) versus C + 1 (overflows).
* ffn_from_twell /
  ffn_from_active_set    equal to the dense definition (skipped terms are exact
                         zeros), including rows that overflow.
* column_rms             a closed-form 2x2 case.
* ffn_backward           a hand-worked example with closed-form gradients;
                         central finite differences of <y, dy> along random
                         directions, for x and all three weights (fp64 inputs,
                         no pre-activation near the ReLU kink).
* hybrid_pack            a hand-worked example (ascending order, width K,
                         reserve rows kept whole as dense g rows).
* ffn_backward_from_hybrid  equal to the dense definition, reserve rows
                         included.
* up_projections /
  pack_twell_hidden /
  ffn_from_hidden_packing   (gate-only variant) a hand-worked example with a
                         negative and a zero h at active units and an overflow
                         row (tests/golden/); exact integer brute force; with
                         H = ReLU(Z) the hidden packing is the gate packing bit
                         for bit; the sum over stored h_j Wd[j] equals the
                         dense definition, overflow rows included.
* column_activity,
  live_layout,
  compact_rows           hand-worked cases (strict activity, ascending order,
                         padding to whole tiles, zero padding rows); and on
                         random layers with planted dead units, the dense
                         definition on the compacted weights equals it on the
                         full weights (dropped terms are exact zeros).
"""

import json
import os
import types

import numpy as np
import pytest
import scipy.sparse as sps

import oracle as O
from synth import WORKLOADS, make_inputs


# ------------------------------------------------------------------ helpers
def bf(values) -> np.ndarray:
    """Exact bf16 bits of values that bf16 represents exactly (checked)."""
    a = np.asarray(values, dtype=np.float32)
    u = a.view(np.uint32)
    assert np.all((u & np.uint32(0xFFFF)) == 0), "value is not exactly representable in bf16"
    return (u >> np.uint32(16)).astype(np.uint16)


def rand_bf16(rng, shape, scale=1.0):
    """Random bf16 bits by truncating fp32 (independent of the generator module)."""
    a = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def neg_bits(b):
    return (b ^ np.uint16(0x8000)).astype(np.uint16)


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# The hand-worked examples (inputs, expected values, derivation and the
# passages they follow) are stored under tests/golden/.
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


HAND = golden("forward_hand_example.json")
HAND_BWD = golden("backward_hand_example.json")
HAND_GU = golden("gateup_hand_example.json")


# --------------------------------------------------------------------- pins
def pin_decode(o):
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F7F, 0x8000, 0x0000], dtype=np.uint16)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127, -0.0, 0.0]
    got = o.decode_bf16(bits)
    assert got.dtype == np.float64
    assert list(got) == want
    assert np.signbit(got[5]) and not np.signbit(got[6])


def pin_hand_example(o):
    h = {k: bf(v) for k, v in HAND.items() if k in ("x", "Wg", "WuT", "Wd")}
    Z = o.gate_preactivations(h["x"], h["Wg"])
    assert np.array_equal(Z, np.array(HAND["z"], dtype=np.float64))
    y = o.dense_gated_ffn(h["x"], h["Wg"], h["WuT"], h["Wd"])
    assert np.array_equal(y, np.array(HAND["y"], dtype=np.float64))
    p = o.pack_twell(Z.astype(np.float32), T=HAND["T"], C=HAND["C"])
    assert p.counts.tolist() == HAND["counts"]
    for r in range(2):
        for t in range(2):
            if HAND["idx0"][r][t] is not None:
                assert int(p.idx[r, t, 0]) == HAND["idx0"][r][t]
                assert float(p.vals[r, t, 0]) == HAND["val0"][r][t]
    assert sorted(int(r) for r in p.ovf) == HAND["overflow_rows"]
    G = o.unpack_twell(p, 4)
    assert np.array_equal(G, np.maximum(np.array(HAND["z"], dtype=np.float32), 0))
    assert np.array_equal(o.ffn_from_twell(p, h["x"], h["Wg"], h["WuT"], h["Wd"]), y)
    assert np.array_equal(o.ffn_from_active_set(h["x"], h["WuT"], h["Wd"], Z), y)


def pin_integer_bruteforce(o):
    rng = np.random.default_rng(7)
    M, d, F = 3, 5, 6
    xi = rng.integers(-3, 4, (M, d))
    gi = rng.integers(-3, 4, (F, d))
    ui = rng.integers(-3, 4, (F, d))
    di = rng.integers(-3, 4, (F, d))
    want = np.zeros((M, d), dtype=np.int64)
    for r in range(M):
        for j in range(F):
            z = sum(int(xi[r, k]) * int(gi[j, k]) for k in range(d))
            u = sum(int(xi[r, k]) * int(ui[j, k]) for k in range(d))
            g = z if z > 0 else 0
            for e in range(d):
                want[r, e] += g * u * int(di[j, e])
    args = [bf(a) for a in (xi, gi, ui, di)]
    got = o.dense_gated_ffn(*args)
    assert np.array_equal(got, want.astype(np.float64))
    Z = o.gate_preactivations(args[0], args[1])
    assert np.array_equal(o.ffn_from_active_set(args[0], args[2], args[3], Z), want.astype(np.float64))


def pin_relu_identity(o):
    # ReLU(z) - ReLU(-z) = z and ReLU(z) + ReLU(-z) = |z|: flipping the sign of
    # the gate weights turns the FFN difference/sum into plain einsum forms.
    rng = np.random.default_rng(11)
    M, d, F = 7, 16, 24
    x, Wg, WuT, Wd = (rand_bf16(rng, s) for s in ((M, d), (F, d), (F, d), (F, d)))
    X, G, U, D = (o_ref_decode(a) for a in (x, Wg, WuT, Wd))
    bilinear = np.einsum("rk,jk,rl,jl,je->re", X, G, X, U, D, optimize=True)
    Zabs = np.abs(np.einsum("rk,jk->rj", X, G))
    absform = np.einsum("rj,rl,jl,je->re", Zabs, X, U, D, optimize=True)
    y_pos = o.dense_gated_ffn(x, Wg, WuT, Wd)
    y_neg = o.dense_gated_ffn(x, neg_bits(Wg), WuT, Wd)
    assert rel(y_pos - y_neg, bilinear) < 1e-12
    assert rel(y_pos + y_neg, absform) < 1e-12


def o_ref_decode(b):
    """Independent bf16 decode for the pins (bit arithmetic through frexp-free ldexp)."""
    b = np.asarray(b, dtype=np.int64)
    sign = np.where(b & 0x8000, -1.0, 1.0)
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    normal = sign * np.ldexp(1.0 + m / 128.0, e - 127)
    sub = sign * np.ldexp(m / 128.0, -126)
    return np.where(e == 0, sub, normal)


def pin_all_active(o):
    # a large positive bias column makes every gate active: ReLU is the identity
    rng = np.random.default_rng(12)
    M, d, F = 6, 8, 16
    x = rand_bf16(rng, (M, d))
    x[:, 0] = bf(1.0)
    Wg = rand_bf16(rng, (F, d), 0.05)
    Wg[:, 0] = bf(64.0)
    WuT, Wd = rand_bf16(rng, (F, d)), rand_bf16(rng, (F, d))
    X, G, U, D = (o_ref_decode(a) for a in (x, Wg, WuT, Wd))
    want = np.einsum("rk,jk,rl,jl,je->re", X, G, X, U, D, optimize=True)
    assert rel(o.dense_gated_ffn(x, Wg, WuT, Wd), want) < 1e-12
    Z = o.gate_preactivations(x, Wg)
    p = o.pack_twell(Z.astype(np.float32), T=8, C=4)
    assert (p.counts == 8).all() and list(p.ovf) == list(range(M))
    assert rel(o.ffn_from_twell(p, x, Wg, WuT, Wd), want) < 1e-12


def pin_zero_density(o):
    rng = np.random.default_rng(13)
    M, d, F = 5, 8, 16
    x = rand_bf16(rng, (M, d))
    x[:, 0] = bf(1.0)
    Wg = rand_bf16(rng, (F, d), 0.05)
    Wg[:, 0] = bf(-64.0)
    WuT, Wd = rand_bf16(rng, (F, d)), rand_bf16(rng, (F, d))
    y = o.dense_gated_ffn(x, Wg, WuT, Wd)
    assert np.all(y == 0)
    p = o.pack_twell(o.gate_preactivations(x, Wg).astype(np.float32), T=4, C=2)
    assert (p.counts == 0).all() and len(p.ovf) == 0
    assert np.all(o.ffn_from_twell(p, x, Wg, WuT, Wd) == 0)


def pin_one_active_unit(o):
    # One active gate unit per row: x_r = e_0 + e_{1+j(r)} and Wg_j = -0.5 e_0 +
    # e_{1+j} give z[r, j] = 0.5 for j = j(r) and -0.5 elsewhere, so
    # y_r = 0.5 (x_r . WuT_j(r)) Wd_j(r) in closed form, and the packing holds
    # exactly that unit.
    rng = np.random.default_rng(17)
    M, F, T, C = 6, 16, 8, 2
    d = F + 8
    jr = rng.permutation(F)[:M]
    xf = np.zeros((M, d))
    xf[:, 0] = 1.0
    xf[np.arange(M), 1 + jr] = 1.0
    gf = np.zeros((F, d))
    gf[:, 0] = -0.5
    gf[np.arange(F), 1 + np.arange(F)] = 1.0
    x, Wg = bf(xf), bf(gf)
    WuT, Wd = rand_bf16(rng, (F, d)), rand_bf16(rng, (F, d))
    U, D = o_ref_decode(WuT), o_ref_decode(Wd)
    want = np.stack([0.5 * (xf[r] @ U[jr[r]]) * D[jr[r]] for r in range(M)])
    assert rel(o.dense_gated_ffn(x, Wg, WuT, Wd), want) < 1e-12
    Z = o.gate_preactivations(x, Wg)
    p = o.pack_twell(Z.astype(np.float32), T=T, C=C)
    for r in range(M):
        t = int(jr[r]) // T
        assert p.counts[r].tolist() == [1 if k == t else 0 for k in range(F // T)]
        assert int(p.idx[r, t, 0]) == int(jr[r]) % T and float(p.vals[r, t, 0]) == 0.5
    assert len(p.ovf) == 0
    assert rel(o.ffn_from_twell(p, x, Wg, WuT, Wd), want) < 1e-12


def _csr_reference(Z, T, C):
    """Per-tile slices of each CSR row of ReLU(Z) (scipy keeps sorted columns)."""
    A = sps.csr_matrix(np.maximum(Z, 0))
    A.sort_indices()
    M, F = Z.shape
    nT = F // T
    counts = np.zeros((M, nT), dtype=np.int64)
    slots = {}
    for r in range(M):
        cols = A.indices[A.indptr[r]:A.indptr[r + 1]]
        data = A.data[A.indptr[r]:A.indptr[r + 1]]
        for t in range(nT):
            sel = (cols // T) == t
            counts[r, t] = sel.sum()
            slots[(r, t)] = (list(cols[sel][:C] - t * T), list(data[sel][:C]))
    return counts, slots


def pin_pack_csr(o):
    rng = np.random.default_rng(14)
    Z = rng.standard_normal((11, 48)).astype(np.float32)
    Z[rng.random(Z.shape) < 0.55] = 0.0
    Z[rng.random(Z.shape) < 0.05] = -0.0
    Z[0, :] = np.abs(Z[0, :]) + 1  # one fully active row
    for T in (4, 8, 16, 48):
        for C in (1, 2, 3, 5):
            p = o.pack_twell(Z, T, C)
            counts, slots = _csr_reference(Z, T, C)
            assert np.array_equal(p.counts.astype(np.int64), counts)
            for (r, t), (ci, dv) in slots.items():
                n = len(ci)
                assert p.idx[r, t, :n].tolist() == ci
                assert p.vals[r, t, :n].tolist() == dv
            want_ovf = [r for r in range(Z.shape[0]) if counts[r].max() > C]
            assert p.ovf.tolist() == want_ovf


def pin_pack_rowwise_ell(o):
    # T = F and C = F: one tile per row, never overflowing -> CSR rows exactly
    rng = np.random.default_rng(15)
    Z = rng.standard_normal((9, 32)).astype(np.float32)
    A = sps.csr_matrix(np.maximum(Z, 0))
    A.sort_indices()
    p = o.pack_twell(Z, T=32, C=32)
    assert len(p.ovf) == 0
    for r in range(9):
        n = A.indptr[r + 1] - A.indptr[r]
        assert p.counts[r, 0] == n
        assert p.idx[r, 0, :n].tolist() == A.indices[A.indptr[r]:A.indptr[r + 1]].tolist()
        assert p.vals[r, 0, :n].tolist() == A.data[A.indptr[r]:A.indptr[r + 1]].tolist()


def pin_pack_strict(o):
    tiny = np.float32(1e-45)  # smallest positive subnormal
    Z = np.array([[0.0, -0.0, np.nan, tiny, -tiny, 1.0, np.inf, -np.inf]], dtype=np.float32)
    p = o.pack_twell(Z, T=8, C=8)
    assert p.counts.tolist() == [[3]]
    assert p.idx[0, 0, :3].tolist() == [3, 5, 6]
    assert p.vals[0, 0, :3].view(np.uint32).tolist() == Z[0, [3, 5, 6]].view(np.uint32).tolist()


def pin_overflow_boundary(o):
    Z = np.zeros((3, 8), dtype=np.float32)
    Z[0, :2] = 1.0  # tile 0 holds exactly C = 2
    Z[1, :3] = 1.0  # tile 0 holds C + 1
    Z[2, 4:7] = 1.0  # tile 1 holds C + 1
    p = o.pack_twell(Z, T=4, C=2)
    assert p.counts.tolist() == [[2, 0], [3, 0], [0, 3]]
    assert p.ovf.tolist() == [1, 2]
    assert o.overflow_rows(np.array([[2, 2]]), 2).tolist() == []
    assert o.overflow_rows(np.array([[0, 3]]), 2).tolist() == [0]
    # overflow rows still hold the first C active units of each tile
    assert p.idx[1, 0].tolist() == [0, 1] and p.idx[2, 1].tolist() == [0, 1]


def pin_sparse_equals_dense(o):
    inp = make_inputs(WORKLOADS["tiny"])
    w = inp.workload
    args = (inp.x, inp.Wg, inp.WuT, inp.Wd)
    Y = o.dense_gated_ffn(*args)
    Z = o.gate_preactivations(inp.x, inp.Wg)
    assert rel(o.ffn_from_active_set(inp.x, inp.WuT, inp.Wd, Z), Y) < 1e-12
    seen_ovf = False
    for C in (1, w.C, w.T):
        p = o.pack_twell(Z, w.T, C)
        seen_ovf |= len(p.ovf) > 0
        assert rel(o.ffn_from_twell(p, *args), Y) < 1e-12
    assert seen_ovf


def pin_unpack_roundtrip(o):
    rng = np.random.default_rng(16)
    Z = rng.standard_normal((13, 64)).astype(np.float32) - 1.0
    p = o.pack_twell(Z, T=16, C=3)
    G = o.unpack_twell(p, 64)
    fit = np.setdiff1d(np.arange(13), p.ovf)
    assert np.array_equal(G[fit].view(np.uint32), np.maximum(Z[fit], 0).view(np.uint32))
    # per-row counts add up to the row's non-zeros (all rows, overflow included)
    assert np.array_equal(p.counts.sum(axis=1), (Z > 0).sum(axis=1))


def pin_column_rms(o):
    got = o.column_rms(np.array([[3.0, 4.0], [0.0, 0.0]]))
    assert np.allclose(got, [np.sqrt(4.5), np.sqrt(8.0)], rtol=0, atol=1e-15)


def pin_column_activity(o):
    Z = np.array([[0.0, -1.0, 2.0, -0.0, np.nan, 1e-40],
                  [0.0, -3.0, -2.0, -5.0, -np.inf, -1e-40],
                  [-1.0, -2.0, 0.0, 0.0, np.nan, 0.0]])
    assert o.column_activity(Z).tolist() == [False, False, True, False, False, True]
    assert o.column_activity(np.zeros((0, 3))).tolist() == [False, False, False]


def pin_live_layout(o):
    act = np.array([False, True, False, True, True, False, False, False, True])
    assert o.live_layout(act, 4).tolist() == [1, 3, 4, 8]
    assert o.live_layout(act, 3).tolist() == [1, 3, 4, 8, -1, -1]
    assert o.live_layout(np.zeros(8, dtype=bool), 4).tolist() == [-1, -1, -1, -1]
    assert o.live_layout(np.ones(8, dtype=bool), 4).tolist() == list(range(8))


def pin_compact_rows(o):
    W = np.arange(12, dtype=np.uint16).reshape(4, 3)
    got = o.compact_rows(W, np.array([2, 0, -1]))
    assert got.dtype == np.uint16
    assert got.tolist() == [[6, 7, 8], [0, 1, 2], [0, 0, 0]]


def pin_compaction_keeps_ffn(o):
    rng = np.random.default_rng(7)
    M, d, F, T = 9, 8, 24, 4
    x = rand_bf16(rng, (M, d))
    x[:, 0] = bf([1.0])[0]
    Wg, WuT, Wd = (rand_bf16(rng, (F, d), 0.5) for _ in range(3))
    dead = rng.permutation(F)[:10]
    Wg[dead, 0] = bf([-64.0])[0]  # z = -64 + (bounded rest) < 0 for every token
    Z = o.gate_preactivations(x, Wg)
    act = o.column_activity(Z)
    assert not act[dead].any() and act.sum() >= 4
    src = o.live_layout(act, T)
    Wg_c, WuT_c, Wd_c = (o.compact_rows(W, src) for W in (Wg, WuT, Wd))
    y = o.dense_gated_ffn(x, Wg, WuT, Wd)
    y_c = o.dense_gated_ffn(x, Wg_c, WuT_c, Wd_c)
    assert np.abs(y_c - y).max() <= 1e-12 * max(np.abs(y).max(), 1e-300)
    # dropping one live unit does change y: the equality above is not vacuous
    src_short = src[src >= 0][1:]
    y_s = o.dense_gated_ffn(x, *(o.compact_rows(W, src_short) for W in (Wg, WuT, Wd)))
    assert np.abs(y_s - y).max() > 1e-6 * np.abs(y).max()


def pin_backward_hand_example(o):
    h = {k: bf(HAND_BWD[k]) for k in ("x", "Wg", "WuT", "Wd", "dy")}
    dx, dWg, dWu, dWd = o.ffn_backward(h["x"], h["Wg"], h["WuT"], h["Wd"], h["dy"])
    assert dx.tolist() == HAND_BWD["dx"]
    assert dWg.tolist() == HAND_BWD["dWg"]
    assert dWu.tolist() == HAND_BWD["dWu"]
    assert dWd.tolist() == HAND_BWD["dWd"]


def pin_backward_finite_difference(o):
    rng = np.random.default_rng(11)
    M, d, F = 5, 6, 7
    P = [rng.standard_normal(s) for s in ((M, d), (F, d), (F, d), (F, d))]
    Z = P[0] @ P[1].T
    P[1][np.abs(Z).min(axis=0) < 0.05] *= -1.0  # keep clear of the kink (re-checked below)
    assert np.abs(P[0] @ P[1].T).min() > 1e-3
    R = rng.standard_normal((M, d))

    def loss(X, Wg, WuT, Wd):  # <y, R> with y written out from its definition
        return float(np.sum(((np.maximum(X @ Wg.T, 0) * (X @ WuT.T)) @ Wd) * R))

    grads = o.ffn_backward(*P, R)
    eps = 1e-6
    for i in range(4):
        V = rng.standard_normal(P[i].shape)
        hi = [p + eps * V if k == i else p for k, p in enumerate(P)]
        lo = [p - eps * V if k == i else p for k, p in enumerate(P)]
        fd = (loss(*hi) - loss(*lo)) / (2 * eps)
        an = float(np.sum(grads[i] * V))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (i, fd, an)


def pin_hybrid_pack(o):
    Z = np.array([[0.5, -1.0, 2.0, 0.0, 3.0],
                  [-1.0, -2.0, -3.0, -4.0, -5.0],
                  [1.0, 2.0, 3.0, -1.0, 4.0],
                  [0.0, 0.0, 7.0, 0.0, 0.0]], dtype=np.float32)
    h = o.hybrid_pack(Z, 3)
    assert h.count.tolist() == [3, 0, 4, 1]
    assert h.idx.tolist() == [[0, 2, 4], [-1, -1, -1], [-1, -1, -1], [2, -1, -1]]
    assert h.vals.tolist() == [[0.5, 2.0, 3.0], [0, 0, 0], [0, 0, 0], [7.0, 0, 0]]
    assert h.res_rows.tolist() == [2]
    assert h.res_vals.tolist() == [[1.0, 2.0, 3.0, 0.0, 4.0]]


def pin_backward_hybrid_equals_dense(o):
    rng = np.random.default_rng(12)
    M, d, F, K = 7, 16, 24, 12
    x = rand_bf16(rng, (M, d))
    Wg, WuT, Wd = (rand_bf16(rng, (F, d), 0.5) for _ in range(3))
    dy = rand_bf16(rng, (M, d))
    Z = o.gate_preactivations(x, Wg)
    h = o.hybrid_pack(Z.astype(np.float32), K)
    assert len(h.res_rows) >= 1 and (h.count <= K).sum() >= 1  # both kinds of rows occur
    want = o.ffn_backward(x, Wg, WuT, Wd, dy)
    got = o.ffn_backward_from_hybrid(h, x, Wg, WuT, Wd, dy)
    for a, b in zip(got, want):  # g went through fp32 in the format
        assert np.abs(a - b).max() <= 1e-6 * max(np.abs(b).max(), 1e-300)


def pin_gateup_hand_example(o):
    """The gate-only variant's hand-worked example: h < 0 and h = 0 at active
    units are stored, the overflow row takes the dense path."""
    h = {k: bf(v) for k, v in HAND_GU.items() if k in ("x", "Wg", "WuT", "Wd")}
    Z = o.gate_preactivations(h["x"], h["Wg"])
    U = o.up_projections(h["x"], h["WuT"])
    assert np.array_equal(Z, np.array(HAND_GU["z"], dtype=np.float64))
    assert np.array_equal(U, np.array(HAND_GU["u"], dtype=np.float64))
    H = np.array(HAND_GU["h"], dtype=np.float32)
    p = o.pack_twell_hidden(Z.astype(np.float32), H, HAND_GU["T"], HAND_GU["C"])
    assert p.counts.tolist() == HAND_GU["counts"]
    for r in range(2):
        for t in range(2):
            if HAND_GU["idx0"][r][t] is not None:
                assert int(p.idx[r, t, 0]) == HAND_GU["idx0"][r][t]
                assert float(p.vals[r, t, 0]) == HAND_GU["val0"][r][t]
    assert sorted(int(r) for r in p.ovf) == HAND_GU["overflow_rows"]
    y = o.ffn_from_hidden_packing(p, h["x"], h["Wg"], h["WuT"], h["Wd"])
    assert np.array_equal(y, np.array(HAND_GU["y"], dtype=np.float64))


def pin_up_integer_bruteforce(o):
    """x WuT^T on small integers, against Python-int triple loops."""
    rng = np.random.default_rng(21)
    M, d, F = 3, 5, 4
    xi = rng.integers(-8, 9, size=(M, d))
    wi = rng.integers(-8, 9, size=(F, d))
    want = [[sum(int(xi[r, k]) * int(wi[j, k]) for k in range(d)) for j in range(F)] for r in range(M)]
    got = o.up_projections(bf(xi), bf(wi))
    assert got.tolist() == want
    assert o.up_projections(bf(xi), bf(wi), rows=np.array([2, 0])).tolist() == [want[2], want[0]]


def pin_hidden_pack_reduces_to_gate_pack(o):
    """With H = ReLU(Z) the hidden packing is the gate packing, bit for bit."""
    rng = np.random.default_rng(22)
    Z = rng.standard_normal((11, 48)).astype(np.float32)
    Z[rng.random(Z.shape) < 0.2] = 0.0
    for T, C in ((8, 2), (16, 16), (48, 3)):
        a = o.pack_twell_hidden(Z, np.maximum(Z, 0), T, C)
        b = o.pack_twell(Z, T, C)
        assert np.array_equal(a.counts, b.counts) and np.array_equal(a.ovf, b.ovf)
        used = np.arange(C)[None, None, :] < np.minimum(b.counts, C)[:, :, None]
        assert np.array_equal(a.idx[used], b.idx[used])
        assert np.array_equal(a.vals[used].view(np.uint32), b.vals[used].view(np.uint32))


def pin_hidden_ffn_equals_dense(o):
    """Sum over stored h_j Wd[j] (dense for overflow rows) is the definition."""
    rng = np.random.default_rng(23)
    M, d, F, T, C = 9, 16, 24, 8, 4
    x = rand_bf16(rng, (M, d))
    Wg, WuT, Wd = (rand_bf16(rng, (F, d), 0.5) for _ in range(3))
    Z = o.gate_preactivations(x, Wg)
    H = np.maximum(Z, 0) * o.up_projections(x, WuT)
    p = o.pack_twell_hidden(Z, H, T, C)
    assert 0 < len(p.ovf) < M  # both kinds of rows occur
    y = o.ffn_from_hidden_packing(p, x, Wg, WuT, Wd)
    want = o.dense_gated_ffn(x, Wg, WuT, Wd)
    assert np.abs(y - want).max() <= 1e-12 * np.abs(want).max()


PINS = [
    pin_decode, pin_hand_example, pin_integer_bruteforce, pin_relu_identity, pin_all_active,
    pin_zero_density, pin_one_active_unit, pin_pack_csr, pin_pack_rowwise_ell, pin_pack_strict, pin_overflow_boundary,
    pin_sparse_equals_dense, pin_unpack_roundtrip, pin_column_rms,
    pin_column_activity, pin_live_layout, pin_compact_rows, pin_compaction_keeps_ffn,
    pin_backward_hand_example, pin_backward_finite_difference, pin_hybrid_pack,
    pin_backward_hybrid_equals_dense,
    pin_gateup_hand_example, pin_up_integer_bruteforce, pin_hidden_pack_reduces_to_gate_pack,
    pin_hidden_ffn_equals_dense,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(O)


# ------------------------------------------------------ invariants on workloads
@pytest.mark.parametrize("name", ["tiny"])
def test_invariants_tiny_workload(name):
    inp = make_inputs(WORKLOADS[name])
    w = inp.workload
    Z32 = O.gate_preactivations(inp.x, inp.Wg).astype(np.float32)
    p = O.pack_twell(Z32, w.T, w.C)
    nT = w.F // w.T
    act = Z32.reshape(w.M, nT, w.T) > 0
    assert np.array_equal(p.counts, act.sum(axis=2))  # I1
    assert np.array_equal(p.counts.sum(axis=1), (Z32 > 0).sum(axis=1))  # I2
    G = O.unpack_twell(p, w.F)
    fit = np.setdiff1d(np.arange(w.M), p.ovf)
    assert np.array_equal(G[fit], np.maximum(Z32[fit], 0))  # I3 (rows that fit)
    assert np.array_equal(p.ovf, np.flatnonzero(p.counts.max(axis=1) > w.C))  # I4
    used = np.minimum(p.counts, w.C)
    for r in range(w.M):  # I6
        for t in range(nT):
            n = used[r, t]
            assert np.all(np.diff(p.idx[r, t, :n].astype(int)) > 0)
            assert np.all(p.vals[r, t, :n] > 0)


# --------------------------------------------------- planted mistakes (CPU only)
def _mutant(**overrides):
    ns = {k: getattr(O, k) for k in O.__all__ if hasattr(O, k)} if hasattr(O, "__all__") else dict(vars(O))
    ns.update(overrides)
    return types.SimpleNamespace(**ns)


def _dense_variant(kind):
    def f(x, Wg, WuT, Wd, rows=None, chunk=512):
        r = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
        X = O.decode_bf16(x[r])
        G, U, D = O.decode_bf16(Wg), O.decode_bf16(WuT), O.decode_bf16(Wd)
        Z, Uo = X @ G.T, X @ U.T
        if kind == "no_relu":
            return (Z * Uo) @ D
        if kind == "swap_gate_up":
            return (np.maximum(Uo, 0) * Z) @ D
        if kind == "up_as_down":
            return (np.maximum(Z, 0) * Uo) @ U
        if kind == "leaky":
            return (np.where(Z > 0, Z, 0.01 * Z) * Uo) @ D
        raise AssertionError(kind)
    return f


def _pack_variant(kind):
    def f(Z, T, C):
        Z = np.asarray(Z)
        if kind == "ge":  # activity test >= 0 instead of > 0
            M, F = Z.shape
            tiles = Z.reshape(M, F // T, T)
            act = tiles >= 0
            left = np.cumsum(act, axis=2, dtype=np.int32) - act
            r, t, c = np.nonzero(act & (left < C))
            idx = np.zeros((M, F // T, C), np.uint8)
            vals = np.zeros((M, F // T, C), Z.dtype)
            idx[r, t, left[r, t, c]] = c
            vals[r, t, left[r, t, c]] = tiles[r, t, c]
            cnt = act.sum(axis=2)
            return O.TwellPacking(cnt.astype(np.uint16), idx, vals, O.overflow_rows(cnt, C), T, C)
        p = O.pack_twell(Z, T, C)
        if kind == "descending":  # slots filled from the right end of the tile
            q = O.pack_twell(Z.reshape(Z.shape[0], -1, T)[:, :, ::-1].reshape(Z.shape), T, C)
            q.idx = (T - 1 - q.idx.astype(int)).astype(np.uint8)
            return q
        if kind == "global_idx":
            p.idx = ((p.idx.astype(int) + np.arange(p.n_tiles)[None, :, None] * T) % 256).astype(np.uint8)
            return p
        if kind == "clamped":
            p.counts = np.minimum(p.counts, C).astype(np.uint16)
            return p
        if kind == "ovf_ge":
            p.ovf = np.flatnonzero(p.counts.max(axis=1) >= C)
            return p
        raise AssertionError(kind)
    return f


def _twell_no_gate(p, x, Wg, WuT, Wd):
    q = O.TwellPacking(p.counts, p.idx, np.ones_like(p.vals), p.ovf, p.T, p.C)
    return O.ffn_from_twell(q, x, Wg, WuT, Wd)


def _twell_ignore_ovf(p, x, Wg, WuT, Wd):
    q = O.TwellPacking(p.counts, p.idx, p.vals, np.zeros(0, dtype=np.int64), p.T, p.C)
    return O.ffn_from_twell(q, x, Wg, WuT, Wd)


def _unpack_no_tile_offset(p, F):
    M = p.counts.shape[0]
    G = np.zeros((M, F), dtype=p.vals.dtype)
    used = np.minimum(p.counts.astype(np.int64), p.C)
    r, t, s = np.nonzero(np.arange(p.C)[None, None, :] < used[:, :, None])
    G[r, p.idx[r, t, s].astype(np.int64)] = p.vals[r, t, s]
    return G


MUTANTS = {
    "decode_shift15": dict(decode_bf16=lambda b: (np.asarray(b).astype(np.uint32) << 15).view(np.float32).astype(np.float64)),
    "gate_uses_up": dict(gate_preactivations=lambda x, Wg, rows=None: O.gate_preactivations(x, Wg, rows) * 0 + O.decode_bf16(x) @ O.decode_bf16(Wg)[::-1].T),
    "dense_no_relu": dict(dense_gated_ffn=_dense_variant("no_relu")),
    "dense_swap_gate_up": dict(dense_gated_ffn=_dense_variant("swap_gate_up")),
    "dense_up_as_down": dict(dense_gated_ffn=_dense_variant("up_as_down")),
    "dense_leaky": dict(dense_gated_ffn=_dense_variant("leaky")),
    "pack_ge": dict(pack_twell=_pack_variant("ge")),
    "pack_descending": dict(pack_twell=_pack_variant("descending")),
    "pack_global_idx": dict(pack_twell=_pack_variant("global_idx")),
    "pack_clamped_counts": dict(pack_twell=_pack_variant("clamped")),
    "pack_ovf_ge": dict(pack_twell=_pack_variant("ovf_ge")),
    "overflow_ge": dict(overflow_rows=lambda c, C: np.flatnonzero(np.asarray(c).max(axis=1) >= C)),
    "twell_drops_gate_value": dict(ffn_from_twell=_twell_no_gate),
    "twell_ignores_overflow": dict(ffn_from_twell=_twell_ignore_ovf),
    "unpack_no_tile_offset": dict(unpack_twell=_unpack_no_tile_offset),
    "active_set_negative": dict(ffn_from_active_set=lambda x, WuT, Wd, Z: O.ffn_from_active_set(x, WuT, Wd, -Z)),
    "rms_no_sqrt": dict(column_rms=lambda Z: np.mean(np.asarray(Z) ** 2, axis=0)),
    "activity_ge": dict(column_activity=lambda Z: (np.asarray(Z) >= 0).any(axis=0)),
    "activity_all_rows": dict(column_activity=lambda Z: (np.asarray(Z) > 0).all(axis=0)),
    "layout_no_padding": dict(live_layout=lambda a, T: np.flatnonzero(a)),
    "layout_descending": dict(live_layout=lambda a, T: O.live_layout(a, T)[::-1].copy()),
    "layout_pad_with_zero_col": dict(live_layout=lambda a, T: np.maximum(O.live_layout(a, T), 0)),
    "compact_off_by_one": dict(compact_rows=lambda W, src: O.compact_rows(W, np.where(src >= 0, (src + 1) % len(W), src))),
    "compact_pad_copies": dict(compact_rows=lambda W, src: np.asarray(W)[np.asarray(src)]),
    "bwd_no_relu_mask": dict(ffn_backward=lambda *a: _bwd_variant("no_mask", *a)),
    "bwd_du_uses_u": dict(ffn_backward=lambda *a: _bwd_variant("du_u", *a)),
    "bwd_dx_drops_du": dict(ffn_backward=lambda *a: _bwd_variant("dx_no_du", *a)),
    "bwd_dwd_uses_g": dict(ffn_backward=lambda *a: _bwd_variant("dwd_g", *a)),
    "bwd_dwg_uses_du": dict(ffn_backward=lambda *a: _bwd_variant("dwg_du", *a)),
    "hybrid_ge_k": dict(hybrid_pack=lambda Z, K: _hybrid_variant("ge", Z, K)),
    "hybrid_descending": dict(hybrid_pack=lambda Z, K: _hybrid_variant("desc", Z, K)),
    "hybrid_reserve_z": dict(hybrid_pack=lambda Z, K: _hybrid_variant("res_z", Z, K)),
    "hidden_activity_from_h": dict(pack_twell_hidden=lambda Z, H, T, C: O.pack_twell_hidden(H, H, T, C)),
    "hidden_stores_g": dict(pack_twell_hidden=lambda Z, H, T, C: O.pack_twell_hidden(Z, np.maximum(Z, 0), T, C)),
    "hidden_down_ignores_overflow": dict(ffn_from_hidden_packing=lambda p, *a: O.ffn_from_hidden_packing(
        O.TwellPacking(p.counts, p.idx, p.vals, np.zeros(0, dtype=np.int64), p.T, p.C), *a)),
    "hidden_down_uses_up": dict(ffn_from_hidden_packing=lambda p, x, Wg, WuT, Wd: O.ffn_from_hidden_packing(
        p, x, Wg, WuT, WuT)),
    "up_not_transposed": dict(up_projections=lambda x, WuT, rows=None: O.decode_bf16(
        x if rows is None else x[rows]) @ O.decode_bf16(WuT)),
    "hybrid_bwd_drops_reserve": dict(ffn_backward_from_hybrid=lambda h, *a: O.ffn_backward_from_hybrid(
        O.HybridFormat(h.idx, h.vals, h.count, h.res_rows[:0], h.res_vals[:0]), *a)),
}


def _bwd_variant(kind, x, Wg, WuT, Wd, dy):
    X, G_, U_, D_, dY = (O._f64(a) for a in (x, Wg, WuT, Wd, dy))
    Z = X @ G_.T
    G = np.maximum(Z, 0)
    U = X @ U_.T
    dH = dY @ D_.T
    dZ = dH * U * (1.0 if kind == "no_mask" else (Z > 0))
    dU = dH * (U if kind == "du_u" else G)
    dX = dZ @ G_ + (0 if kind == "dx_no_du" else dU @ U_)
    dWg = (dU if kind == "dwg_du" else dZ).T @ X
    dWd = (G if kind == "dwd_g" else G * U).T @ dY
    return dX, dWg, dU.T @ X, dWd


def _hybrid_variant(kind, Z, K):
    h = O.hybrid_pack(Z, K - 1 if kind == "ge" else K)
    if kind == "ge":
        return O.HybridFormat(np.pad(h.idx, ((0, 0), (0, 1)), constant_values=-1),
                              np.pad(h.vals, ((0, 0), (0, 1))), h.count, h.res_rows, h.res_vals)
    if kind == "desc":
        idx, vals = h.idx.copy(), h.vals.copy()
        for r in range(len(idx)):
            n = int(min(h.count[r], K)) if r not in set(h.res_rows.tolist()) else 0
            idx[r, :n], vals[r, :n] = idx[r, :n][::-1], vals[r, :n][::-1]
        return O.HybridFormat(idx, vals, h.count, h.res_rows, h.res_vals)
    Zr = np.asarray(Z, dtype=np.float32)[h.res_rows]
    return O.HybridFormat(h.idx, h.vals, h.count, h.res_rows, Zr)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    o = _mutant(**MUTANTS[name])
    failures = 0
    for pin in PINS:
        try:
            pin(o)
        except Exception:
            failures += 1
    assert failures > 0, f"no pin catches the planted mistake {name}"
