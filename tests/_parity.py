"""Comparison rules between the HIP path and the oracle (used by the GPU tests
and smoke()). Acceptance bar:

* packing fed the same pre-activations: bit-exact counts, tile-local indices,
  value bits of every used slot, and the same overflow-row set;
* active sets from the GPU's own fp32 gate versus the fp64 definition: a
  mismatch at (r, j) only where |Z_ref[r, j]| < 1e-3 * rms_j, rms_j being the
  root-mean-square of column j of Z_ref over all tokens;
* y: relative L2 error <= 1e-3 and max |error| <= 1e-2 * max |Y_ref|.
"""

from __future__ import annotations

import numpy as np

ACTIVE_TOL = 1e-3
Y_REL_L2 = 1e-3
Y_MAX_REL = 1e-2


def to_device(bits: np.ndarray, device):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def host_packing(p):
    """numpy copies of a device Packed: counts (uint16), idx, vals, sorted ovf."""
    n = int(p.n_ovf.cpu().item())
    ovf = np.sort(p.ovf_rows[:n].cpu().numpy().astype(np.int64)) if n else np.zeros(0, np.int64)
    return dict(
        counts=p.counts.cpu().numpy().view(np.uint16),
        idx=p.idx.cpu().numpy(),
        vals=p.vals.cpu().numpy(),
        ovf=ovf,
        n_ovf=n,
    )


def used_slots(counts, C):
    return np.arange(C)[None, None, :] < np.minimum(counts.astype(np.int64), C)[:, :, None]


def check_packing_bitexact(g: dict, o, rows=None):
    """GPU packing g (host_packing) equals oracle packing o (TwellPacking)."""
    sel = slice(None) if rows is None else rows
    gc, oc = g["counts"][sel], o.counts
    assert gc.shape == oc.shape, (gc.shape, oc.shape)
    bad = np.argwhere(gc != oc)
    assert bad.size == 0, f"{len(bad)} counts differ, first at {bad[:3].tolist()}: gpu {gc[tuple(bad[0])]} oracle {oc[tuple(bad[0])]}"
    used = used_slots(oc, o.C)
    gi, gv = g["idx"][sel], g["vals"][sel]
    assert np.array_equal(gi[used], o.idx[used]), "tile-local indices differ"
    assert np.array_equal(gv[used].view(np.uint32), o.vals[used].astype(np.float32).view(np.uint32)), "values differ"
    if rows is None:
        assert np.array_equal(g["ovf"], o.ovf), f"overflow sets differ: gpu {g['ovf'][:10]} oracle {o.ovf[:10]}"


def check_active_set(g: dict, Zref: np.ndarray, rms: np.ndarray, T: int, C: int, rows=None):
    """Active sets of the GPU packing against the fp64 pre-activations Zref
    (rows of Zref correspond to `rows` of the GPU packing). Returns stats."""
    sel = slice(None) if rows is None else rows
    counts = g["counts"][sel].astype(np.int64)
    idx, vals = g["idx"][sel], g["vals"][sel]
    Mr, nT = counts.shape
    tol = ACTIVE_TOL * rms
    tiles = Zref.reshape(Mr, nT, T)
    border = np.abs(tiles) < tol.reshape(nT, T)[None]
    ref_act = tiles > 0
    ref_cnt = ref_act.sum(axis=2)
    slack = border.sum(axis=2)
    assert np.all(np.abs(counts - ref_cnt) <= slack), "count differs beyond near-zero units"
    used = used_slots(counts, C)
    r, t, s = np.nonzero(used)
    loc = idx[r, t, s].astype(np.int64)
    ok = ref_act[r, t, loc] | border[r, t, loc]
    assert ok.all(), f"{(~ok).sum()} stored units are inactive in the definition and not near zero"
    zt = tiles[r, t, loc]
    err = np.abs(vals[r, t, s].astype(np.float64) - zt)
    colrms = rms.reshape(nT, T)[t, loc]
    assert np.all(err <= ACTIVE_TOL * colrms + 1e-30), f"stored gate values off by up to {err.max()}"
    # every clearly active unit of a tile that fits is stored
    fits = counts <= C
    missing = ref_act & ~border & fits[:, :, None]
    stored = np.zeros_like(ref_act)
    stored[r, t, loc] = True
    assert not (missing & ~stored).any(), "a clearly active unit is missing from a tile that fits"
    return dict(mismatch_budget=int(slack.sum()), max_val_err=float(err.max()) if err.size else 0.0)


def y_errors(y: np.ndarray, yref: np.ndarray):
    y = y.astype(np.float64)
    diff = y - yref
    nref = np.linalg.norm(yref)
    rel = np.linalg.norm(diff) / nref if nref > 0 else np.linalg.norm(diff)
    mref = np.abs(yref).max() if yref.size else 0.0
    mx = np.abs(diff).max() if diff.size else 0.0
    return float(rel), float(mx), float(mref)


def check_y(y: np.ndarray, yref: np.ndarray):
    assert np.isfinite(y).all(), "y has non-finite entries (a row was not written?)"
    rel, mx, mref = y_errors(y, yref)
    if mref == 0:
        assert mx == 0, f"expected y == 0 exactly, max |y| = {mx}"
        return rel, mx
    assert rel <= Y_REL_L2, f"relative L2 error {rel:.3e} > {Y_REL_L2}"
    assert mx <= Y_MAX_REL * mref, f"max abs error {mx:.3e} > {Y_MAX_REL} * {mref:.3e}"
    return rel, mx
