"""Parity of the HIP path (through the C ABI) with the CPU oracle, on MI355X.

Oracle-sized cases span several workgroup tiles and ragged tails; full-size
cases run the exact launch configuration bench.py times (twell_ffn_forward on
the full workload) and compare the whole layer: packing bits, active sets and
every row of y. All inputs come from the seeded generator.
"""

from __future__ import annotations

import functools

import numpy as np
import pytest

import oracle as O
from synth import WORKLOADS, make_inputs, make_upstream_grad, scaled

from _parity import (
    check_active_set,
    check_packing_bitexact,
    check_y,
    host_packing,
    to_device,
    used_slots,
    y_errors,
)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU only to be deselected by -m
    pytest.skip("needs a GPU", allow_module_level=True)

import activation_sparse_ffn_gate_amd as tw  # noqa: E402

DEV = torch.device("cuda", 0)

SMALL = {
    "tiny": WORKLOADS["tiny"],
    "uniform_ragged": scaled(WORKLOADS["ffn1p5b"], M=300, d=512, F=2048),
    "heavytail_small": scaled(WORKLOADS["ffn1p5b_heavytail"], M=1100, d=1024, F=4096),
    "zipf_small": scaled(WORKLOADS["ffn2b_zipf"], M=520, d=768, F=1280, T=64, C=8, mean_nnz=20.0),
    "t64_odd_tiles": scaled(WORKLOADS["tiny"], M=130, d=512, F=192, T=64, C=4),
    "dense11_small": scaled(WORKLOADS["sweep_p11pct"], M=257, d=512, F=1024),
    # ~900 stored units per row, 128 tiles of capacity T: never overflows, and
    # every row's list spans several LDS rounds and tile groups of both kernels
    "long_rows": scaled(WORKLOADS["sweep_p11pct"], M=96, d=512, F=8192, T=64, C=64),
    # d = 2304 is not one the sliced kernels take: the forward uses the fused one
    "fused_only_d2304": scaled(WORKLOADS["ffn1p5b"], M=200, d=2304, F=1024, mean_nnz=12.0),
    # Few rows: the gate's 32-token tiles and the fused kernel's workgroup per
    # token. d = 768 takes 8-byte lanes and leaves 5 of 8 waves without output
    # columns; d = 2560 gives two column groups per lane, the second held by 2
    # waves; 30% density at C = T = 64 never overflows and gives > 1024 list
    # entries per 64-tile group (several LDS rounds).
    "few_rows_d768": scaled(WORKLOADS["ffn1p5b"], M=5, d=768, F=2048),
    "few_rows_d2560": scaled(WORKLOADS["ffn2b_zipf"], M=7, d=2560, F=2560),
    "few_rows_dense30": scaled(WORKLOADS["sweep_p11pct"], M=9, d=512, F=8192, T=64, C=64, mean_nnz=2458.0),
    # ~490 units a row with C = 8: rows cut over several workgroups that also
    # hold spilled (overflowing) tiles
    "few_rows_cut_spill": scaled(WORKLOADS["sweep_p3pct"], M=24, d=512, F=16384, C=8),
    # the headline's d = 2048 through the small-batch forward and the training path
    "d2048_small": scaled(WORKLOADS["ffn1p5b"], M=200, d=2048, F=1024, mean_nnz=24.0),
    # The gate's K split (64 tiles of 32 x 128) with ~490 units a row at C = 8:
    # every row overflows (its tiles' z spilled) and is cut over several
    # workgroups
    "split_cut_overflow": scaled(WORKLOADS["sweep_p3pct"], M=24, d=512, F=8192, C=8, mean_nnz=490.0),
    # The fallback's ring kernels take a list of at least 1793 rows at
    # d = 8192: every one of 1800 rows overflows here; in the second case
    # 1459 do, so the ring launches find the list too short and return.
    "ring_fallback_all": scaled(WORKLOADS["sweep_p11pct"], M=1800, d=8192, F=512, C=4),
    "ring_fallback_short": scaled(WORKLOADS["sweep_p3pct"], M=1800, d=8192, F=512, C=4),
    # the same with F % 128 == 64: the last gated-up tile holds 64 units
    "ring_fallback_f576": scaled(WORKLOADS["sweep_p11pct"], M=1800, d=8192, F=576, T=64, C=4),
    # d = 4096: the ring path from 3841 rows, 16 down tiles across
    "ring_fallback_d4096": scaled(WORKLOADS["sweep_p11pct"], M=3900, d=4096, F=512, C=4),
}
FULL = ["ffn1p5b", "ffn1p5b_heavytail", "ffn2b_zipf"] + [
    k for k in WORKLOADS if k.startswith(("sweep_", "decode_"))
]


@functools.lru_cache(maxsize=2)
def small_case(name):
    inp = make_inputs(SMALL[name])
    Z = O.gate_preactivations(inp.x, inp.Wg)
    return inp, Z, O.column_rms(Z), O.dense_gated_ffn(inp.x, inp.Wg, inp.WuT, inp.Wd)


def dev(inp):
    return [to_device(a, DEV) for a in (inp.x, inp.Wg, inp.WuT, inp.Wd)]


def nan_y(M, d):
    return torch.full((M, d), float("nan"), dtype=torch.float32, device=DEV)


def run_gate(inp, debug=True):
    w = inp.workload
    x, Wg, _, _ = dev(inp)
    z = torch.empty((w.M, w.F), dtype=torch.float32, device=DEV) if debug else None
    p = tw.gate_pack(x, Wg, w.T, w.C, z_debug=z)
    torch.cuda.synchronize()
    return p, (z.cpu().numpy() if debug else None)


# ------------------------------------------------------------------ small cases
@pytest.mark.parametrize("name", list(SMALL))
def test_packing_bitexact(name):
    inp, Z, rms, _ = small_case(name)
    w = inp.workload
    p, z = run_gate(inp)
    # the fp32 gate agrees with the fp64 definition (checks the MFMA layout)
    assert np.abs(z - Z).max() <= 1e-4 * rms.max()
    ref = O.pack_twell(z, w.T, w.C)
    check_packing_bitexact(host_packing(p), ref)
    # the instance without z output (the forward's) computes the same z, so
    # its packing equals the same reference bit for bit
    p_fwd, _ = run_gate(inp, debug=False)
    check_packing_bitexact(host_packing(p_fwd), ref)


@pytest.mark.parametrize("name", list(SMALL))
def test_active_set_end_to_end(name):
    inp, Z, rms, _ = small_case(name)
    p, _ = run_gate(inp, debug=False)
    check_active_set(host_packing(p), Z, rms, inp.workload.T, inp.workload.C)


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_matches_definition(name):
    inp, _, _, Y = small_case(name)
    w = inp.workload
    y = tw.ffn_forward(*dev(inp), w.T, w.C, y=nan_y(w.M, w.d))
    rel, mx = check_y(y.cpu().numpy(), Y)
    print(f"{name}: rel L2 {rel:.2e}, max abs {mx:.2e}")


def sliced_ok(d):
    return tw.workspace_bytes(tw.OP_SLICED_UPDOWN, 1, d, 1024, 64, 8) > 0


@pytest.mark.parametrize("name", list(SMALL))
def test_components_compose(name):
    """gate_pack + (sliced or fused) up/down + dense_fallback == ffn_forward,
    bit for bit; the up/down kernels leave overflow rows alone; packed_view
    shows the packing. Up to 256 rows the forward does overflow rows from the
    gate's spilled z instead of the fallback, and cuts rows of more than 384
    units over several workgroups (another sum order): there the other rows
    are compared bit for bit and these against the definition."""
    inp, _, _, Y = small_case(name)
    w = inp.workload
    x, Wg, WuT, Wd = dev(inp)
    y_full = tw.ffn_forward(x, Wg, WuT, Wd, w.T, w.C, y=nan_y(w.M, w.d))
    view = host_packing(tw.packed_view(w.M, w.d, w.F, w.T, w.C, device=DEV))
    p = tw.gate_pack(x, Wg, w.T, w.C)
    g = host_packing(p)
    assert np.array_equal(view["counts"], g["counts"]) and np.array_equal(view["ovf"], g["ovf"])
    # the forward's gate (for few tokens split over K across workgroups, in the
    # same sum order) packs the same bits as the standalone single launch
    used = used_slots(g["counts"], w.C)
    assert np.array_equal(view["idx"][used], g["idx"][used])
    assert np.array_equal(view["vals"][used].view(np.uint32), g["vals"][used].view(np.uint32))
    # the forward's choice: the sliced form above 256 rows, where d allows it
    updown = tw.sliced_updown if (w.M > 256 and sliced_ok(w.d)) else tw.fused_updown
    y = updown(x, WuT, Wd, p, y=nan_y(w.M, w.d))
    yh = y.cpu().numpy()
    ovf = g["ovf"]
    fit = np.setdiff1d(np.arange(w.M), ovf)
    assert np.isnan(yh[ovf]).all(), "up/down kernel wrote an overflow row"
    assert np.isfinite(yh[fit]).all()
    tw.dense_fallback(x, Wg, WuT, Wd, p, y)
    yc, yf = y.cpu().numpy(), y_full.cpu().numpy()
    if w.M > 256:
        assert np.array_equal(yc.view(np.uint32), yf.view(np.uint32))
    else:
        total = g["counts"].astype(np.int64).sum(axis=1)
        same = np.setdiff1d(fit, np.flatnonzero(total > 384))
        other = np.union1d(ovf, np.flatnonzero(total > 384))
        assert np.array_equal(yc[same].view(np.uint32), yf[same].view(np.uint32))
        if len(other):
            rel, _ = check_y(yf[other], Y[other])
            print(f"{name}: {len(ovf)} overflow rows from the spill, {len(other)} rows spilled or cut, rel L2 {rel:.2e}")


@pytest.mark.parametrize("name", list(SMALL))
def test_updown_kernels_match_definition(name):
    """Both up/down forms, each completed by the fallback, against the fp64
    definition, and against each other."""
    inp, _, _, Y = small_case(name)
    w = inp.workload
    x, Wg, WuT, Wd = dev(inp)
    p = tw.gate_pack(x, Wg, w.T, w.C)
    g = host_packing(p)
    outs = {}
    forms = [("fused", tw.fused_updown)] + ([("sliced", tw.sliced_updown)] if sliced_ok(w.d) else [])
    for label, fn in forms:
        y = fn(x, WuT, Wd, p, y=nan_y(w.M, w.d))
        tw.dense_fallback(x, Wg, WuT, Wd, p, y)
        outs[label] = y.cpu().numpy()
        rel, mx = check_y(outs[label], Y)
        print(f"{name} [{label}]: rel L2 {rel:.2e}, max abs {mx:.2e}, overflow rows {g['n_ovf']}")
    if "sliced" in outs:
        a, b = outs["fused"], outs["sliced"]
        assert np.abs(a - b).max() <= 1e-5 * max(np.abs(a).max(), 1e-30)


@pytest.mark.parametrize("name", ["uniform_ragged", "zipf_small", "long_rows", "fused_only_d2304", "few_rows_d2560"])
def test_fused_forms_agree(name):
    """The fused kernel runs a workgroup per token up to 256 rows and a wave
    per token above; rows are independent and both forms take every
    product and sum in the same order, so a batch's first rows alone give the
    same bits as the whole batch. The case's rows are repeated up to 300."""
    inp, _, _, _ = small_case(name)
    w = inp.workload
    x, Wg, WuT, Wd = dev(inp)
    big = x.repeat(-(-300 // w.M), 1)[:max(300, w.M)].contiguous()
    p = tw.gate_pack(big, Wg, w.T, w.C)
    full = tw.fused_updown(big, WuT, Wd, p, y=nan_y(big.shape[0], w.d))
    k = 37
    head = tw.Packed(p.vals[:k], p.idx[:k], p.counts[:k], p.ovf_rows[:k], p.n_ovf, p.T, p.C)
    part = tw.fused_updown(big[:k].contiguous(), WuT, Wd, head, y=nan_y(k, w.d))
    a, b = full[:k].cpu().numpy(), part.cpu().numpy()
    assert np.array_equal(np.isnan(a), np.isnan(b))  # overflow rows: written by neither
    assert np.isfinite(a).any()
    assert np.array_equal(a[~np.isnan(a)].view(np.uint32), b[~np.isnan(b)].view(np.uint32))


@pytest.mark.parametrize("name", ["few_rows_d768", "heavytail_small", "dense11_small"])
def test_forward_graph_replay(name):
    """The forward holds no host synchronisation and no allocation, and its
    control block is zero again after every call, so a HIP graph of two
    forwards replays to the eager result's bits every time (cases with and
    without overflow rows; eager work and a synchronisation between replays)."""
    inp, _, _, _ = small_case(name)
    w = inp.workload
    x, Wg, WuT, Wd = dev(inp)
    ws, ctrl = tw.Workspace(DEV), tw.Workspace(DEV, zeroed=True)
    y = nan_y(w.M, w.d)
    tw.ffn_forward(x, Wg, WuT, Wd, w.T, w.C, y=y, workspace=ws, ctrl=ctrl)
    torch.cuda.synchronize()
    ref = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(2):
            tw.ffn_forward(x, Wg, WuT, Wd, w.T, w.C, y=y, workspace=ws, ctrl=ctrl)
    for _ in range(4):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), ref.view(torch.int32))
    del g
    tw.ffn_forward(x, Wg, WuT, Wd, w.T, w.C, y=y, workspace=ws, ctrl=ctrl)  # eager again after the replays
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), ref.view(torch.int32))


def _bits_to_mask(bits, F):
    w = bits.cpu().numpy().view(np.uint32)
    return ((w[np.arange(F) // 32] >> (np.arange(F) % 32).astype(np.uint32)) & 1).astype(bool)


@pytest.mark.parametrize("name", ["heavytail_small", "uniform_ragged", "t64_odd_tiles", "few_rows_d768",
                                  "dense11_small", "zipf_small"])
def test_column_activity(name):
    """Unit activity over the batch: equal to the oracle's on the kernel's own
    z (bit-exact mode); against fp64 z only near-zero columns may differ;
    never-active units by construction stay inactive; two half batches
    accumulate to the whole batch's bits."""
    inp, Z, rms, _ = small_case(name)
    w = inp.workload
    x, Wg, _, _ = dev(inp)
    bits = tw.column_activity(x, Wg, w.T, w.C)
    got = _bits_to_mask(bits, w.F)
    _, z32 = run_gate(inp, debug=True)
    assert np.array_equal(got, O.column_activity(z32))
    ref = O.column_activity(Z)
    diff = np.flatnonzero(got != ref)
    for j in diff:  # a differing column may only hold |z| near zero where the two disagree
        rows = np.flatnonzero((z32[:, j] > 0) != (Z[:, j] > 0))
        assert np.abs(Z[rows, j]).max() < 1e-3 * rms[j]
    if "dead" in inp.info and inp.info["dead"].any():
        assert not got[inp.info["dead"]].any()
    k = w.M // 2
    acc = tw.column_activity(x[:k].contiguous(), Wg, w.T, w.C)
    acc = tw.column_activity(x[k:].contiguous(), Wg, w.T, w.C, bits=acc)
    assert torch.equal(acc, bits)


@pytest.mark.parametrize("name", ["heavytail_small", "t64_odd_tiles", "few_rows_d2560"])
def test_compacted_layer(name):
    """The layer without its never-active units: rows bit-exact against the
    oracle's selection, and the forward on it equals the full layer's
    definition (the dropped units contribute exact zeros)."""
    inp, Z, _, Y = small_case(name)
    w = inp.workload
    x, Wg, WuT, Wd = dev(inp)
    bits = tw.column_activity(x, Wg, w.T, w.C)
    Wg_c, WuT_c, Wd_c, src = tw.compact_layer(Wg, WuT, Wd, bits, w.T)
    _, z32 = run_gate(inp, debug=True)
    want_src = O.live_layout(O.column_activity(z32), w.T)
    assert np.array_equal(src.cpu().numpy().astype(np.int64), want_src)
    for dev_c, host in ((Wg_c, inp.Wg), (WuT_c, inp.WuT), (Wd_c, inp.Wd)):
        got = dev_c.cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, O.compact_rows(host, want_src))
    Fc = Wg_c.shape[0]
    assert Fc % w.T == 0 and Fc <= w.F
    y = tw.ffn_forward(x, Wg_c, WuT_c, Wd_c, w.T, w.C, y=nan_y(w.M, w.d)).cpu().numpy()
    rel, mx = check_y(y, Y)
    print(f"{name}: F {w.F} -> {Fc} live+pad, rel L2 {rel:.2e}")


# ------------------------------------------------------------------ training
# (case, K, R): K near the mean active count so both kinds of rows occur; the
# reserve holds every row that needs it.
TRAIN = {
    "tiny": (48, 64),
    "uniform_ragged": (8, 300),
    "heavytail_small": (40, 1100),
    "zipf_small": (16, 520),
    "few_rows_d768": (6, 5),
    "d2048_small": (20, 200),
}


@functools.lru_cache(maxsize=1)
def train_case(name):
    inp = make_inputs(SMALL[name] if name in SMALL else WORKLOADS[name])
    w = inp.workload
    K, R = TRAIN[name]
    x, Wg, WuT, Wd = dev(inp)
    z = torch.empty((w.M, w.F), dtype=torch.float32, device=DEV)
    p = tw.gate_pack(x, Wg, w.T, w.T, z_debug=z)  # C = T: every active unit is kept
    hy = tw.hybrid_pack(p, w.F, K, R)
    torch.cuda.synchronize()
    z32 = z.cpu().numpy()
    return inp, z32, O.hybrid_pack(z32, K), hy, make_upstream_grad(w)


def check_hybrid(hy, ref, K, R):
    """A device hybrid format against the oracle's, bit for bit."""
    count = hy.count.cpu().numpy()
    assert np.array_equal(count, ref.count)
    idx, vals = hy.idx.cpu().numpy(), hy.vals.cpu().numpy()
    for r in np.flatnonzero(count <= K):
        n = count[r]
        assert np.array_equal(idx[r, :n], ref.idx[r, :n])
        assert np.array_equal(vals[r, :n].view(np.uint32), ref.vals[r, :n].view(np.uint32))
    n_res = int(hy.n_res.item())
    assert n_res == len(ref.res_rows) and n_res <= R
    rows = hy.res_rows.cpu().numpy()[:n_res]
    assert np.array_equal(np.sort(rows), ref.res_rows)
    dense = hy.res_vals.cpu().numpy()[:n_res]
    order = np.argsort(rows)
    assert np.array_equal(dense[order].view(np.uint32), ref.res_vals.view(np.uint32))
    for i, r in enumerate(rows):  # a reserve row's block names its slot
        assert idx[r, 0] == i
    return count, n_res


@pytest.mark.parametrize("name", list(TRAIN))
def test_hybrid_pack(name):
    """Hybrid format against the oracle's on the kernel's own z: bit-exact."""
    inp, z32, ref, hy, _ = train_case(name)
    w = inp.workload
    K, R = TRAIN[name]
    count, n_res = check_hybrid(hy, ref, K, R)
    print(f"{name}: K={K}, reserve rows {n_res} of {w.M}, mean count {count.mean():.1f}")


@pytest.mark.parametrize("name", list(TRAIN))
def test_backward(name):
    """dx, dWg, dWuT, dWd against the oracle on the same active set (fp64
    sparse evaluation of the oracle's hybrid format) and against the dense
    definition; two runs give the same bits."""
    inp, z32, ref, hy, dy_bits = train_case(name)
    w = inp.workload
    x, Wg, WuT, Wd = dev(inp)
    dy = to_device(dy_bits, DEV)
    got = [t.cpu().numpy() for t in tw.ffn_backward(x, Wg, WuT, Wd, dy, hy)]
    want = O.ffn_backward_from_hybrid(ref, inp.x, inp.Wg, inp.WuT, inp.Wd, dy_bits)
    dense = O.ffn_backward(inp.x, inp.Wg, inp.WuT, inp.Wd, dy_bits)
    for label, g, a, b in zip(("dx", "dWg", "dWuT", "dWd"), got, want, dense):
        rel, mx = check_y(g, a)
        rel_d, _ = check_y(g, b)
        print(f"{name} {label}: rel L2 {rel:.2e} (same active set), {rel_d:.2e} (dense definition)")
    again = [t.cpu().numpy() for t in tw.ffn_backward(x, Wg, WuT, Wd, dy, hy)]
    for g, h in zip(got, again):
        assert np.array_equal(g.view(np.uint32), h.view(np.uint32))


@pytest.mark.parametrize("name", list(SMALL))
def test_dense_baseline(name):
    inp, _, _, Y = small_case(name)
    w = inp.workload
    y = tw.dense_ffn_forward(*dev(inp), y=nan_y(w.M, w.d)).cpu().numpy()
    assert np.isfinite(y).all()
    rel, mx, mref = y_errors(y, Y)
    print(f"{name}: dense baseline (bf16 hidden) rel L2 {rel:.2e}")
    assert rel < 5e-3  # bf16 rounding of h gives ~1.5e-3 by design; reported, not gated at 1e-3


# Shapes for the dense baseline's tiling: 256-token x 128-unit gated-up tiles
# and 256 x 256 down tiles whose K range is split when there are fewer tiles
# than CUs (S = 1, 4, 5, 7, 8 below), ragged token counts, F % 128 == 64.
DENSE_SHAPES = {
    "one_token_s8": scaled(WORKLOADS["ffn1p5b"], M=1, d=512, F=2048),
    "ragged_f1088_s4": scaled(WORKLOADS["ffn1p5b"], M=300, d=256, F=1088, T=64),
    "d768_s5": scaled(WORKLOADS["ffn1p5b"], M=600, d=768, F=1280),
    "d1024_s7": scaled(WORKLOADS["ffn1p5b"], M=2100, d=1024, F=4096),
    "unsplit_d4096": scaled(WORKLOADS["ffn1p5b"], M=4100, d=4096, F=512),
    # the largest d the library takes (32 down tiles across, S = 2)
    "d8192_max": scaled(WORKLOADS["ffn1p5b"], M=300, d=8192, F=512),
    # F / 32 below the ring's 8 chunks: the register-staged kernels run it
    "register_staged_f128": scaled(WORKLOADS["ffn1p5b"], M=100, d=256, F=128),
}


@pytest.mark.parametrize("name", list(DENSE_SHAPES))
def test_dense_baseline_shapes(name):
    inp = make_inputs(DENSE_SHAPES[name])
    w = inp.workload
    Y = O.dense_gated_ffn(inp.x, inp.Wg, inp.WuT, inp.Wd)
    args = dev(inp)
    y = tw.dense_ffn_forward(*args, y=nan_y(w.M, w.d))
    again = tw.dense_ffn_forward(*args, y=nan_y(w.M, w.d))
    y, again = y.cpu().numpy(), again.cpu().numpy()
    assert np.isfinite(y).all()
    assert np.array_equal(y.view(np.uint32), again.view(np.uint32))  # fixed sum order
    rel, mx, mref = y_errors(y, Y)
    print(f"{name}: dense baseline rel L2 {rel:.2e}, max {mx:.2e} of {mref:.2e}")
    assert rel < 5e-3 and mx <= 2e-2 * mref


# ------------------------------------------------------------------ edge cases
def _edge_inputs(M, d, F, bias, seed=5):
    rng = np.random.default_rng(seed)

    def b16(a):
        return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)

    x = rng.standard_normal((M, d)).astype(np.float32)
    x[:, 0] = 1
    Wg = (rng.standard_normal((F, d)) / np.sqrt(d)).astype(np.float32)
    Wg[:, 0] = bias
    WuT = (rng.standard_normal((F, d)) / np.sqrt(d)).astype(np.float32)
    Wd = (rng.standard_normal((F, d)) / np.sqrt(F)).astype(np.float32)
    return [b16(a) for a in (x, Wg, WuT, Wd)]


def test_empty_batch():
    d, F, T, C = 256, 1024, 64, 8
    x = torch.empty((0, d), dtype=torch.bfloat16, device=DEV)
    Ws = [torch.zeros((F, d), dtype=torch.bfloat16, device=DEV) for _ in range(3)]
    y = tw.ffn_forward(x, *Ws, T, C)
    p = tw.gate_pack(x, Ws[0], T, C)
    torch.cuda.synchronize()
    assert y.shape == (0, d) and int(p.n_ovf.item()) == 0


def test_single_row_and_zero_density():
    for M, bias in ((1, 0.0), (77, -1000.0)):
        d, F, T, C = 512, 1024, 128, 16
        arrs = _edge_inputs(M, d, F, bias)
        x, Wg, WuT, Wd = (to_device(a, DEV) for a in arrs)
        y = tw.ffn_forward(x, Wg, WuT, Wd, T, C, y=nan_y(M, d)).cpu().numpy()
        Y = O.dense_gated_ffn(*arrs)
        check_y(y, Y)
        if bias < 0:
            assert np.all(y == 0)
            assert np.all(host_packing(tw.gate_pack(x, Wg, T, C))["counts"] == 0)


def test_all_active_goes_to_fallback():
    M, d, F, T, C = 200, 512, 1024, 64, 8
    arrs = _edge_inputs(M, d, F, 1000.0)
    x, Wg, WuT, Wd = (to_device(a, DEV) for a in arrs)
    g = host_packing(tw.gate_pack(x, Wg, T, C))
    assert np.all(g["counts"] == T) and np.array_equal(g["ovf"], np.arange(M))
    y = tw.ffn_forward(x, Wg, WuT, Wd, T, C, y=nan_y(M, d)).cpu().numpy()
    check_y(y, O.dense_gated_ffn(*arrs))


def test_deterministic_and_control_block_reset():
    inp, _, _, _ = small_case("heavytail_small")
    w = inp.workload
    x, Wg, WuT, Wd = dev(inp)
    y1 = tw.ffn_forward(x, Wg, WuT, Wd, w.T, w.C).cpu().numpy()
    p1 = host_packing(tw.packed_view(w.M, w.d, w.F, w.T, w.C, device=DEV))
    assert p1["n_ovf"] > 0
    # a call with no overflow rows in between must leave an empty set
    x0 = x.clone()
    x0[:, 1:] = 0  # every gate pre-activation is its (negative) bias: nothing fires
    p0 = host_packing(tw.gate_pack(x0, Wg, w.T, w.C))
    assert p0["n_ovf"] == 0 and np.all(p0["counts"] == 0)
    y2 = tw.ffn_forward(x, Wg, WuT, Wd, w.T, w.C).cpu().numpy()
    p2 = host_packing(tw.packed_view(w.M, w.d, w.F, w.T, w.C, device=DEV))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    assert np.array_equal(p1["ovf"], p2["ovf"]) and np.array_equal(p1["counts"], p2["counts"])


@pytest.mark.parametrize("name", ["heavytail_small", "few_rows_d768"])
def test_forward_timed(name):
    """twell_ffn_forward_timed runs the forward's kernels (large and
    small-batch paths): the same y bits as twell_ffn_forward, and its two
    events bracket a non-empty gate."""
    inp, _, _, _ = small_case(name)
    w = inp.workload
    x, Wg, WuT, Wd = dev(inp)
    y1 = tw.ffn_forward(x, Wg, WuT, Wd, w.T, w.C).cpu().numpy()
    b, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    y2 = tw.ffn_forward_timed(x, Wg, WuT, Wd, w.T, w.C, b, e, y=nan_y(w.M, w.d))
    torch.cuda.synchronize()
    assert np.array_equal(y1.view(np.uint32), y2.cpu().numpy().view(np.uint32))
    assert b.elapsed_time(e) > 0.0


# ------------------------------------------------------------------ full sizes
def _chunked(fn, M, step=2048):
    return np.concatenate([fn(np.arange(s, min(s + step, M))) for s in range(0, M, step)])


@pytest.mark.parametrize("name", FULL)
def test_full_size(name):
    """The bench configuration (twell_ffn_forward) at the full workload size,
    checked over the whole layer: the forward's own packing and the bit-exact
    mode's packing both equal the oracle's packing of the bit-exact mode's z,
    every active set against the fp64 pre-activations, and every row of y
    against the fp64 definition; then the single-kernel form and the dense
    baseline on the same layer."""
    inp = make_inputs(WORKLOADS[name])
    w = inp.workload
    print(f"[full] {name} M={w.M} d={w.d} F={w.F} T={w.T} C={w.C}", flush=True)
    x, Wg, WuT, Wd = dev(inp)
    y = tw.ffn_forward(x, Wg, WuT, Wd, w.T, w.C, y=nan_y(w.M, w.d))
    view = host_packing(tw.packed_view(w.M, w.d, w.F, w.T, w.C, device=DEV))
    yh = y.cpu().numpy()
    assert np.isfinite(yh).all(), "some row of y was not written"

    # bit-exact packing of the whole layer: the bit-exact mode's z packed by the
    # oracle, against that mode's packing and against the forward's own (the
    # gate instance the forward runs computes the same z)
    z = torch.empty((w.M, w.F), dtype=torch.float32, device=DEV)
    dbg = host_packing(tw.gate_pack(x, Wg, w.T, w.C, z_debug=z))
    zh = z.cpu().numpy()
    del z
    ref = O.pack_twell(zh, w.T, w.C)
    del zh
    check_packing_bitexact(dbg, ref)
    check_packing_bitexact(view, ref)
    del ref

    # whole layer: active sets and y against the fp64 definition
    Z = _chunked(lambda r: O.gate_preactivations(inp.x, inp.Wg, rows=r), w.M)
    rms = O.column_rms(Z)
    check_active_set(view, Z, rms, w.T, w.C)
    del Z
    Y = _chunked(lambda r: O.dense_gated_ffn(inp.x, inp.Wg, inp.WuT, inp.Wd, rows=r), w.M)
    rel, mx = check_y(yh, Y)
    print(f"[full] {name}: overflow rows {view['n_ovf']}, whole-tensor rel L2 {rel:.2e}, max abs {mx:.2e}",
          flush=True)

    # the single-kernel up/down form on the same packing, completed by the fallback
    p = tw.gate_pack(x, Wg, w.T, w.C)
    yf = tw.fused_updown(x, WuT, Wd, p, y=nan_y(w.M, w.d))
    tw.dense_fallback(x, Wg, WuT, Wd, p, yf)
    rel_f, _ = check_y(yf.cpu().numpy(), Y)
    print(f"[full] {name}: fused form whole-tensor rel L2 {rel_f:.2e}")

    # the dense baseline on the same layer (bf16 hidden: its error is reported
    # and loosely bounded, as in the small cases)
    yd = tw.dense_ffn_forward(x, Wg, WuT, Wd, y=nan_y(w.M, w.d)).cpu().numpy()
    assert np.isfinite(yd).all()
    rel_d, mx_d, mref_d = y_errors(yd, Y)
    print(f"[full] {name}: dense baseline whole-tensor rel L2 {rel_d:.2e}")
    assert rel_d < 5e-3 and mx_d <= 2e-2 * mref_d


@pytest.mark.parametrize("name", ["ffn1p5b", "ffn1p5b_heavytail"])
def test_backward_full_size(name):
    """The training backward at full size (K = 64, R = 512, as bench.py runs
    it): counts and sampled rows' blocks of the hybrid format bit-exact,
    dx on sampled rows and the three weight gradients on sampled units against
    the oracle on the kernel's active set (its fp32 z decides, as in the
    packing)."""
    inp = make_inputs(WORKLOADS[name])
    w = inp.workload
    K, R = 64, 512
    print(f"[full-bwd] {name} M={w.M} d={w.d} F={w.F} K={K} R={R}", flush=True)
    x, Wg, WuT, Wd = dev(inp)
    dy_bits = make_upstream_grad(w)
    dy = to_device(dy_bits, DEV)
    z = torch.empty((w.M, w.F), dtype=torch.float32, device=DEV)
    p = tw.gate_pack(x, Wg, w.T, w.T, z_debug=z)
    hy = tw.hybrid_pack(p, w.F, K, R)
    dx, dWg, dWu, dWd = (t.cpu().numpy() for t in tw.ffn_backward(x, Wg, WuT, Wd, dy, hy))
    z32 = z.cpu().numpy()
    del z
    count = hy.count.cpu().numpy()
    assert np.array_equal(count, (z32 > 0).sum(axis=1))
    n_res = int(hy.n_res.item())
    assert n_res == int((count > K).sum()) and n_res <= R
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([rng.choice(w.M, 48, replace=False),
                                     np.flatnonzero(count > K)[:16]]))  # reserve rows too
    ref_rows = O.hybrid_pack(z32[rows], K)
    idx = hy.idx.cpu().numpy()
    for i, r in enumerate(rows):
        if count[r] <= K:
            assert np.array_equal(idx[r, :count[r]], ref_rows.idx[i, :count[r]])
    hy_rows = O.hybrid_pack(z32[rows], w.F)  # every sampled row as one block
    want_dx = O.ffn_backward_from_hybrid(hy_rows, inp.x[rows], inp.Wg, inp.WuT, inp.Wd, dy_bits[rows])[0]
    rel, _ = check_y(dx[rows], want_dx)
    units = np.unique(rng.choice(w.F, 48, replace=False))
    hy_units = O.hybrid_pack(z32[:, units], len(units))  # the sampled units alone
    _, gWg, gWu, gWd = O.ffn_backward_from_hybrid(hy_units, inp.x, inp.Wg[units], inp.WuT[units],
                                                  inp.Wd[units], dy_bits)
    rels = [check_y(got[units], want)[0] for got, want in ((dWg, gWg), (dWu, gWu), (dWd, gWd))]
    print(f"[full-bwd] {name}: reserve rows {n_res}, dx rel L2 {rel:.2e}, dW rel L2 {max(rels):.2e}")


def test_training_edge_cases():
    """M = 0 (weight gradients all zero, nothing else touched), one row, a
    batch with no active unit, and R = 0 with every row in blocks."""
    w = SMALL["few_rows_d768"]
    inp = make_inputs(w)
    x, Wg, WuT, Wd = dev(inp)
    dy_bits = make_upstream_grad(w)
    dy = to_device(dy_bits, DEV)
    # M = 0
    p0 = tw.gate_pack(x[:0], Wg, w.T, w.T)
    hy0 = tw.hybrid_pack(p0, w.F, 8, 0)
    assert int(hy0.n_res.item()) == 0
    g0 = tw.ffn_backward(x[:0], Wg, WuT, Wd, dy[:0], hy0)
    for t in g0[1:]:
        assert torch.count_nonzero(t).item() == 0
    # one row, K large enough for every row (R = 0)
    z = torch.empty((1, w.F), dtype=torch.float32, device=DEV)
    p1 = tw.gate_pack(x[:1].contiguous(), Wg, w.T, w.T, z_debug=z)
    hy1 = tw.hybrid_pack(p1, w.F, w.F, 0)
    got = [t.cpu().numpy() for t in tw.ffn_backward(x[:1].contiguous(), Wg, WuT, Wd, dy[:1].contiguous(), hy1)]
    want = O.ffn_backward_from_hybrid(O.hybrid_pack(z.cpu().numpy(), w.F), inp.x[:1], inp.Wg, inp.WuT, inp.Wd,
                                      dy_bits[:1])
    for g, r in zip(got, want):
        check_y(g, r)
    # no active unit at all: every gradient is exactly zero
    Wneg = (-Wg.float().abs()).to(torch.bfloat16).contiguous()
    xpos = x.float().abs().to(torch.bfloat16).contiguous()
    pz = tw.gate_pack(xpos, Wneg, w.T, w.T)
    hyz = tw.hybrid_pack(pz, w.F, 8, w.M)
    assert int(hyz.count.sum().item()) == 0
    for t in tw.ffn_backward(xpos, Wneg, WuT, Wd, dy, hyz):
        assert torch.count_nonzero(t).item() == 0


# ------------------------------------------------------------ gate-only variant
GATEUP_SMALL = ["tiny", "uniform_ragged", "heavytail_small", "zipf_small", "t64_odd_tiles", "dense11_small",
                "long_rows", "few_rows_d768", "few_rows_cut_spill", "d2048_small"]


def run_gateup(inp, debug=True):
    w = inp.workload
    x, Wg, WuT, _ = dev(inp)
    z = torch.empty((w.M, w.F), dtype=torch.float32, device=DEV) if debug else None
    h = torch.empty((w.M, w.F), dtype=torch.float32, device=DEV) if debug else None
    p = tw.gateup_pack(x, Wg, WuT, w.T, w.C, z_debug=z, h_debug=h)
    torch.cuda.synchronize()
    return p, (z.cpu().numpy() if debug else None), (h.cpu().numpy() if debug else None)


@pytest.mark.parametrize("name", GATEUP_SMALL)
def test_gateup_packing_bitexact(name):
    """Packing of h against the oracle fed the kernel's own z and h, bit for
    bit; the debug-free instance gives the same bits; z and h agree with the
    fp64 definition (checks the two MFMA products and their layout)."""
    inp, Z, rms, _ = small_case(name)
    w = inp.workload
    p, z, h = run_gateup(inp)
    assert np.abs(z - Z).max() <= 1e-4 * rms.max()
    U = O.up_projections(inp.x, inp.WuT)
    H = np.maximum(Z, 0) * U
    act = z > 0
    assert np.abs(h[act] - (np.maximum(z, 0) * U)[act]).max() <= 1e-4 * max(np.abs(H).max(), 1e-30)
    ref = O.pack_twell_hidden(z, h, w.T, w.C)
    check_packing_bitexact(host_packing(p), ref)
    p2, _, _ = run_gateup(inp, debug=False)
    check_packing_bitexact(host_packing(p2), ref)
    # z is summed in the same k order as in the gate kernel, so the counts,
    # indices and overflow set are that kernel's; the active sets against fp64 z
    g = host_packing(tw.gate_pack(*dev(inp)[:2], w.T, w.C))
    assert np.array_equal(g["counts"], ref.counts) and np.array_equal(g["ovf"], ref.ovf)
    check_active_set(dict(counts=ref.counts, idx=ref.idx, vals=O.pack_twell(z, w.T, w.C).vals), Z, rms, w.T, w.C)


@pytest.mark.parametrize("name", GATEUP_SMALL)
def test_gateup_forward_matches_definition(name):
    """The gate-only forward against the fp64 definition over the whole
    tensor; gateup_pack + hidden_down + dense_fallback give its bits, and
    hidden_down leaves overflow rows untouched."""
    inp, _, _, Y = small_case(name)
    w = inp.workload
    x, Wg, WuT, Wd = dev(inp)
    y = tw.ffn_forward_gateup(x, Wg, WuT, Wd, w.T, w.C, y=nan_y(w.M, w.d))
    yh = y.cpu().numpy()
    rel, mx = check_y(yh, Y)
    p = tw.gateup_pack(x, Wg, WuT, w.T, w.C)
    g = host_packing(p)
    yc = tw.hidden_down(Wd, p, nan_y(w.M, w.d))
    yc_h = yc.cpu().numpy()
    fit = np.setdiff1d(np.arange(w.M), g["ovf"])
    assert np.isnan(yc_h[g["ovf"]]).all() and np.isfinite(yc_h[fit]).all()
    tw.dense_fallback(x, Wg, WuT, Wd, p, yc)
    assert np.array_equal(yc.cpu().numpy().view(np.uint32), yh.view(np.uint32))
    print(f"{name}: gate-only forward rel L2 {rel:.2e}, overflow rows {g['n_ovf']}")


def test_gateup_unsupported_d():
    inp, _, _, _ = small_case("fused_only_d2304")
    w = inp.workload
    with pytest.raises(tw.TwellError) as e:
        tw.ffn_forward_gateup(*dev(inp), w.T, w.C)
    assert e.value.status == -2


@pytest.mark.parametrize("name", ["ffn1p5b", "sweep_p1pct", "sweep_p3pct", "sweep_p11pct"])
def test_gateup_full_size(name):
    """The gate-only forward at full size: packing bit-exact against the
    oracle on the kernel's z and h, y over the whole tensor against the fp64
    definition."""
    inp = make_inputs(WORKLOADS[name])
    w = inp.workload
    print(f"[gateup-full] {name} M={w.M} d={w.d} F={w.F} T={w.T} C={w.C}", flush=True)
    x, Wg, WuT, Wd = dev(inp)
    ws = tw.Workspace(DEV)
    y = tw.ffn_forward_gateup(x, Wg, WuT, Wd, w.T, w.C, y=nan_y(w.M, w.d), workspace=ws)
    view = host_packing(tw.packed_view(w.M, w.d, w.F, w.T, w.C, workspace=ws, device=DEV))
    yh = y.cpu().numpy()
    assert np.isfinite(yh).all()
    p, z, h = run_gateup(inp)
    ref = O.pack_twell_hidden(z, h, w.T, w.C)
    del z, h
    check_packing_bitexact(host_packing(p), ref)
    check_packing_bitexact(view, ref)
    del ref
    Y = _chunked(lambda r: O.dense_gated_ffn(inp.x, inp.Wg, inp.WuT, inp.Wd, rows=r), w.M)
    rel, mx = check_y(yh, Y)
    print(f"[gateup-full] {name}: overflow rows {view['n_ovf']}, whole-tensor rel L2 {rel:.2e}", flush=True)


# ------------------------------------------- training gate with spill records
# (case, K, R) with C < T: tiles over C reach the hybrid format through the
# spill list instead of a C = T packing.
SPILL_TRAIN = {
    "tiny": (48, 64),
    "uniform_ragged": (8, 300),
    "heavytail_small": (40, 1100),
    "zipf_small": (16, 520),
    "dense11_small": (40, 257),
    "few_rows_cut_spill": (600, 24),
}


def run_gate_spill(inp, cap=None):
    w = inp.workload
    x, Wg, _, _ = dev(inp)
    nT = w.F // w.T
    cap = w.M * nT if cap is None else cap
    z = torch.empty((w.M, w.F), dtype=torch.float32, device=DEV)
    p, sp = tw.gate_pack_spill(x, Wg, w.T, w.C, cap, z_debug=z)
    torch.cuda.synchronize()
    return p, sp, z.cpu().numpy()


@pytest.mark.parametrize("name", list(SPILL_TRAIN))
def test_gate_spill_records(name):
    """The training gate: packing bit-exact against the oracle on its own z;
    one spill record per (row, tile) over C holding that tile's z bits; with
    a list too short the count still covers every tile."""
    inp, _, _, _ = small_case(name)
    w = inp.workload
    nT = w.F // w.T
    p, sp, z32 = run_gate_spill(inp)
    ref = O.pack_twell(z32, w.T, w.C)
    check_packing_bitexact(host_packing(p), ref)
    over = ref.counts.astype(np.int64) > w.C
    n = int(sp.n_spill.item())
    assert n == int(over.sum())
    slots = sp.slot.cpu().numpy()[over]
    assert np.array_equal(np.sort(slots), np.arange(n))
    recs = sp.z.cpu().numpy()[slots]
    assert np.array_equal(recs.view(np.uint32), z32.reshape(w.M, nT, w.T)[over].view(np.uint32))
    if w.M > 256:  # the forward's gate kernel gives the same bits
        g = host_packing(tw.gate_pack(*dev(inp)[:2], w.T, w.C))
        check_packing_bitexact(g, ref)
    if n > 1:  # half the records: the rest are not stored, n_spill says so
        _, sp2, _ = run_gate_spill(inp, cap=n // 2)
        assert int(sp2.n_spill.item()) == n
    print(f"{name}: {n} spilled tiles of {w.M * nT}")


@pytest.mark.parametrize("name", list(SPILL_TRAIN))
def test_hybrid_from_spill(name):
    """The hybrid format from a C < T packing and its spill list equals the
    oracle's on the gate's z, bit for bit, and the backward over it matches
    the oracle on the same active set."""
    inp, _, _, _ = small_case(name)
    w = inp.workload
    K, R = SPILL_TRAIN[name]
    p, sp, z32 = run_gate_spill(inp)
    hy = tw.hybrid_pack(p, w.F, K, R, spill=sp)
    ref = O.hybrid_pack(z32, K)
    count, n_res = check_hybrid(hy, ref, K, R)
    x, Wg, WuT, Wd = dev(inp)
    dy_bits = make_upstream_grad(w)
    got = [t.cpu().numpy() for t in tw.ffn_backward(x, Wg, WuT, Wd, to_device(dy_bits, DEV), hy)]
    want = O.ffn_backward_from_hybrid(ref, inp.x, inp.Wg, inp.WuT, inp.Wd, dy_bits)
    for label, g, a in zip(("dx", "dWg", "dWuT", "dWd"), got, want):
        rel, _ = check_y(g, a)
    print(f"{name}: K={K}, C={w.C}, spilled {int(sp.n_spill.item())}, reserve rows {n_res}")


def test_training_spill_full_size():
    """Heavy-tailed layer at full size (C = 16, K = 64, R = 512): the hybrid
    format from the spill list is the C = T route's, bit for bit, and so are
    the gradients."""
    w = WORKLOADS["ffn1p5b_heavytail"]
    inp = make_inputs(w)
    K, R = 64, 512
    x, Wg, WuT, Wd = dev(inp)
    dy = to_device(make_upstream_grad(w), DEV)
    p, sp = tw.gate_pack_spill(x, Wg, w.T, w.C, 16384)
    hy = tw.hybrid_pack(p, w.F, K, R, spill=sp)
    n = int(sp.n_spill.item())
    assert 0 < n <= 16384
    full = tw.hybrid_pack(tw.gate_pack(x, Wg, w.T, w.T), w.F, K, R)
    for a, b in ((hy.count, full.count), (hy.n_res, full.n_res)):
        assert torch.equal(a, b)
    count = hy.count.cpu().numpy()
    fit = count <= K
    for a, b in ((hy.idx, full.idx), (hy.vals, full.vals)):
        ah, bh = a.cpu().numpy(), b.cpu().numpy()
        for r in np.flatnonzero(fit):
            assert np.array_equal(ah[r, :count[r]].view(np.uint32), bh[r, :count[r]].view(np.uint32))
    g1 = [t.cpu().numpy() for t in tw.ffn_backward(x, Wg, WuT, Wd, dy, hy)]
    g2 = [t.cpu().numpy() for t in tw.ffn_backward(x, Wg, WuT, Wd, dy, full)]
    for a, b in zip(g1, g2):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    print(f"[train-spill] spilled tiles {n}, reserve rows {int(hy.n_res.item())}")
