"""twell_ffn_forward_static (the allocation-free forward, scratch in a static
device buffer) against twell_ffn_forward on the same inputs, through the C
ABI: bit for bit (the same kernels run in the same order) and within the y
bar of the fp64 definition, on calls in a row that shrink, so a later call
finds the buffer holding an earlier, larger call's contents."""

from __future__ import annotations

import numpy as np
import pytest

import oracle as O
from synth import WORKLOADS, make_inputs, scaled

from _parity import check_y, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU only to be deselected by -m
    pytest.skip("needs a GPU", allow_module_level=True)

import activation_sparse_ffn_gate_amd as tw  # noqa: E402

DEV = torch.device("cuda", 0)

# Largest first: the decode batch of the 1.5B-like layer (256 rows), then rows
# of ~490 active units with C = 8 (overflowing tiles spilled, long rows cut
# over several workgroups), then one row of the 2B-like width.
CASES = [
    ("decode_m256", WORKLOADS["decode_m256"]),
    ("cut_spill_m24", scaled(WORKLOADS["sweep_p3pct"], M=24, d=512, F=16384, C=8)),
    ("zipf_m1", scaled(WORKLOADS["ffn2b_zipf"], M=1, d=2560, F=2560)),
]


def _run(w, inp):
    x, Wg, WuT, Wd = (to_device(a, DEV) for a in (inp.x, inp.Wg, inp.WuT, inp.Wd))
    nan = lambda: torch.full((w.M, w.d), float("nan"), dtype=torch.float32, device=DEV)  # noqa: E731
    y_static = tw.ffn_forward_static(x, Wg, WuT, Wd, w.T, w.C, y=nan())
    y_ref = tw.ffn_forward(x, Wg, WuT, Wd, w.T, w.C, y=nan())
    torch.cuda.synchronize()
    return y_static.cpu().numpy(), y_ref.cpu().numpy()


def test_static_forward_matches_forward():
    for name, w in CASES:
        print(f"[static] {name} M={w.M} d={w.d} F={w.F} T={w.T} C={w.C}", flush=True)
        inp = make_inputs(w)
        ys, yr = _run(w, inp)
        assert np.isfinite(ys).all(), f"{name}: a row of y was not written"
        assert np.array_equal(ys.view(np.uint32), yr.view(np.uint32)), f"{name}: differs from twell_ffn_forward"
        Y = O.dense_gated_ffn(inp.x, inp.Wg, inp.WuT, inp.Wd)
        rel, mx = check_y(ys, Y)
        counts = (O.gate_preactivations(inp.x, inp.Wg) > 0).reshape(w.M, w.F // w.T, w.T).sum(axis=2)
        print(f"[static] {name}: overflow rows {(counts.max(axis=1) > w.C).sum()}, rel L2 {rel:.2e}", flush=True)
    # a repeat of the first, larger case after the smaller ones
    w = CASES[0][1]
    ys, yr = _run(w, make_inputs(w))
    assert np.array_equal(ys.view(np.uint32), yr.view(np.uint32))


def test_static_forward_rejects_before_launch():
    w = CASES[0][1]
    x = torch.zeros((257, w.d), dtype=torch.bfloat16, device=DEV)
    W = torch.zeros((w.F, w.d), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(tw.TwellError) as e:
        tw.ffn_forward_static(x, W, W, W, w.T, w.C)
    assert e.value.status == -2
    W32 = torch.zeros((32768, 1024), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(tw.TwellError) as e:
        tw.ffn_forward_static(x[:256, :1024].contiguous(), W32, W32, W32, 128, 16)
    assert e.value.status == -5
    y = tw.ffn_forward_static(x[:0], W, W, W, w.T, w.C)
    assert y.shape == (0, w.d)
