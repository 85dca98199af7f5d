"""Throughput of the TwELL sparse gated-FFN forward on one MI355X.

One step = one twell_ffn_forward (gate GEMM + TwELL packing, up+down
projections over the packed non-zeros, dense fallback of overflow rows) over
the whole synthetic layer, inputs resident in HBM. Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--no-sweep]

The default workload is the 1.5B-like layer: M=4096 tokens, d=2048, F=8192,
about 29 active gate units per token, T=128, C=16. Besides the headline the
line carries per-kernel times, the roofline of the dominant kernel, warm and
cold (MALL flushed) latency percentiles of one forward, the dense baselines
(this library's MFMA kernels and a hipBLASLt one through torch) and a
density sweep (M=8192, d=2048, F=8192 at 0.1 .. 11 % active units) with the
sparse/dense ratio at every point.
"""

from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse FFN fwd tokens/s at d=2048,F=8192,~29 nnz/tok; % of HBM/MFMA roofline"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "activation_sparse_ffn_gate_amd", "csrc")
COPY_BYTES = 1 << 30  # --only copy default: 1 GiB read and 1 GiB written per launch


def sources_hash():
    """sha256 of the kernel sources, so recorded counters go stale with them."""
    import hashlib

    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def _counter_kib(path, counter, kernel=None):
    """Mean per-dispatch value of one rocprofv3 --pmc counter (KiB), over the
    dispatches whose kernel name contains `kernel` (all if None)."""
    import csv
    import glob

    vals = {}
    for fn in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter and (kernel is None or kernel in r["Kernel_Name"]):
                    vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} readings under {path}")
    return sum(vals.values()) / len(vals)


def record_traffic(root, workload):
    """Write profiles/traffic.json from rocprofv3 --pmc runs stored under root:
    pmc_<workload>_<leg>_fetch / _write for leg in gate, fused and sliced (the
    sliced leg holds its three kernels, row lists, up and down; their traffic
    is summed), scaled by
    pmc_copy_fetch / pmc_copy_write of a plain copy of known size. Workloads
    already recorded from the same kernel sources are kept."""
    cf = COPY_BYTES / 1024.0 / _counter_kib(os.path.join(root, "pmc_copy_fetch"), "FETCH_SIZE")
    cw = COPY_BYTES / 1024.0 / _counter_kib(os.path.join(root, "pmc_copy_write"), "WRITE_SIZE")
    rec = {"sources_sha256": sources_hash(), "calibration": {"fetch_factor": cf, "write_factor": cw,
                                                             "copy_bytes": COPY_BYTES}, "workloads": {}}
    if os.path.exists(TRAFFIC_FILE):  # keep other workloads recorded from the same sources
        with open(TRAFFIC_FILE) as f:
            old = json.load(f)
        if old.get("sources_sha256") == rec["sources_sha256"]:
            rec["workloads"] = old.get("workloads", {})
    ent = {}
    for leg, name, kernels in (("gate", "gate_pack", ["gate_pack"]), ("fused", "fused_updown", ["fused_updown"]),
                               ("sliced", "sliced_updown", ["row_list_kernel", "sliced_up_kernel", "sliced_down_kernel"])):
        d_f = os.path.join(root, f"pmc_{workload}_{leg}_fetch")
        if not os.path.isdir(d_f):
            continue
        fk = sum(_counter_kib(d_f, "FETCH_SIZE", k) for k in kernels)
        wk = sum(_counter_kib(os.path.join(root, f"pmc_{workload}_{leg}_write"), "WRITE_SIZE", k) for k in kernels)
        ent[name] = {"fetch_kib_raw": fk, "write_kib_raw": wk,
                     "traffic_bytes": fk * 1024.0 * cf + wk * 1024.0 * cw}
    rec["workloads"][workload] = ent
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ffn1p5b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="time budget of the CPU oracle sample")
    ap.add_argument("--only", choices=["forward", "gate", "fused", "sliced", "fallback", "dense", "copy", "backward",
                                       "gateup"],
                    default=None,
                    help="run only this leg (for profiler runs); prints a short line")
    ap.add_argument("--copy-mb", type=int, default=1024, help="size of the calibration copy (--only copy)")
    ap.add_argument("--record-traffic", metavar="DIR", default=None,
                    help="write profiles/traffic.json from rocprofv3 --pmc outputs under DIR (no GPU needed)")
    ap.add_argument("--no-sweep", action="store_true", help="skip the density sweep")
    ap.add_argument("--no-layers", action="store_true",
                    help="skip the heavy-tailed and 2B-like layers' forward legs")
    ap.add_argument("--compact", action="store_true",
                    help="with --only: run on the layer with its never-active units dropped")
    ap.add_argument("--sweep-steps", type=int, default=10)
    return ap.parse_args()


def time_loop(fn, steps, stream):
    import torch

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / steps  # ms per call


def latency(fn, n, flush=None):
    """Median / p10 / p90 milliseconds of single calls, each timed with HIP
    events on the current stream. With `flush` (a 512 MB buffer) the caches,
    MALL included, are overwritten before every call (outside the events)."""
    import numpy as np
    import torch

    stream = torch.cuda.current_stream()
    ts = []
    for _ in range(n):
        if flush is not None:
            flush.fill_(1)  # also keeps the GPU busy while the timed call is queued
        else:
            fn()  # an untimed call in front keeps the timed one from waiting on the host
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        fn()
        e.record(stream)
        e.synchronize()
        ts.append(s.elapsed_time(e))
    q = np.percentile(ts, [50, 10, 90])
    return {"median_ms": round(float(q[0]), 5), "p10_ms": round(float(q[1]), 5), "p90_ms": round(float(q[2]), 5),
            "n": n}


def graph_time(fn, out, calls=10, replays=20, checks=3):
    """Milliseconds per call of `fn` replayed from a HIP graph that holds
    `calls` back-to-back calls, so host-side launch costs drop out (they
    dominate below ~50 us). `out` is the tensor the call writes, or None when
    `fn` returns its result. Every checked replay must give the eager result's
    bits, with eager work and a synchronisation between replays."""
    import torch

    r = fn()
    torch.cuda.synchronize()
    ref = (out if out is not None else r).clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            r = fn()
    res = out if out is not None else r
    same = True
    for _ in range(checks):
        res.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same &= bool(torch.equal(res, ref))
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g.replay()
    s.record()
    for _ in range(replays):
        g.replay()
    e.record()
    e.synchronize()
    del g
    return s.elapsed_time(e) / (calls * replays), same


def dense_torch(x, Wg, WuT, Wd):
    """The dense gated FFN on hipBLASLt through torch (bf16 products, bf16
    hidden): z|u = x [Wg; WuT]^T in one GEMM, h = ReLU(z) * u, y = h Wd."""
    import torch

    F = Wg.shape[0]
    Wgu = torch.cat([Wg, WuT], 0).contiguous()

    def run():
        zu = torch.nn.functional.linear(x, Wgu)
        h = torch.relu(zu[:, :F]) * zu[:, F:]
        return h @ Wd

    return run


def layer_sweep(dev, names, steps, warmup, graphs=False, with_gateup=False):
    """Sparse forward vs the dense baselines on each named layer (and, with
    `with_gateup`, the gate-only variant); with `graphs`, every leg is timed
    by HIP graph replay (graph_time)."""
    import numpy as np
    import torch

    import activation_sparse_ffn_gate_amd as tw
    from synth import WORKLOADS, make_inputs

    out = []
    for name in names:
        w = WORKLOADS[name]
        inp = make_inputs(w)
        x, Wg, WuT, Wd = (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
                          for a in (inp.x, inp.Wg, inp.WuT, inp.Wd))
        y = torch.empty((w.M, w.d), dtype=torch.float32, device=dev)
        ws, ctrl, wsd = tw.Workspace(dev), tw.Workspace(dev, zeroed=True), tw.Workspace(dev)
        stream = torch.cuda.current_stream(dev)
        fwd = lambda: tw.ffn_forward(x, Wg, WuT, Wd, w.T, w.C, y=y, workspace=ws, ctrl=ctrl)  # noqa: E731
        dense = lambda: tw.dense_ffn_forward(x, Wg, WuT, Wd, y=y, workspace=wsd)  # noqa: E731
        dt = dense_torch(x, Wg, WuT, Wd)
        legs = [("sparse", fwd, y), ("dense", dense, y), ("dense_hipblaslt", dt, None)]
        gateup_ok = with_gateup and tw.workspace_bytes(tw.OP_FFN_FORWARD_GATEUP, w.M, w.d, w.F, w.T, w.C) > 0
        if gateup_ok:  # the gate-only variant (dense gate and up products, sparse down)
            wsg = tw.Workspace(dev)
            gu = lambda: tw.ffn_forward_gateup(x, Wg, WuT, Wd, w.T, w.C, y=y, workspace=wsg, ctrl=ctrl)  # noqa: E731
            legs.append(("sparse_gateup", gu, y))
        res, replay_ok = {}, {}
        for key, fn, o in legs:
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            if graphs:
                res[key], replay_ok[key] = graph_time(fn, o, replays=max(2, steps // 10))
            else:
                res[key] = time_loop(fn, steps, stream)
        view = tw.packed_view(w.M, w.d, w.F, w.T, w.C, workspace=ws, device=dev)
        counts = view.counts.cpu().numpy().view(np.uint16).astype(np.int64)
        out.append({
            "workload": name, "M": w.M, "d": w.d, "F": w.F, "T": w.T, "C": w.C,
            "active_pct": round(100.0 * counts.sum() / (w.M * w.F), 3),
            "overflow_rows": int(view.n_ovf.item()),
            "sparse_tokens_per_s": round(w.M / (res["sparse"] * 1e-3), 1),
            "sparse_ms": round(res["sparse"], 5), "dense_ms": round(res["dense"], 5),
            "dense_hipblaslt_ms": round(res["dense_hipblaslt"], 5),
            "speedup_vs_dense": round(res["dense"] / res["sparse"], 3),
            "speedup_vs_dense_hipblaslt": round(res["dense_hipblaslt"] / res["sparse"], 3),
        })
        if gateup_ok:
            out[-1]["gateup_ms"] = round(res["sparse_gateup"], 5)
            out[-1]["gateup_speedup_vs_dense_hipblaslt"] = round(res["dense_hipblaslt"] / res["sparse_gateup"], 3)
            out[-1]["gateup_speedup_vs_sparse"] = round(res["sparse"] / res["sparse_gateup"], 3)
        if graphs:
            out[-1]["timing"] = "hip_graph"
            out[-1]["graph_replays_match_eager"] = replay_ok
        del x, Wg, WuT, Wd, y, ws, ctrl, wsd, dt, view
        torch.cuda.empty_cache()
    return out


def dense_backward_torch(x, Wg, WuT, Wd, dy):
    """The dense gated FFN's backward on hipBLASLt through torch (bf16
    products, fp32 accumulate), from the forward's saved z, u: dH = dy Wd^T,
    dZ = dH u [z > 0], dU = dH ReLU(z), dx = [dZ dU] [Wg; WuT],
    d[Wg; WuT] = [dZ dU]^T x, dWd = h^T dy."""
    import torch

    F = Wg.shape[0]
    Wgu = torch.cat([Wg, WuT], 0).contiguous()
    zu = torch.nn.functional.linear(x, Wgu)
    z, u = zu[:, :F], zu[:, F:]
    h = (torch.relu(z) * u).contiguous()
    mask = (z > 0).to(x.dtype)
    WdT = Wd.t().contiguous()
    xT = x.t().contiguous()
    dyT = dy.t().contiguous()

    def run():
        dH = dy @ WdT
        dZU = torch.cat([dH * u * mask, dH * torch.relu(z)], 1)
        dx = dZU @ Wgu
        dWgu = (dZU.t().contiguous() @ x)
        dWd = (h.t().contiguous() @ dy)
        return dx, dWgu, dWd

    return run


def dense_forward_torch_train(x, Wg, WuT, Wd):
    """The dense gated FFN's training forward on hipBLASLt through torch: z|u
    in one GEMM (kept for the backward), h = ReLU(z) u, y = h Wd."""
    import torch

    F = Wg.shape[0]
    Wgu = torch.cat([Wg, WuT], 0).contiguous()

    def run():
        zu = torch.nn.functional.linear(x, Wgu)
        h = torch.relu(zu[:, :F]) * zu[:, F:]
        return zu, h @ Wd

    return run


def training_backward(dev, name, K, R, steps, warmup):
    """The training path of one layer: the training gate (packing of capacity
    C plus the spill list of tiles over C), the forward's up/down and fallback
    from that packing (y), the hybrid format and the sparse backward; against
    the dense path on hipBLASLt (forward keeping z and u, backward). Also the
    bytes each path keeps for the backward and holds in between."""
    import numpy as np
    import torch

    import activation_sparse_ffn_gate_amd as tw
    from synth import WORKLOADS, make_inputs, make_upstream_grad

    w = WORKLOADS[name]
    inp = make_inputs(w)
    td = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)  # noqa: E731
    x, Wg, WuT, Wd = (td(a) for a in (inp.x, inp.Wg, inp.WuT, inp.Wd))
    dy = td(make_upstream_grad(w))
    stream = torch.cuda.current_stream(dev)
    nT = w.F // w.T
    cap = max(1024, w.M * nT // 16)  # spill records (tiles over C) the list holds
    p, sp = tw.gate_pack_spill(x, Wg, w.T, w.C, cap)
    hy = tw.Hybrid.empty(w.M, w.F, K, R, dev)
    ws, ws_s, ws_f = tw.Workspace(dev), tw.Workspace(dev), tw.Workspace(dev)
    y = torch.empty((w.M, w.d), dtype=torch.float32, device=dev)
    outs = (torch.empty((w.M, w.d), dtype=torch.float32, device=dev),
            *(torch.empty((w.F, w.d), dtype=torch.float32, device=dev) for _ in range(3)))
    sliced_ok = tw.workspace_bytes(tw.OP_SLICED_UPDOWN, w.M, w.d, w.F, w.T, w.C) > 0
    gate = lambda: tw.gate_pack_spill(x, Wg, w.T, w.C, cap, out=p, spill=sp)  # noqa: E731

    def updown():
        if sliced_ok:
            tw.sliced_updown(x, WuT, Wd, p, y=y, workspace=ws_s)
        else:
            tw.fused_updown(x, WuT, Wd, p, y=y)
        tw.dense_fallback(x, Wg, WuT, Wd, p, y, workspace=ws_f)

    pack = lambda: tw.hybrid_pack(p, w.F, K, R, out=hy, spill=sp)  # noqa: E731
    bwd = lambda: tw.ffn_backward(x, Wg, WuT, Wd, dy, hy, workspace=ws, out=outs)  # noqa: E731

    def sparse_step():
        gate()
        updown()
        pack()
        bwd()

    dense_fwd = dense_forward_torch_train(x, Wg, WuT, Wd)
    dense_bwd = dense_backward_torch(x, Wg, WuT, Wd, dy)

    def dense_step():
        dense_fwd()
        dense_bwd()

    # the former route: a C = T packing (every unit in its slots), no spill list
    p_ct = tw.Packed.empty(w.M, w.F, w.T, w.T, dev)
    hy_ct = tw.Hybrid.empty(w.M, w.F, K, R, dev)
    gate_ct = lambda: tw.gate_pack(x, Wg, w.T, w.T, out=p_ct)  # noqa: E731
    pack_ct = lambda: tw.hybrid_pack(p_ct, w.F, K, R, out=hy_ct)  # noqa: E731
    res = {}
    for key, fn in (("gate_spill", gate), ("forward_updown_fallback", updown), ("hybrid_pack", pack),
                    ("sparse_backward", bwd), ("sparse_training_step", sparse_step),
                    ("dense_forward_hipblaslt", dense_fwd), ("dense_backward_hipblaslt", dense_bwd),
                    ("dense_training_step_hipblaslt", dense_step), ("gate_c_eq_t", gate_ct),
                    ("hybrid_pack_c_eq_t", pack_ct)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        res[key] = time_loop(fn, steps, stream)
    sparse_step()
    torch.cuda.synchronize()
    count = hy.count.cpu().numpy()
    flops_dense = 12.0 * w.M * w.d * w.F
    nbytes = lambda *ts: int(sum(t.numel() * t.element_size() for t in ts))  # noqa: E731
    mem = {
        # kept from the forward for the backward (x and the weights are common to both)
        "dense_saved_bytes": w.M * 2 * w.F * 2,  # z and u in bf16
        "sparse_saved_bytes": nbytes(hy.idx, hy.vals, hy.count, hy.res_rows, hy.res_vals, hy.n_res),
        # held between the gate and the hybrid format
        "sparse_packing_and_spill_bytes": nbytes(p.vals, p.idx, p.counts, p.ovf_rows, p.n_ovf, sp.z, sp.slot,
                                                 sp.n_spill),
        "c_eq_t_packing_bytes": nbytes(p_ct.vals, p_ct.idx, p_ct.counts, p_ct.ovf_rows, p_ct.n_ovf),
    }
    mem["sparse_peak_bytes"] = mem["sparse_saved_bytes"] + mem["sparse_packing_and_spill_bytes"]
    mem["sparse_vs_dense_saved"] = round(mem["sparse_saved_bytes"] / mem["dense_saved_bytes"], 4)
    mem["sparse_peak_vs_dense_saved"] = round(mem["sparse_peak_bytes"] / mem["dense_saved_bytes"], 4)
    out = {"workload": name, "M": w.M, "d": w.d, "F": w.F, "T": w.T, "C": w.C, "K": K, "R": R,
           "spill_cap": cap, "spilled_tiles": int(sp.n_spill.item()),
           "reserve_rows": int(hy.n_res.item()), "entries": int(count.sum()),
           "dense_backward_tflops": round(flops_dense / (res["dense_backward_hipblaslt"] * 1e-3) / 1e12, 1),
           "memory": mem}
    out.update({f"{k}_ms": round(v, 5) for k, v in res.items()})
    out["speedup_backward_vs_dense"] = round(res["dense_backward_hipblaslt"] / res["sparse_backward"], 3)
    out["speedup_training_step_vs_dense"] = round(res["dense_training_step_hipblaslt"] / res["sparse_training_step"], 3)
    del x, Wg, WuT, Wd, dy, p, sp, hy, ws, ws_s, ws_f, outs, y, dense_fwd, dense_bwd, p_ct, hy_ct
    torch.cuda.empty_cache()
    return out


def dead_unit_compaction(dev, name, steps, warmup):
    """The layer with its never-active units dropped (activity taken over the
    layer's own batch), against the full layer: forward and gate times, the
    compacted width, and how far the two outputs are apart."""
    import numpy as np
    import torch

    import activation_sparse_ffn_gate_amd as tw
    from synth import WORKLOADS, make_inputs

    w = WORKLOADS[name]
    inp = make_inputs(w)
    x, Wg, WuT, Wd = (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
                      for a in (inp.x, inp.Wg, inp.WuT, inp.Wd))
    stream = torch.cuda.current_stream(dev)
    bits = tw.column_activity(x, Wg, w.T, w.C)
    t0 = time.perf_counter()
    Wg_c, WuT_c, Wd_c, src = tw.compact_layer(Wg, WuT, Wd, bits, w.T)
    torch.cuda.synchronize()
    t_compact = time.perf_counter() - t0
    Fc = Wg_c.shape[0]
    live = int((src >= 0).sum().item())
    y = torch.empty((w.M, w.d), dtype=torch.float32, device=dev)
    y_c = torch.empty_like(y)
    ws, ws_c = tw.Workspace(dev), tw.Workspace(dev)
    p, p_c = tw.Packed.empty(w.M, w.F, w.T, w.C, dev), tw.Packed.empty(w.M, Fc, w.T, w.C, dev)
    legs = {
        "forward": lambda: tw.ffn_forward(x, Wg, WuT, Wd, w.T, w.C, y=y, workspace=ws),
        "forward_compacted": lambda: tw.ffn_forward(x, Wg_c, WuT_c, Wd_c, w.T, w.C, y=y_c, workspace=ws_c),
        "gate": lambda: tw.gate_pack(x, Wg, w.T, w.C, out=p),
        "gate_compacted": lambda: tw.gate_pack(x, Wg_c, w.T, w.C, out=p_c),
    }
    res = {}
    for key, fn in legs.items():
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        res[key] = time_loop(fn, steps, stream)
    legs["forward"]()
    legs["forward_compacted"]()
    torch.cuda.synchronize()
    diff = float((y_c - y).norm() / y.norm())
    out = {"workload": name, "F": w.F, "live_units": live, "F_compacted": Fc,
           "dead_units_by_construction": int(inp.info["dead"].sum()) if "dead" in inp.info else None,
           "compaction_s": round(t_compact, 4), "rel_l2_full_vs_compacted": diff}
    out.update({f"{k}_ms": round(v, 5) for k, v in res.items()})
    out["forward_speedup"] = round(res["forward"] / res["forward_compacted"], 3)
    out["gate_speedup"] = round(res["gate"] / res["gate_compacted"], 3)
    del x, Wg, WuT, Wd, Wg_c, WuT_c, Wd_c, y, y_c, ws, ws_c, p, p_c
    torch.cuda.empty_cache()
    return out


def load_traffic(workload):
    """HBM-side bytes per launch recorded from rocprofv3 counters for this
    workload, or {} when the kernel sources changed since they were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return {}
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    if rec.get("sources_sha256") != sources_hash():
        return {}
    return rec.get("workloads", {}).get(workload, {})


def updown_bytes(counts, w):
    """Algorithmic bytes of one up/down pass over a packing (counts [M, F/T]).

    G (gathered): every stored unit of a row that fits reads one WuT and one
    Wd row (4 d bytes); U (distinct): each unit's two rows are read once
    however many rows store it. Both add, per fitting row, x (2 d) and y
    (4 d), and the packing read (2 bytes per count, 5 per stored slot)."""
    nT = w.F // w.T
    fit = counts.max(axis=1) <= w.C
    nnz_fit = int(counts[fit].sum())
    io = float(fit.sum()) * 6.0 * w.d + w.M * 2.0 * nT + nnz_fit * 5.0
    return dict(nnz_fit=nnz_fit, fit_rows=int(fit.sum()), G=nnz_fit * 4.0 * w.d + io, io=io)


def distinct_units(view, w):
    """Units stored by at least one fitting row of a device packing."""
    import torch

    nT = w.F // w.T
    counts = view.counts.view(torch.int16).to(torch.int32) & 0xFFFF
    fit = (counts.max(dim=1).values <= w.C)
    used = torch.arange(w.C, device=counts.device)[None, None, :] < torch.clamp(counts, max=w.C)[:, :, None]
    used &= fit[:, None, None]
    unit = view.idx.to(torch.int64) + (torch.arange(nT, device=counts.device) * w.T)[None, :, None]
    mark = torch.zeros(w.F, dtype=torch.bool, device=counts.device)
    mark[unit[used]] = True
    return int(mark.sum().item())


def gate_events(n):
    """n pairs of timing events for twell_ffn_forward_timed, created (recorded
    once) before any timed region."""
    import torch

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for b, e in ev:
        b.record()
        e.record()
    torch.cuda.synchronize()
    return ev


def gate_in_forward(fwd_timed, steps):
    """Mean time of the gate's launches inside `steps` back-to-back forwards,
    from the event pair each twell_ffn_forward_timed call records around them."""
    import torch

    ev = gate_events(steps)
    for i in range(steps):
        fwd_timed(*ev[i])
    torch.cuda.synchronize()
    return sum(b.elapsed_time(e) for b, e in ev) / steps


def kernel_legs(dev, w, tensors, k_steps, workload, bufs=None):
    """Each component of the forward timed alone with HIP events on its launch
    stream (k_steps back-to-back launches), the dense baselines, and the
    roofline of the slower of the gate and the up/down step. The gate's time
    in the roofline is its time inside the forward: k_steps back-to-back
    forwards (twell_ffn_forward_timed, the forward's kernels) with HIP events
    recorded around the gate's launches in each. They are a loop of their own:
    the two event records between kernels cost about 10 us per forward at
    M = 4096 (0.201 against 0.211 ms a step), so the headline steps carry none."""
    import numpy as np
    import torch

    import activation_sparse_ffn_gate_amd as tw

    x, Wg, WuT, Wd = tensors
    b = bufs or {}

    def buf(key, make):  # the caller's buffer if given, else a new one
        return b[key] if b.get(key) is not None else make()

    y = buf("y", lambda: torch.empty((w.M, w.d), dtype=torch.float32, device=dev))
    ctrl_gate = buf("ctrl_gate", lambda: tw.Workspace(dev, zeroed=True))
    ws_dense = buf("ws_dense", lambda: tw.Workspace(dev))
    packed = buf("packed", lambda: tw.Packed.empty(w.M, w.F, w.T, w.C, dev))
    ws_sliced = buf("ws_sliced", lambda: tw.Workspace(dev))
    stream = torch.cuda.current_stream(dev)
    y_dense = torch.empty_like(y)

    gate = lambda: tw.gate_pack(x, Wg, w.T, w.C, out=packed, ctrl=ctrl_gate)  # noqa: E731
    fused = lambda: tw.fused_updown(x, WuT, Wd, packed, y=y)  # noqa: E731
    sliced_ok = tw.workspace_bytes(tw.OP_SLICED_UPDOWN, w.M, w.d, w.F, w.T, w.C) > 0
    sliced = lambda: tw.sliced_updown(x, WuT, Wd, packed, y=y, workspace=ws_sliced)  # noqa: E731
    fallback = lambda: tw.dense_fallback(x, Wg, WuT, Wd, packed, y, workspace=ws_dense)  # noqa: E731
    dense = lambda: tw.dense_ffn_forward(x, Wg, WuT, Wd, y=y_dense, workspace=ws_dense)  # noqa: E731
    dense_tl = dense_torch(x, Wg, WuT, Wd)

    gate()
    torch.cuda.synchronize()
    counts = packed.counts.cpu().numpy().view(np.uint16).astype(np.int64)
    n_ovf = int(packed.n_ovf.item())
    nnz_all = int(counts.sum())
    ub = updown_bytes(counts, w)
    U = distinct_units(packed, w) * 4.0 * w.d + ub["io"]
    for fn in [gate, fused, fallback, dense, dense_tl] + ([sliced] if sliced_ok else []):
        fn()
    torch.cuda.synchronize()
    t_gate_alone = time_loop(gate, k_steps, stream)
    ws_fwd = buf("ws_fwd", lambda: tw.Workspace(dev))
    ctrl_fwd = buf("ctrl_fwd", lambda: tw.Workspace(dev, zeroed=True))
    for _ in range(3):
        tw.ffn_forward(x, Wg, WuT, Wd, w.T, w.C, y=y, workspace=ws_fwd, ctrl=ctrl_fwd)
    fwd_timed = lambda b, e: tw.ffn_forward_timed(x, Wg, WuT, Wd, w.T, w.C, b, e, y=y,  # noqa: E731
                                                  workspace=ws_fwd, ctrl=ctrl_fwd)
    t_gate, gate_calls = gate_in_forward(fwd_timed, k_steps), k_steps
    t_fused = time_loop(fused, k_steps, stream)
    t_sliced = time_loop(sliced, k_steps, stream) if sliced_ok else None
    t_fb = time_loop(fallback, k_steps, stream)
    t_dense = time_loop(dense, k_steps, stream)
    t_dense_tl = time_loop(dense_tl, k_steps, stream)
    # the up/down form twell_ffn_forward runs above 256 rows
    t_updown = t_sliced if sliced_ok else t_fused
    updown_name = "sliced_updown" if sliced_ok else "fused_updown"

    gate_flops = 2.0 * w.M * w.d * w.F
    gate_tflops = gate_flops / (t_gate * 1e-3) / 1e12
    gbs = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9  # noqa: E731
    traffic = load_traffic(workload)
    hbm = {k: round(v["traffic_bytes"]) for k, v in traffic.items()}

    def hbm_gbs(name, ms):
        return round(gbs(hbm[name], ms), 1) if name in hbm else None

    if t_updown >= t_gate:
        roof = {"kernel": updown_name, "bound": "hbm", "achieved": round(gbs(U, t_updown), 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs(U, t_updown) / PEAK_HBM_GBS, 4),
                "traffic": hbm.get(updown_name), "bytes": "distinct (U)"}
    else:
        roof = {"kernel": "gate_pack", "bound": "mfma", "achieved": round(gate_tflops, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(gate_tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": hbm.get("gate_pack")}
    legs = {
        "gate_pack_ms": round(t_gate, 5),
        "gate_pack_timing": f"inside the forward: HIP events around the gate's launches in {gate_calls} forward calls",
        "gate_pack_alone_ms": round(t_gate_alone, 5),
        "gate_pack_tflops": round(gate_tflops, 1),
        "gate_pack_mfma_frac": round(gate_tflops / PEAK_BF16_TFLOPS, 4),
        "gate_pack_hbm_bytes": hbm.get("gate_pack"),
        "fused_updown_ms": round(t_fused, 5),
        "sliced_updown_ms": round(t_sliced, 5) if sliced_ok else None,
        "forward_updown": updown_name,
        "updown_gathered_bytes": round(ub["G"]),
        "updown_distinct_bytes": round(U),
        "fused_updown_gathered_gbs": round(gbs(ub["G"], t_fused), 1),
        "fused_updown_distinct_gbs": round(gbs(U, t_fused), 1),
        "fused_updown_distinct_hbm_frac": round(gbs(U, t_fused) / PEAK_HBM_GBS, 4),
        "fused_updown_hbm_bytes": hbm.get("fused_updown"),
        "fused_updown_counter_gbs": hbm_gbs("fused_updown", t_fused),
        "dense_fallback_ms": round(t_fb, 5),
        "nnz_per_token": round(nnz_all / w.M, 3),
        "overflow_rows": n_ovf,
        "traffic_current": bool(traffic),
    }
    if sliced_ok:
        legs.update({
            "sliced_updown_gathered_gbs": round(gbs(ub["G"], t_sliced), 1),
            "sliced_updown_distinct_gbs": round(gbs(U, t_sliced), 1),
            "sliced_updown_distinct_hbm_frac": round(gbs(U, t_sliced) / PEAK_HBM_GBS, 4),
            "sliced_updown_hbm_bytes": hbm.get("sliced_updown"),
            "sliced_updown_counter_gbs": hbm_gbs("sliced_updown", t_sliced),
        })
    legs["roofline"] = roof
    legs["dense_baseline"] = {
        "ms": round(t_dense, 5),
        "tokens_per_s": round(w.M / (t_dense * 1e-3), 1),
        "tflops": round(3 * gate_flops / (t_dense * 1e-3) / 1e12, 1),
        "hipblaslt_ms": round(t_dense_tl, 5),
        "hipblaslt_tflops": round(3 * gate_flops / (t_dense_tl * 1e-3) / 1e12, 1),
    }
    return legs


def layer_report(dev, name, k_steps, warmup):
    """Forward throughput of another full-size layer with its kernel legs."""
    import numpy as np
    import torch

    import activation_sparse_ffn_gate_amd as tw
    from synth import WORKLOADS, make_inputs

    w = WORKLOADS[name]
    inp = make_inputs(w)
    x, Wg, WuT, Wd = (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
                      for a in (inp.x, inp.Wg, inp.WuT, inp.Wd))
    y = torch.empty((w.M, w.d), dtype=torch.float32, device=dev)
    ws, ctrl = tw.Workspace(dev), tw.Workspace(dev, zeroed=True)
    stream = torch.cuda.current_stream(dev)
    fwd = lambda: tw.ffn_forward(x, Wg, WuT, Wd, w.T, w.C, y=y, workspace=ws, ctrl=ctrl)  # noqa: E731
    for _ in range(warmup):
        fwd()
    torch.cuda.synchronize()
    t_fwd = time_loop(fwd, k_steps, stream)
    legs = kernel_legs(dev, w, (x, Wg, WuT, Wd), k_steps, name)
    out = {"workload": name, "M": w.M, "d": w.d, "F": w.F, "T": w.T, "C": w.C,
           "forward_ms": round(t_fwd, 5), "tokens_per_s": round(w.M / (t_fwd * 1e-3), 1),
           "roofline": legs.pop("roofline")}
    dense = legs.pop("dense_baseline")
    dense["speedup_sparse_vs_dense"] = round(dense["ms"] / t_fwd, 3)
    dense["speedup_sparse_vs_hipblaslt"] = round(dense["hipblaslt_ms"] / t_fwd, 3)
    out["kernels"] = legs
    out["dense_baseline"] = dense
    del x, Wg, WuT, Wd, y, ws, ctrl
    torch.cuda.empty_cache()
    return out


def cpu_baseline(inp, budget_s):
    """The oracle, as it stands, on a bounded sample of the same layer's rows."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle as O

    w = inp.workload
    chunk = 128
    rows_done = 0
    t0 = time.perf_counter()
    while rows_done < w.M and time.perf_counter() - t0 < budget_s:
        rows = np.arange(rows_done, min(rows_done + chunk, w.M))
        Z = O.gate_preactivations(inp.x, inp.Wg, rows=rows)
        p = O.pack_twell(Z.astype(np.float32), w.T, w.C)
        O.dense_gated_ffn(inp.x, inp.Wg, inp.WuT, inp.Wd, rows=rows)
        O.ffn_from_twell(p, inp.x[rows], inp.Wg, inp.WuT, inp.Wd)
        rows_done += len(rows)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {
        "value": round(rows_done / dt, 2),
        "unit": "tokens/s",
        "cores": int(threads),
        "cpu_model": cpu_model,
        "kind": "oracle",
        "sample": f"first {rows_done} of {w.M} tokens of {w.name}: fp64 gate, TwELL pack, "
                  f"fp64 dense FFN and sparse FFN from the packing ({dt:.1f} s)",
    }


def main():
    args = parse()
    if args.record_traffic:
        record_traffic(args.record_traffic, args.workload)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the forward shards by tokens with no communication)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import activation_sparse_ffn_gate_amd as tw
    from synth import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    inp = make_inputs(w)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def td(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    x, Wg, WuT, Wd = (td(a) for a in (inp.x, inp.Wg, inp.WuT, inp.Wd))
    if args.compact:  # the layer without its never-active units (activity over its own batch)
        if args.only is None:
            print("--compact is for --only runs (the default run reports it in dead_unit_compaction)",
                  file=sys.stderr)
            return 2
        bits = tw.column_activity(x, Wg, w.T, w.C)
        Wg, WuT, Wd, _ = tw.compact_layer(Wg, WuT, Wd, bits, w.T)
        w = dataclasses.replace(w, F=Wg.shape[0])
    y = torch.empty((w.M, w.d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    ws_fwd = tw.Workspace(dev)
    ctrl_fwd = tw.Workspace(dev, zeroed=True)
    ctrl_gate = tw.Workspace(dev, zeroed=True)
    ws_dense = tw.Workspace(dev)
    packed = tw.Packed.empty(w.M, w.F, w.T, w.C, dev)

    fwd = lambda: tw.ffn_forward(x, Wg, WuT, Wd, w.T, w.C, y=y, workspace=ws_fwd, ctrl=ctrl_fwd)  # noqa: E731
    gate = lambda: tw.gate_pack(x, Wg, w.T, w.C, out=packed, ctrl=ctrl_gate)  # noqa: E731
    fused = lambda: tw.fused_updown(x, WuT, Wd, packed, y=y)  # noqa: E731
    ws_sliced = tw.Workspace(dev)
    sliced_ok = tw.workspace_bytes(tw.OP_SLICED_UPDOWN, w.M, w.d, w.F, w.T, w.C) > 0
    sliced = lambda: tw.sliced_updown(x, WuT, Wd, packed, y=y, workspace=ws_sliced)  # noqa: E731
    fallback = lambda: tw.dense_fallback(x, Wg, WuT, Wd, packed, y, workspace=ws_dense)  # noqa: E731
    y_dense = torch.empty_like(y)
    dense = lambda: tw.dense_ffn_forward(x, Wg, WuT, Wd, y=y_dense, workspace=ws_dense)  # noqa: E731

    if args.only == "backward":  # hybrid pack once, then the timed sparse backward
        from synth import make_upstream_grad

        dy = td(make_upstream_grad(w))
        p_tr, sp_tr = tw.gate_pack_spill(x, Wg, w.T, w.C, max(1024, w.M * (w.F // w.T) // 16))
        hy = tw.hybrid_pack(p_tr, w.F, 64, min(512, w.M), spill=sp_tr)
        ws_b = tw.Workspace(dev)
        outs = (torch.empty((w.M, w.d), dtype=torch.float32, device=dev),
                *(torch.empty((w.F, w.d), dtype=torch.float32, device=dev) for _ in range(3)))
        fn = lambda: tw.ffn_backward(x, Wg, WuT, Wd, dy, hy, workspace=ws_b, out=outs)  # noqa: E731
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ms = time_loop(fn, args.steps, stream)
        print(json.dumps({"only": args.only, "ms_per_call": round(ms, 5), "steps": args.steps}))
        return 0
    if args.only is not None:
        if args.only == "copy":
            n = args.copy_mb * (1 << 20) // 4
            # a plain elementwise kernel of known traffic: reads and writes n floats
            src = torch.ones(n, dtype=torch.float32, device=dev)
            dst = torch.empty_like(src)
            fn = lambda: torch.mul(src, 2.0, out=dst)  # noqa: E731
        else:
            ws_gu = tw.Workspace(dev)
            gateup = lambda: tw.ffn_forward_gateup(x, Wg, WuT, Wd, w.T, w.C, y=y, workspace=ws_gu)  # noqa: E731
            fn = {"forward": fwd, "gate": gate, "fused": fused, "sliced": sliced, "dense": dense,
                  "fallback": fallback, "gateup": gateup}[args.only]
            gate()  # the fused leg reads a packing
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ms = time_loop(fn, args.steps, stream)
        print(json.dumps({"only": args.only, "ms_per_call": round(ms, 5), "steps": args.steps}))
        return 0

    # ------------------------------------------------- per-kernel (HIP events)
    # First, so the GPU has been under load for a second or so when the
    # headline's warm-up starts: after the idle time of input generation the
    # first ~10 ms of forwards run about 8% slower (0.2175 against 0.2006 ms a
    # step over 50 forwards, measured) while the clocks come up.
    k_steps = max(args.steps, 20)
    legs = kernel_legs(dev, w, (x, Wg, WuT, Wd), k_steps, args.workload,
                       bufs=dict(y=y, ws_fwd=ws_fwd, ctrl_fwd=ctrl_fwd, ctrl_gate=ctrl_gate, ws_dense=ws_dense,
                                 packed=packed, ws_sliced=ws_sliced))

    # ---------------------------------------------------------------- headline
    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fwd()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    value = w.M * args.steps / elapsed
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    lat = {"warm": latency(fwd, 20), "cold": latency(fwd, 20, flush=flush)}
    del flush
    roof = legs.pop("roofline")
    dense = legs.pop("dense_baseline")
    dense["speedup_sparse_vs_dense"] = round(dense["ms"] / ms_step, 3)
    dense["speedup_sparse_vs_hipblaslt"] = round(dense["hipblaslt_ms"] / ms_step, 3)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "d": w.d, "F": w.F, "T": w.T, "C": w.C,
                   "mean_nnz_target": round(w.mean_nnz, 3), "parallelism": "none"},
        "roofline": roof,
        "kernels": legs,
        "latency_forward": lat,
        "dense_baseline": dense,
    }
    del x, Wg, WuT, Wd, y, ws_fwd, ctrl_fwd, ctrl_gate, ws_dense, packed, ws_sliced
    torch.cuda.empty_cache()
    if not args.no_layers:  # the other full-size layers: heavy-tailed 1.5B-like and 2B-like
        out["layers"] = [layer_report(dev, n, k_steps, args.warmup)
                         for n in ("ffn1p5b_heavytail", "ffn2b_zipf") if n != args.workload]
    if not args.no_sweep:  # HBM holds both layers' buffers easily
        from synth import WORKLOADS as _W

        sweep = sorted((k for k in _W if k.startswith("sweep_")), key=lambda k: _W[k].mean_nnz)
        out["density_sweep"] = layer_sweep(dev, sweep, args.sweep_steps, 2, with_gateup=True)
        decode = sorted((k for k in _W if k.startswith("decode_")), key=lambda k: _W[k].M)
        out["decode_batches"] = layer_sweep(dev, decode, 4 * args.sweep_steps, 4, graphs=True)
        out["dead_unit_compaction"] = dead_unit_compaction(dev, "ffn1p5b_heavytail", 2 * args.sweep_steps, 3)
        out["training_backward"] = [training_backward(dev, n, 64, 512, 2 * args.sweep_steps, 2)
                                    for n in ("ffn1p5b", "ffn1p5b_heavytail")]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
