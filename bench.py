"""Throughput of the ring-step attention hot path on one MI355X.

A step is one pass of the Llama-2-7B-shaped long-context forward: Q, K, V
[1, 32768, 32, 128] bf16 (i.i.d. N(0,1), seed 0), the key/value sequence streamed
as 8 ring-step chunks of 4096 in a seeded random order, every step merging its
partial (O, LSE) pair into the running pair, the last one also storing the
final bf16 output.  Inputs are resident in HBM before timing starts.

Prints ONE JSON line: attention TFLOP/s (algorithmic flops: 4*D per allowed
causal (query, key) pair), the dominant kernel's roofline fraction against the
dense bf16 MFMA peak, and the CPU oracle timed on a bounded sample of the same
workload.  Other workloads: --workload <name> (see workloads/configs.py).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 dense bf16 flop/clk x 2.4 GHz
PEAK_BASIS = "256 CUs x 4096 bf16 flop/clk (dense MFMA) x 2.4 GHz peak engine clock; HBM 8 TB/s"
PEAK_HBM_GBS = 8000.0
METRIC = "causal attention fwd/bwd TFLOP/s and % bf16 MFMA peak at S=32K-128K, D=128"
PROFILE_DIR = os.path.join(ROOT, "profiles")
FWD_SRC = os.path.join(ROOT, "long_context_exact_blockattn_amd", "csrc", "ba_fwd.h")


def _src_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic(kernel_key, src_path, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on this
    workload and the kernel source has not changed since."""
    path = os.path.join(PROFILE_DIR, f"{kernel_key}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != _src_sha(src_path):
        return None
    if rec.get("workload", "").split(" ")[0] != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def run_ring_forward(w, steps, warmup):
    import torch

    import long_context_exact_blockattn_amd as ba
    from long_context_exact_blockattn_amd import _lib
    from workloads import chunk_bounds, chunk_order, make_inputs

    dev = torch.device("cuda:0")
    q, k, v = make_inputs(w.batch, w.seqlen, w.heads_q, w.heads_kv, w.head_dim, seed=w.seed)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    order = chunk_order(w.n_chunks, seed=w.seed)
    bounds = chunk_bounds(w.seqlen, w.n_chunks)
    b, s, hq, d = q.shape
    o_acc = torch.empty(b, s, hq, d, device=dev, dtype=torch.float32)
    lse = torch.empty(b, hq, s, device=dev, dtype=torch.float32)
    out = torch.empty(b, s, hq, d, device=dev, dtype=torch.bfloat16)
    n = len(order)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(steps)]

    def step(events=None):
        for t, c in enumerate(order):
            c0, c1 = bounds[c]
            if events is not None:
                events[t].record()
            _lib.blockattn_fwd(q, k[:, c0:c1], v[:, c0:c1], o_acc, lse,
                               mode=_lib.BA_OVERWRITE if t == 0 else _lib.BA_ACCUMULATE,
                               o_final=out if t == n - 1 else None, k_pos0=c0)
        if events is not None:
            events[n].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [ev[i][t].elapsed_time(ev[i][t + 1]) for i in range(steps) for t in range(n)]
    step_ms = [ev[i][0].elapsed_time(ev[i][n]) for i in range(steps)]
    assert not torch.isnan(out).any(), "NaN in output"
    return {"wall_s": wall, "launch_ms": launch_ms, "step_ms": step_ms, "launches_per_step": n, "order": order,
            "kernel": f"fwd_kernel<{w.head_dim}>", "src": FWD_SRC,
            "tensors": (q, k, v, o_acc, lse, out)}


def _stats(xs):
    import statistics
    return {"median": round(statistics.median(xs), 4), "min": round(min(xs), 4), "max": round(max(xs), 4)}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return None


def _event_ms(fn, reps):
    """Average milliseconds of fn() over reps calls on the current stream (after one warm call)."""
    import torch
    fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def side_measurements(w, tensors, reps=5):
    """Measured after the timed region, on the same inputs:
    - the forward as ONE chunk (S keys in one call), to show what the ring split costs;
    - the HBM-bound kernels of the path at this shape, as algorithmic bytes / time against 8 TB/s:
      lse_merge (fp32 O_acc read+written, fp32 partial read, three LSE rows) and the backward's
      delta preprocess (dO and O read in bf16, delta written); the dQ finalise is fused into the
      last ring step's dq kernel and has no time of its own."""
    import torch

    from long_context_exact_blockattn_amd import _lib
    q, k, v, o_acc, lse, out = tensors
    b, s, hq, d = q.shape
    elems, rows = b * s * hq * d, b * s * hq

    def one_shot():
        _lib.blockattn_fwd(q, k, v, o_acc, lse, mode=_lib.BA_OVERWRITE, o_final=out)
    ms1 = _event_ms(one_shot, reps)
    res = {"one_shot": {"ms": round(ms1, 4), "tflops": round(w.fwd_flop() / ms1 / 1e9, 2)}}

    # a finite partial, so that both operands of every row are read (a -inf partial is skipped)
    o_part = o_acc.clone()
    lse_part = lse.clone()

    def merge():
        _lib.lse_merge(o_acc, lse, o_part, lse_part)
    ms_m = _event_ms(merge, reps)
    bytes_m = elems * (4 + 4 + 4) + rows * 4 * 3
    delta = torch.empty_like(lse)
    k0 = k[:, :0]

    def delta_only():
        _lib.blockattn_bwd(q, k0, k0, out, out, lse, delta, o_acc, k0, k0, flags=_lib.BA_BWD_COMPUTE_DELTA)
    ms_d = _event_ms(delta_only, reps)
    bytes_d = elems * (2 + 2) + rows * 4
    # Ulysses layout permutes at one device's share of this workload on 8 devices (S/8 rows, all
    # heads; fewer devices when the heads do not split 8 ways): every element read once and
    # written once
    n_dev = max(n for n in range(1, 9) if w.heads_q % n == 0)
    x_share = q[:, : s // n_dev].contiguous()
    send = _lib.ulysses_pack(x_share, n_dev)
    ms_pack = _event_ms(lambda: _lib.ulysses_pack(x_share, n_dev, send=send), reps * 4)
    ms_unpack = _event_ms(lambda: _lib.ulysses_unpack(send, n_dev, x=x_share), reps * 4)
    bytes_u = 2 * x_share.numel() * x_share.element_size()
    hbm = {}
    for name, ms, by in (("lse_merge", ms_m, bytes_m), ("bwd_delta", ms_d, bytes_d),
                         ("ulysses_pack", ms_pack, bytes_u), ("ulysses_unpack", ms_unpack, bytes_u)):
        gbs = by / (ms * 1e-3) / 1e9
        hbm[name] = {"bytes": by, "ms": round(ms, 4), "GB/s": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)}
        if name.startswith("ulysses"):
            hbm[name]["n_devices"] = n_dev
    res["hbm_kernels"] = hbm

    # the ring's receive side: each step's chunk copied into one of two staging buffers on a
    # second stream while the previous step computes, against the plain ring on resident chunks
    if w.n_chunks > 1:
        import long_context_exact_blockattn_amd as ba
        from workloads import chunk_order
        order = chunk_order(w.n_chunks, seed=w.seed)
        ms_plain = _event_ms(lambda: ba.ring_forward(q, k, v, w.n_chunks, order, o_acc=o_acc, lse=lse, out=out),
                             reps)
        ms_staged = _event_ms(lambda: ba.ring_forward_staged(q, k, v, w.n_chunks, order), reps)
        kb = torch.empty_like(k)
        vb = torch.empty_like(v)

        def copies():
            kb.copy_(k)
            vb.copy_(v)
        ms_copy = _event_ms(copies, reps)
        chunk_bytes = 2 * k.numel() * k.element_size() // w.n_chunks
        res["ring_staged"] = {"plain_ms": round(ms_plain, 4), "staged_ms": round(ms_staged, 4),
                              "overhead_pct": round(100 * (ms_staged / ms_plain - 1), 2),
                              "copy_bytes_per_step": chunk_bytes,
                              "copy_alone_ms_per_step": round(ms_copy / w.n_chunks, 4)}
    return res


def run_training(w, steps, warmup):
    """Ring forward + ring backward (training step of attention), or S2 forward + backward."""
    import torch

    import long_context_exact_blockattn_amd as ba
    from long_context_exact_blockattn_amd import _lib
    from workloads import chunk_bounds, chunk_order, make_inputs

    dev = torch.device("cuda:0")
    q, k, v, do = make_inputs(w.batch, w.seqlen, w.heads_q, w.heads_kv, w.head_dim, seed=w.seed, with_dout=True)
    q, k, v, do = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    b, s, hq, d = q.shape
    if w.s2_group is not None:
        o = torch.empty(b, s, hq, d, device=dev, dtype=torch.bfloat16)
        lse = torch.empty(b, hq, s, device=dev)
        delta = torch.empty(b, hq, s, device=dev)
        dq_acc = torch.empty(b, s, hq, d, device=dev)
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dv = torch.empty_like(v)

        def fwd():
            _lib.s2attn_fwd(q, k, v, o, lse, group=w.s2_group, shift_head0=w.s2_shift_head0)

        def bwd():
            dq_acc.zero_()
            _lib.s2attn_bwd(q, k, v, o, do, lse, delta, dq_acc, dk, dv, group=w.s2_group,
                            shift_head0=w.s2_shift_head0, dq_final=dq,
                            flags=_lib.BA_BWD_COMPUTE_DELTA | _lib.BA_BWD_FINALIZE_DQ)
        order = None
    else:
        order = chunk_order(w.n_chunks, seed=w.seed)
        bounds = chunk_bounds(w.seqlen, w.n_chunks)
        o_acc = torch.empty(b, s, hq, d, device=dev)
        lse = torch.empty(b, hq, s, device=dev)
        o = torch.empty(b, s, hq, d, device=dev, dtype=torch.bfloat16)
        delta = torch.empty(b, hq, s, device=dev)
        dq_acc = torch.empty(b, s, hq, d, device=dev)
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dv = torch.empty_like(v)
        n = len(order)

        def fwd():
            for t, c in enumerate(order):
                c0, c1 = bounds[c]
                _lib.blockattn_fwd(q, k[:, c0:c1], v[:, c0:c1], o_acc, lse,
                                   mode=_lib.BA_OVERWRITE if t == 0 else _lib.BA_ACCUMULATE,
                                   o_final=o if t == n - 1 else None, k_pos0=c0)

        def bwd():
            dq_acc.zero_()
            for t, c in enumerate(order):
                c0, c1 = bounds[c]
                flags = (_lib.BA_BWD_COMPUTE_DELTA if t == 0 else 0) | (_lib.BA_BWD_FINALIZE_DQ if t == n - 1 else 0)
                _lib.blockattn_bwd(q, k[:, c0:c1], v[:, c0:c1], o, do, lse, delta, dq_acc,
                                   dk[:, c0:c1], dv[:, c0:c1], dq_final=dq, flags=flags, k_pos0=c0)

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for _ in range(warmup):
        fwd(); bwd()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in ev:
        e[0].record(); fwd(); e[1].record(); bwd(); e[2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = [e[0].elapsed_time(e[1]) for e in ev]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in ev]
    assert not torch.isnan(dq).any() and not torch.isnan(dk).any(), "NaN in gradients"
    return {"wall_s": wall, "fwd_ms": fwd_ms, "bwd_ms": bwd_ms, "order": order}


def cpu_baseline(w, budget_heads=2, budget_flop=6e11, rows_budget_flop=1.5e11):
    """The oracle as it stands, timed on a bounded sample of the same workload: the first query
    heads with all ring steps (about 12 s of host work at the 32K headline shape; short sequences
    in full), or, where two whole heads exceed the budget, the last query rows of head 0 (the rows
    with the most allowed keys) against the whole sequence, in blocks of rows."""
    import numpy as np

    from oracle import ring_attention_forward, rows_forward
    from workloads import chunk_order, make_inputs

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    print(f"timing the oracle on the host ({w.name}) ...", file=sys.stderr, flush=True)
    q, k, v = make_inputs(w.batch, w.seqlen, w.heads_q, w.heads_kv, w.head_dim, seed=w.seed)
    heads = list(range(w.heads_q if w.seqlen <= 4096 else min(budget_heads, w.heads_q)))
    flop = w.fwd_flop() * len(heads) / w.heads_q
    if flop <= budget_flop:
        kv_heads = sorted({h // (w.heads_q // w.heads_kv) for h in heads})
        qn = q[:, :, heads].float().numpy().astype(np.float64)
        kn = k[:, :, kv_heads].float().numpy().astype(np.float64)
        vn = v[:, :, kv_heads].float().numpy().astype(np.float64)
        order = chunk_order(w.n_chunks, seed=w.seed)
        t0 = time.perf_counter()
        ring_attention_forward(qn, kn, vn, order, w.chunk_len)
        dt = time.perf_counter() - t0
        sample = (f"{w.name}: query heads 0-{len(heads) - 1} of {w.heads_q} at full S={w.seqlen}, all "
                  f"{w.n_chunks} ring steps in the seeded order, numpy float64")
    else:
        # causal: row i has i + 1 allowed keys; take rows from the end while the budget lasts
        S, per_key = w.seqlen, 4 * w.head_dim
        n, flop = 0, 0
        while n < S and flop + per_key * (S - n) <= rows_budget_flop:
            flop += per_key * (S - n)
            n += 1
        qn = q[:, :, :1].float().numpy()
        kn = k[:, :, :1].float().numpy()
        vn = v[:, :, :1].float().numpy()
        t0 = time.perf_counter()
        for r0 in range(S - n, S, 256):
            rows_forward(qn, kn, vn, 0, 0, range(r0, min(r0 + 256, S)))
        dt = time.perf_counter() - t0
        sample = (f"{w.name}: the last {n} query rows of head 0 of {w.heads_q} against all S={w.seqlen} keys "
                  f"(a row's result is the same for any chunk order), numpy float64 in blocks of 256 rows")
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{sample}; {dt:.1f} s for {flop:.3e} algorithmic flop",
            "seconds": round(dt, 3),
            "extrapolated_full_config_s": round(dt * w.fwd_flop() / flop, 1),
            "cpu_model": _cpu_model(), "os_cpu_count": os.cpu_count()}


def copy_calibration(reps):
    """A plain copy kernel of known size: reads and writes exactly 1 GiB per launch."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(max(reps, 1)):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": max(reps, 1)}), flush=True)


def _result_dbs(d):
    import glob
    dbs = sorted(glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True))
    if not dbs:
        sys.exit(f"no rocprofv3 *_results.db under {d}")
    return dbs


def trace_summary(d):
    """Per-kernel calls, average duration and launch shape from a rocprofv3 --kernel-trace database."""
    import sqlite3
    agg = {}
    for db in _result_dbs(d):
        con = sqlite3.connect(db)
        q = ("select name, duration, grid_x, workgroup_x, vgpr_count, accum_vgpr_count, scratch_size, "
             "lds_size from kernels")
        for name, dur, gx, wx, vg, ag, sc, lds in con.execute(q):
            a = agg.setdefault(name, [0, 0.0, gx, wx, vg, ag, sc, lds])
            a[0] += 1
            a[1] += dur
    for name, a in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        print(f"{a[0]:6d} calls avg {a[1] / a[0] / 1e3:10.3f} us  grid {a[2]} wg {a[3]} vgpr {a[4]} agpr {a[5]} "
              f"scratch {a[6]} lds {a[7]}  {name[:100]}")


def _counter_per_dispatch(d, counter, kernel_substr):
    """Sum of one counter per dispatch of the kernels whose name contains kernel_substr."""
    import sqlite3
    per = {}
    for db in _result_dbs(d):
        con = sqlite3.connect(db)
        q = "select dispatch_id, kernel_name, value from counters_collection where counter_name = ?"
        for disp, name, val in con.execute(q, (counter,)):
            if kernel_substr in name:
                per[(db, disp)] = per.get((db, disp), 0.0) + val
    return [per[k] for k in sorted(per)]


COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_LDS "
            "SQ_WAIT_ANY SQ_WAVE_CYCLES GRBM_GUI_ACTIVE")


def _counters(kernel_key, src_path, workload):
    """MFMA-busy / VALU-busy of the committed counter summary, if it was taken on this workload and
    the kernel source has not changed since."""
    path = os.path.join(PROFILE_DIR, f"{kernel_key}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != _src_sha(src_path) or rec.get("workload") != workload:
        return None
    return {k: rec[k] for k in ("mfma_busy", "valu_busy_est", "valu_per_mfma", "trans_per_mfma",
                                "lds_per_mfma", "wave_waiting")}


def counter_summary(d, out=None, kernel=None):
    """MFMA-busy beside VALU-busy for one kernel (default: the D=128 forward), from one rocprofv3
    --pmc pass with COUNTERS; the summary record is written for the forward only.

    Per dispatch: cycles = GRBM_GUI_ACTIVE / 8 (the counter sums the 8 XCDs); MFMA busy =
    SQ_VALU_MFMA_BUSY_CYCLES (32 per MFMA, summed over SIMDs) / (1024 SIMDs x cycles); VALU busy is
    estimated from instruction counts at the SIMD issue rates measured on this part (a non-MFMA
    VALU instruction occupies the SIMD 2 cycles, a transcendental ~6.2); waiting = SQ_WAIT_ANY /
    SQ_WAVE_CYCLES."""
    import sqlite3
    per = {}
    for db in _result_dbs(d):
        con = sqlite3.connect(db)
        q = "select dispatch_id, kernel_name, counter_name, value from counters_collection"
        for disp, name, cname, val in con.execute(q):
            if (kernel or "fwd_kernel<128>") in name:
                rec = per.setdefault((db, disp), {})
                rec[cname] = rec.get(cname, 0.0) + val
    rows = []
    for key in sorted(per):
        c = per[key]
        cyc = c["GRBM_GUI_ACTIVE"] / 8.0
        valu = c["SQ_INSTS_VALU"] - c["SQ_INSTS_MFMA"]
        rows.append({
            "mfma_busy": c["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * cyc),
            "valu_busy_est": (2.0 * valu + 4.2 * c["SQ_INSTS_VALU_TRANS_F32"]) / (1024 * cyc),
            "valu_per_mfma": valu / c["SQ_INSTS_MFMA"],
            "trans_per_mfma": c["SQ_INSTS_VALU_TRANS_F32"] / c["SQ_INSTS_MFMA"],
            "lds_per_mfma": c["SQ_INSTS_LDS"] / c["SQ_INSTS_MFMA"],
            "wave_waiting": c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"],
            "mfma": c["SQ_INSTS_MFMA"],
        })
    tot = sum(r["mfma"] for r in rows)
    keys = ("mfma_busy", "valu_busy_est", "valu_per_mfma", "trans_per_mfma", "lds_per_mfma", "wave_waiting")
    avg = {k: sum(r[k] * r["mfma"] for r in rows) / tot for k in keys}
    print(f"{len(rows)} dispatches of {kernel or 'fwd_kernel<128>'}; MFMA-weighted averages:")
    for k in keys:
        print(f"  {k:15s} {avg[k]:8.3f}")
    if out and kernel is None:
        rec = {"kernel": "ba::fwd_kernel<128>", "workload": "llama2_7b_s32k_ring8",
               "kernel_source_sha": _src_sha(FWD_SRC), "dispatches": len(rows),
               "command": f"rocprofv3 --pmc {COUNTERS} -d {d} -o busy -- python -u bench.py --steps 1 "
                          "--warmup 0 --no-cpu-baseline --no-side-measurements",
               **{k: round(v, 4) for k, v in avg.items()}}
        with open(out, "w") as f:
            json.dump(rec, f, indent=1)


def traffic_summary(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, out):
    """HBM bytes per forward launch from FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch), each scaled
    by what the same counter reads for a plain copy of 1 GiB; written to the traffic summary that
    bench.py reports while the kernel source is unchanged."""
    kern = "fwd_kernel<128>"
    fetch = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", kern)
    write = _counter_per_dispatch(write_dir, "WRITE_SIZE", kern)
    cf = _counter_per_dispatch(copy_fetch_dir, "FETCH_SIZE", "")
    cw = _counter_per_dispatch(copy_write_dir, "WRITE_SIZE", "")
    n = 1 << 30
    # the copy launches dominate the calibration runs; take the largest dispatch (the 1 GiB copy)
    fscale = n / 1024.0 / max(cf)
    wscale = n / 1024.0 / max(cw)
    fb = sum(fetch) / len(fetch) * 1024 * fscale
    wb = sum(write) / len(write) * 1024 * wscale
    rec = {
        "kernel": "ba::fwd_kernel<128>",
        "workload": "llama2_7b_s32k_ring8 (8 ring steps, one dispatch each)",
        "kernel_source_sha": _src_sha(FWD_SRC),
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE -d {fetch_dir} -o fetch -- python -u bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-side-measurements",
            f"rocprofv3 --pmc WRITE_SIZE -d {write_dir} -o write -- python -u bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-side-measurements",
            f"rocprofv3 --pmc FETCH_SIZE -d {copy_fetch_dir} -o cfetch -- python -u bench.py --copy-calibration --steps 3",
            f"rocprofv3 --pmc WRITE_SIZE -d {copy_write_dir} -o cwrite -- python -u bench.py --copy-calibration --steps 3",
            f"python bench.py --traffic-summary {fetch_dir} {write_dir} {copy_fetch_dir} {copy_write_dir}",
        ],
        "copy_calibration": {"bytes_per_copy": n, "fetch_size_kib": max(cf), "write_size_kib": max(cw),
                             "fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4)},
        "fetch_size_kib_per_dispatch": [round(x, 1) for x in fetch],
        "write_size_kib_per_dispatch": [round(x, 1) for x in write],
        "hbm_bytes_per_launch": int(fb + wb),
        "hbm_fetch_bytes_per_launch": int(fb),
        "hbm_write_bytes_per_launch": int(wb),
    }
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps({"hbm_bytes_per_launch": rec["hbm_bytes_per_launch"], "out": out}))


def ffn_cpu_baseline(w, sample_rows=32768):
    """The feedforward oracle as it stands, on the first sample_rows rows with the full weights."""
    import numpy as np

    from oracle.ffn import swiglu_ffn
    from workloads import make_ffn_inputs
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    x, w1, w3, w2 = make_ffn_inputs(w.rows, w.d_model, w.d_ff, seed=w.seed)
    sample_rows = min(sample_rows, w.rows)
    xs = x[:sample_rows].float().numpy().astype(np.float64)
    w1n, w3n, w2n = (t.float().numpy().astype(np.float64) for t in (w1, w3, w2))
    t0 = time.perf_counter()
    swiglu_ffn(xs, w1n, w3n, w2n)
    dt = time.perf_counter() - t0
    flop = 6.0 * sample_rows * w.d_model * w.d_ff
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{w.name}: the first {sample_rows} of {w.rows} rows with the full weights, numpy "
                      f"float64; {dt:.2f} s for {flop:.3e} algorithmic flop"}


def ffn_line(w, args):
    """One JSON line for the blockwise feedforward workload (two GEMM launches per row block)."""
    import torch

    import long_context_exact_blockattn_amd as ba
    from workloads import make_ffn_inputs
    dev = torch.device("cuda:0")
    x, w1, w3, w2 = (t.to(dev) for t in make_ffn_inputs(w.rows, w.d_model, w.d_ff, seed=w.seed))
    out = torch.empty_like(x)
    hidden = torch.empty(w.block_rows, w.d_ff, device=dev, dtype=torch.bfloat16)

    def step():
        ba.bpt_ffn(x, w1, w3, w2, block_rows=w.block_rows, out=out, hidden=hidden)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / args.steps
    tflops = w.flop() / (ms * 1e-3) / 1e12
    ev_ms = e0.elapsed_time(e1) / args.steps
    achieved = w.flop() / (ev_ms * 1e-3) / 1e12
    launches = 2 * -(-w.rows // w.block_rows)
    line = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (random weights)",
        "config": {"workload": w.name, "rows": w.rows, "d_model": w.d_model, "d_ff": w.d_ff,
                   "block_rows": w.block_rows, "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "gemm_nt_kernel (SwiGLU and plain epilogues)",
                     "avg_launch_ms": round(ev_ms / launches, 4), "launches_per_step": launches},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = ffn_cpu_baseline(w)
    print(json.dumps(line), flush=True)


def training_line(w, args):
    """One JSON line for a forward+backward workload (attention training step)."""
    import statistics
    r = run_training(w, args.steps, args.warmup)
    ms = r["wall_s"] * 1e3 / args.steps
    fwd_med, bwd_med = statistics.median(r["fwd_ms"]), statistics.median(r["bwd_ms"])
    flop = w.fwd_flop() + w.bwd_flop()
    tflops = flop / (ms * 1e-3) / 1e12
    line = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
                   "seq_len": w.seqlen, "head_dim": w.head_dim, "ring_chunks": w.n_chunks,
                   "s2_group": w.s2_group, "chunk_order": r["order"], "phases": "forward+backward",
                   "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
                   # medians of per-step HIP-event times of each phase
                   "fwd_ms": round(fwd_med, 4), "bwd_ms": round(bwd_med, 4),
                   "fwd_tflops": round(w.fwd_flop() / fwd_med / 1e9, 2),
                   "bwd_tflops": round(w.bwd_flop() / bwd_med / 1e9, 2)},
        "step_ms": {"fwd": _stats(r["fwd_ms"]), "bwd": _stats(r["bwd_ms"])},
        "peak_basis": PEAK_BASIS,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=120)  # about 1 s of timed work on the headline workload
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama2_7b_s32k_ring8")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (to scale HBM byte counters)")
    ap.add_argument("--no-side-measurements", action="store_true",
                    help="skip the one-chunk forward and the HBM-bound kernel timings (for profiled runs)")
    ap.add_argument("--counter-summary", metavar="DIR",
                    help="print MFMA-busy and VALU-busy of the forward kernel from a rocprofv3 --pmc run "
                         "with the counters in bench.COUNTERS")
    ap.add_argument("--counter-kernel", metavar="NAME",
                    help="with --counter-summary: summarise this kernel instead of the forward (printed only)")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="print per-kernel statistics of a rocprofv3 --kernel-trace output directory")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="write the forward kernel's HBM traffic summary from four rocprofv3 --pmc runs")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be at least 1 and --warmup at least 0")
    if args.counter_summary:
        counter_summary(args.counter_summary, os.path.join(PROFILE_DIR, "fwd_kernel_d128_counters.json"),
                        kernel=args.counter_kernel)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary, os.path.join(PROFILE_DIR, "fwd_kernel_d128_traffic.json"))
        return
    if args.copy_calibration:
        copy_calibration(args.steps)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the multi-GPU ring (key/value exchange between "
              "devices) is not part of this build; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    from workloads import FFN_CONFIGS, get
    if args.workload in FFN_CONFIGS:
        ffn_line(FFN_CONFIGS[args.workload], args)
        return
    w = get(args.workload)
    if w.s2_group is not None or w.backward:
        training_line(w, args)
        return
    r = run_ring_forward(w, args.steps, args.warmup)
    ms_per_step = r["wall_s"] * 1e3 / args.steps
    flop = w.fwd_flop()
    tflops = flop / (ms_per_step * 1e-3) / 1e12
    launch_ms = r["launch_ms"]
    avg_launch_ms = sum(launch_ms) / len(launch_ms)
    achieved = flop / r["launches_per_step"] / (avg_launch_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": _traffic("fwd_kernel_d128", r["src"], w.name),
                # MFMA-busy beside VALU-busy from the committed rocprofv3 --pmc summary
                "counters": _counters("fwd_kernel_d128", r["src"], w.name),
                "kernel": r["kernel"], "avg_launch_ms": round(avg_launch_ms, 4),
                "launches_per_step": r["launches_per_step"]}
    line = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
                   "seq_len": w.seqlen, "head_dim": w.head_dim, "ring_chunks": w.n_chunks,
                   "chunk_order": r["order"], "causal": True, "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2)},
        "roofline": roofline,
        # per-step HIP-event times on the working stream (the value above is from the wall clock)
        "step_ms": _stats(r["step_ms"]),
        "peak_basis": PEAK_BASIS,
    }
    tensors = r.pop("tensors")
    if not args.no_side_measurements:
        side = side_measurements(w, tensors)
        line["one_shot"] = dict(side["one_shot"],
                                ring_overhead_pct=round(100 * (ms_per_step / side["one_shot"]["ms"] - 1), 2))
        line["hbm_kernels"] = side["hbm_kernels"]
        if "ring_staged" in side:
            line["ring_staged"] = side["ring_staged"]
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
