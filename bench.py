"""Throughput of the exact-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one pass of the path over one batch of synthetic inputs already
resident in HBM. The default workload is the causal bf16 softmax-stress
forward (B=2, H=32, N=8192, d=128, Q scaled by 4). The same JSON line also
carries the forward+backward measurement on the dropout workload
(B=2, H=16, N=4096, d=64, p=0.1; the backward in both its fused atomic form
and its two-pass deterministic form), the backward at the default workload's
shape, the fp32 B1 H1 N128 d64 and bf16 causal B4 H16 N2048 d64 forwards
(`other_configs`), the long-context forward (B=1, H=16, N=32768, d=128) with an N sweep
and the device memory each call takes, the decode-shaped forward on its three workloads (HBM-bound: GB/s
against 8 TB/s), the general entry points on head sizes 32/96/256, fp16,
[B, N, H, d] storage and a packed variable-length batch (`coverage`), the
roofline of the dominant kernel and the CPU oracle's throughput on a bounded
sample.

FLOPs are counted as 4*B*H*N^2*d for the forward, halved when causal, and
2.5x that for the backward.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s (fwd; fwd+bwd) and % of MI355X bf16 MFMA peak, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0
DEFAULT_WORKLOAD = "fwd_causal_q4_bf16_b2h32n8192d128"
FWD_BWD_WORKLOAD = "fwdbwd_causal_dropout_bf16_b2h16n4096d64"
LONG_WORKLOAD = "fwd_causal_bf16_b1h16n32768d128"
FWD_SOURCES = ["exact_io_aware_53_amd/csrc/fa_fwd.hip", "exact_io_aware_53_amd/csrc/fa_fwd_kernel.hpp",
               "exact_io_aware_53_amd/csrc/fa_device.hpp", "exact_io_aware_53_amd/csrc/fa_tiles.hpp",
               "exact_io_aware_53_amd/csrc/fa_launch.hpp"]


DECODE_SOURCES = ["exact_io_aware_53_amd/csrc/fa_decode_bf16.hip", "exact_io_aware_53_amd/csrc/fa_device.hpp",
                  "exact_io_aware_53_amd/csrc/fa_tiles.hpp", "exact_io_aware_53_amd/csrc/fa_launch.hpp"]
BWD_SOURCES = ["exact_io_aware_53_amd/csrc/fa_bwd.hip", "exact_io_aware_53_amd/csrc/fa_bwd_kernels.hpp",
               "exact_io_aware_53_amd/csrc/fa_bwd_dq.hpp", "exact_io_aware_53_amd/csrc/fa_device.hpp",
               "exact_io_aware_53_amd/csrc/fa_tiles.hpp", "exact_io_aware_53_amd/csrc/fa_launch.hpp"]
# Vector-instruction issue ceiling: a full-rate wave64 VALU instruction (fp32 add, fma,
# integer add/xor) occupies a SIMD's 16 lanes for 4 cycles, so 1024 SIMDs at 2.4 GHz issue
# at most 614.4e9 of them per second (the fp32 vector peak 157.3 TFLOP/s is the same figure
# times 64 lanes x 2 FLOP per FMA x 2 for packed pairs, which these kernels do not use).
PEAK_VALU_GINSTR = 614.4


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _profile_value(path, key, sources):
    if not os.path.exists(path):
        return None
    fields = dict(re.findall(r"^- (\w+): (\S+)$", open(path).read(), flags=re.M))
    if fields.get("source_hash") != source_hash(sources):
        return None
    try:
        return float(fields[key])
    except (KeyError, ValueError):
        return None


def decode_traffic(workload_name):
    """HBM bytes per decode call (split + merge passes) from the committed counter
    summary, or None when absent or the decode source changed since."""
    return _profile_value(os.path.join(ROOT, "profiles", f"fa_decode_{workload_name}_counters.md"),
                          "hbm_bytes_per_call", DECODE_SOURCES)


def counter_traffic(workload_name):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when
    no summary exists for this workload or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"fa_fwd_bf16_{workload_name}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    fields = dict(re.findall(r"^- (\w+): (\S+)$", text, flags=re.M))
    if fields.get("source_hash") != source_hash(FWD_SOURCES):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def profile_fields(name, sources):
    """The `- key: value` fields of a committed counter summary under profiles/, or {}
    when it is absent or its kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return {}
    fields = dict(re.findall(r"^- (\w+): (\S+)$", open(path).read(), flags=re.M))
    if fields.get("source_hash") != source_hash(sources):
        return {}
    return {k: float(v) for k, v in fields.items() if k != "source_hash"}


def mfma_roofline(flops, ms, traffic=None):
    tf = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(tf, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": traffic}


def valu_roofline(instr, ms, what):
    """Issue rate of the launch's vector instructions (from the committed counters)."""
    if instr is None:
        return None
    g = instr / (ms * 1e-3) / 1e9
    return {"bound": "alu", "achieved": round(g, 1), "peak": PEAK_VALU_GINSTR, "unit": "G VALU instr/s",
            "frac": round(g / PEAK_VALU_GINSTR, 4), "work": what}


def time_launches(fn, steps, warmup, stream):
    """Run fn warmup times, then `steps` timed times; returns (wall ms/step, per-launch event ms)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return wall, [a.elapsed_time(b) for a, b in evs]


def cpu_baseline(w, inputs, budget_s):
    """The CPU oracle (unchanged) on whole heads of the workload until ~budget_s of work."""
    import numpy as np
    import threadpoolctl

    import oracle
    from exact_io_aware_53_amd.inputs import to_f64

    threads = max(int(info.get("num_threads", 1)) for info in threadpoolctl.threadpool_info()) \
        if threadpoolctl.threadpool_info() else 1
    heads_done, rows_done, flops = 0, 0, 0.0
    t0 = time.perf_counter()
    chunk = 1024
    for bh in range(w.B * w.H):
        b, h = divmod(bh, w.H)
        q, k, v = (to_f64(inputs[n][b, h]) for n in ("q", "k", "v"))
        for r0 in range(0, w.N, chunk):
            rows = np.arange(r0, min(w.N, r0 + chunk))
            oracle.forward(q, k, v, w.scale, w.causal, w.dropout_p, w.dropout_seed, b, h, rows=rows)
            rows_done += len(rows)
        heads_done += 1
        flops += w.fwd_flops() / (w.B * w.H)
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    executed = 4.0 * rows_done * w.N * w.d       # the oracle forms every key's score and masks
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "executed_tflops": round(executed / dt / 1e12, 6),
            "sample": f"{heads_done} of {w.B * w.H} heads ({rows_done} query rows) of {w.name}, "
                      f"fp64 NumPy, {dt:.1f} s. The oracle forms dense score rows (every key, then the "
                      f"causal mask), {executed / max(flops, 1):.2f}x the FLOPs it is credited with: value "
                      f"counts 4*N^2*d/2 per causal head as for the GPU; executed_tflops counts what it ran"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fwd-bwd", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the fp32 B1 H1 N128 and bf16 B4 H16 N2048 d64 forward timings")
    ap.add_argument("--no-long", action="store_true", help="skip the long-context forward and its N sweep")
    ap.add_argument("--no-coverage", action="store_true",
                    help="skip the head-size / fp16 / layout / packed-batch measurements")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB copy kernel (for HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(every workload fits one MI355X). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_io_aware_53_amd as fa
    from exact_io_aware_53_amd.inputs import WORKLOADS, make_inputs

    fa.lib()
    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    host = make_inputs(w, with_grad_out=False)
    q, k, v = (host[n].to(dev) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    mem0 = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)

    def fwd_step():
        fa.fwd(q, k, v, scale=w.scale, causal=w.causal, dropout_p=w.dropout_p,
               seed=w.dropout_seed, out=o, lse=lse)

    wall_ms, ev_ms = time_launches(fwd_step, args.steps, args.warmup, stream)
    peak_extra = torch.cuda.max_memory_allocated(dev) - mem0
    kern_ms = sum(ev_ms) / len(ev_ms)
    flops = w.fwd_flops()
    value = flops / (wall_ms * 1e-3) / 1e12
    achieved = flops / (kern_ms * 1e-3) / 1e12
    traffic = counter_traffic(w.name)
    io_bytes = (4 * w.B * w.H * w.N * w.d * q.element_size()) + 4 * w.B * w.H * w.N

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded i.i.d. N(0,1) Q, K, V (Q x4 where the workload says so)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "dropout_p": w.dropout_p, "q_mult": w.q_mult,
                   "flops_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "kernel": "fwd_pp_kernel" if w.d == 128 and w.dropout_p == 0.0 else "fwd_kernel",
                     "kernel_ms": round(kern_ms, 4), "ideal_io_bytes": io_bytes},
        "pct_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "peak_extra_device_bytes": int(peak_extra),
    }

    if not args.no_fwd_bwd:
        w2 = WORKLOADS[FWD_BWD_WORKLOAD]
        h2 = make_inputs(w2)
        q2, k2, v2, do2 = (h2[n].to(dev) for n in ("q", "k", "v", "do"))
        o2 = torch.empty_like(q2)
        l2 = torch.empty((w2.B, w2.H, w2.N), dtype=torch.float32, device=dev)
        dq2, dk2, dv2 = torch.empty_like(q2), torch.empty_like(k2), torch.empty_like(v2)
        ws = torch.empty(fa.workspace_size(w2.B, w2.H, w2.N, w2.d), dtype=torch.uint8, device=dev)

        def f2():
            fa.fwd(q2, k2, v2, scale=w2.scale, causal=True, dropout_p=w2.dropout_p,
                   seed=w2.dropout_seed, out=o2, lse=l2)

        def b2():
            fa.bwd(q2, k2, v2, o2, l2, do2, scale=w2.scale, causal=True, dropout_p=w2.dropout_p,
                   seed=w2.dropout_seed, dq=dq2, dk=dk2, dv=dv2, workspace=ws)

        def b2_det():
            fa.bwd(q2, k2, v2, o2, l2, do2, scale=w2.scale, causal=True, dropout_p=w2.dropout_p,
                   seed=w2.dropout_seed, dq=dq2, dk=dk2, dv=dv2, workspace=ws, deterministic=True)

        f2()
        tf, _ = time_launches(f2, args.steps, args.warmup, stream)
        tb, _ = time_launches(b2, args.steps, args.warmup, stream)
        td, _ = time_launches(b2_det, args.steps, args.warmup, stream)
        line["fwd_bwd"] = {
            "workload": w2.name, "ms_fwd": round(tf, 4), "ms_bwd": round(tb, 4),
            "tflops_fwd": round(w2.fwd_flops() / (tf * 1e-3) / 1e12, 3),
            "tflops_bwd": round(w2.bwd_flops() / (tb * 1e-3) / 1e12, 3),
            "tflops_fwd_bwd": round((w2.fwd_flops() + w2.bwd_flops()) / ((tf + tb) * 1e-3) / 1e12, 3),
            # two-pass deterministic form: the dropout mask is generated twice
            "ms_bwd_deterministic": round(td, 4),
            "tflops_bwd_deterministic": round(w2.bwd_flops() / (td * 1e-3) / 1e12, 3),
        }
        # Philox-bound: vector-instruction issue against its ceiling (counts from the
        # committed counters), with the matrix-core fraction beside it.
        pf = profile_fields(f"fa_fwd_bf16_{w2.name}_counters.md", FWD_SOURCES)
        pb = profile_fields(f"fa_bwd_bf16_{w2.name}_counters.md", BWD_SOURCES)
        line["fwd_bwd"]["roofline_fwd"] = valu_roofline(
            pf.get("valu_instr_per_launch"), tf, "softmax and one Philox-4x32-10 call per unmasked score")
        line["fwd_bwd"]["roofline_bwd"] = valu_roofline(
            pb.get("fused_valu_instr_per_call"), tb, "recompute, one Philox call per unmasked score, five products")
        line["fwd_bwd"]["roofline_bwd_deterministic"] = valu_roofline(
            pb.get("det_valu_instr_per_call"), td, "as the fused form, with the Philox calls made in both passes")
        line["fwd_bwd"]["mfma_fwd"] = mfma_roofline(w2.fwd_flops(), tf, pf.get("hbm_bytes_per_launch"))
        line["fwd_bwd"]["mfma_bwd"] = mfma_roofline(w2.bwd_flops(), tb, pb.get("fused_hbm_bytes_per_call"))
        del q2, k2, v2, do2, o2, l2, dq2, dk2, dv2, ws

        # The backward at the forward workload's shape (no dropout: the two-pass
        # form, no atomics), on the same seeded Q, K, V plus a seeded dO.
        h3 = make_inputs(w, with_grad_out=True)
        do3 = h3["do"].to(dev)
        del h3
        dq3, dk3, dv3 = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws3 = torch.empty(fa.workspace_size(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=dev)
        fwd_step()

        def b3():
            fa.bwd(q, k, v, o, lse, do3, scale=w.scale, causal=w.causal, dropout_p=w.dropout_p,
                   seed=w.dropout_seed, dq=dq3, dk=dk3, dv=dv3, workspace=ws3)

        t3, _ = time_launches(b3, args.steps, args.warmup, stream)
        p3 = profile_fields(f"fa_bwd_bf16_b{w.B}h{w.H}n{w.N}d{w.d}_counters.md", BWD_SOURCES)
        line["bwd"] = {"workload": w.name, "ms_bwd": round(t3, 4),
                       "tflops_bwd": round(w.bwd_flops() / (t3 * 1e-3) / 1e12, 3),
                       "frac": round(w.bwd_flops() / (t3 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                       "roofline": mfma_roofline(w.bwd_flops(), t3, p3.get("hbm_bytes_per_call"))}
        del do3, dq3, dk3, dv3, ws3

    if not args.no_long:
        # Long-context forward (B1 H16 N32768 d128 causal) and an N sweep at the same
        # B, H, d: time, and device memory the call itself takes (free memory read
        # by hipMemGetInfo around it, outputs preallocated): zero at every N.
        wl = WORKLOADS[LONG_WORKLOAD]
        sweep = []
        for n in (4096, 8192, 16384, wl.N):
            hl = make_inputs(wl, with_grad_out=False) if n == wl.N else None
            if hl is None:
                from exact_io_aware_53_amd.inputs import normal_tensors
                ql, kl, vl = (x.to(dev) for x in normal_tensors((wl.B, wl.H, n, wl.d), wl.data_seed, 3,
                                                                  torch.bfloat16))
            else:
                ql, kl, vl = (hl[x].to(dev) for x in ("q", "k", "v"))
                del hl
            ol = torch.empty_like(ql)
            ll = torch.empty((wl.B, wl.H, n), dtype=torch.float32, device=dev)

            def fl():
                fa.fwd(ql, kl, vl, scale=wl.scale, causal=True, out=ol, lse=ll)

            fl()
            torch.cuda.synchronize()
            free0 = torch.cuda.mem_get_info(dev)[0]
            _, evl = time_launches(fl, max(5, args.steps // 3), 2, stream)
            free1 = torch.cuda.mem_get_info(dev)[0]
            ml = sum(evl) / len(evl)
            fl_flops = 4.0 * wl.B * wl.H * n * n * wl.d / 2
            sweep.append({"N": n, "ms": round(ml, 4), "tflops": round(fl_flops / (ml * 1e-3) / 1e12, 3),
                          "tensor_bytes": 4 * wl.B * wl.H * n * wl.d * 2 + 4 * wl.B * wl.H * n,
                          "call_device_bytes": int(free0 - free1)})
            del ql, kl, vl, ol, ll
            torch.cuda.empty_cache()
        line["long_context"] = {"workload": wl.name, "sweep": sweep,
                                "s_matrix_bytes_avoided_bf16": 2 * wl.B * wl.H * wl.N * wl.N}

    if not args.no_other:
        # The two remaining forward configurations: the fp32 B1 H1 N128 d64
        # non-causal forward (launch-bound: microseconds are what it shows) and
        # the causal bf16 B4 H16 N2048 d64 forward.
        others = []
        for name in ("fwd_f32_b1h1n128d64", "fwd_causal_bf16_b4h16n2048d64"):
            wo = WORKLOADS[name]
            ho = make_inputs(wo, with_grad_out=False)
            qo, ko, vo = (ho[x].to(dev) for x in ("q", "k", "v"))
            oo = torch.empty_like(qo)
            lo = torch.empty((wo.B, wo.H, wo.N), dtype=torch.float32, device=dev)

            def fo():
                fa.fwd(qo, ko, vo, scale=wo.scale, causal=wo.causal, out=oo, lse=lo)

            _, evo = time_launches(fo, args.steps, args.warmup, stream)
            mo = sum(evo) / len(evo)
            entry = {"workload": name, "dtype": wo.dtype, "us": round(mo * 1e3, 2),
                     "tflops": round(wo.fwd_flops() / (mo * 1e-3) / 1e12, 3)}
            if wo.dtype == "bf16":
                po = profile_fields(f"fa_fwd_bf16_{name}_counters.md", FWD_SOURCES)
                entry["roofline"] = mfma_roofline(wo.fwd_flops(), mo, po.get("hbm_bytes_per_launch"))
                entry["valu"] = valu_roofline(po.get("valu_instr_per_launch"), mo,
                                              "softmax: fma, exp2, add, half a cvt and half a max3 per score")
            else:
                entry["bound"] = "launch latency (one 128-row head, 8 workgroups)"
            others.append(entry)
            del qo, ko, vo, oo, lo
        line["other_configs"] = others

    if not args.no_decode:
        from exact_io_aware_53_amd.inputs import DECODE_WORKLOADS, make_decode_inputs
        dec = []
        for wd in DECODE_WORKLOADS.values():
            hd = make_decode_inputs(wd)
            names = ("q", "k_pages", "v_pages", "block_table", "seq_lens") if wd.page else ("q", "k", "v")
            td = [hd[n].to(dev) for n in names]
            od = torch.empty_like(td[0])
            ld = torch.empty((wd.B, wd.H, wd.Nq), dtype=torch.float32, device=dev)
            wsd = torch.empty(1 << 26, dtype=torch.uint8, device=dev)    # above either need

            def fd():
                if wd.page:
                    fa.fwd_decode_paged(*td, scale=wd.scale, causal=wd.causal, out=od, lse=ld,
                                        workspace=wsd)
                else:
                    fa.fwd_decode(*td, scale=wd.scale, causal=wd.causal, out=od, lse=ld,
                                  workspace=wsd)

            _, evd = time_launches(fd, args.steps, args.warmup, stream)
            dms = sum(evd) / len(evd)
            gbs = wd.io_bytes() / (dms * 1e-3) / 1e9
            dec.append({"workload": wd.name, "ms": round(dms, 4),
                        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                                     "traffic": decode_traffic(wd.name), "ideal_io_bytes": wd.io_bytes()}})
            del td, od, ld, wsd
        line["decode"] = dec

    if not args.no_coverage:
        from exact_io_aware_53_amd.inputs import COVERAGE_WORKLOADS, make_coverage_inputs
        cov = []
        for wc in COVERAGE_WORKLOADS.values():
            hc = make_coverage_inputs(wc)
            t = {n: x.to(dev) for n, x in hc.items()}
            del hc
            if wc.layout == "varlen":
                mx = int(wc.lengths().max())
                o_c, l_c = fa.fwd_varlen(t["q"], t["k"], t["v"], t["cu_seqlens"], mx, causal=wc.causal)

                def fc():
                    fa.fwd_varlen(t["q"], t["k"], t["v"], t["cu_seqlens"], mx, causal=wc.causal,
                                  out=o_c, lse=l_c)

                def bc():
                    fa.bwd_varlen(t["q"], t["k"], t["v"], o_c, l_c, t["do"], t["cu_seqlens"], mx,
                                  causal=wc.causal)
            else:
                view = (lambda x: x.transpose(1, 2)) if wc.layout == "bshd" else (lambda x: x)
                q_c, k_c, v_c, do_c = (view(t[n]) for n in ("q", "k", "v", "do"))
                o_c, l_c = fa.fwd_ex(q_c, k_c, v_c, causal=wc.causal)

                def fc():
                    fa.fwd_ex(q_c, k_c, v_c, causal=wc.causal, out=o_c, lse=l_c)

                def bc():
                    fa.bwd_ex(q_c, k_c, v_c, o_c, l_c, do_c, causal=wc.causal)

            _, evf = time_launches(fc, args.steps, args.warmup, stream)
            _, evb = time_launches(bc, max(5, args.steps // 3), 2, stream)
            mf, mb = sum(evf) / len(evf), sum(evb) / len(evb)
            cov.append({"workload": wc.name, "ms_fwd": round(mf, 4), "ms_bwd": round(mb, 4),
                        "tflops_fwd": round(wc.fwd_flops() / (mf * 1e-3) / 1e12, 3),
                        "tflops_bwd": round(wc.bwd_flops() / (mb * 1e-3) / 1e12, 3)})
            del t, o_c, l_c
            torch.cuda.empty_cache()
        line["coverage"] = cov

    if args.calibrate_copy:
        # A plain elementwise copy of known size: reads and writes 2^30 bytes per launch.
        src = torch.ones(2**28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = 2**30
        del src, dst

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, host, args.cpu_budget)

    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
