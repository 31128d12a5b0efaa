"""Attention-forward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2..9] [--no-cpu-baseline]
                    [--extra]

One step is one pass of the hot path over one batch: a single fa_fwd call
(bf16 workloads) or a single fa_fwd_int8qk call (the quantised workload,
prepass kernels included).  Inputs are seeded synthetic tensors already
resident in device memory.  Prints ONE JSON line.

The default workload is FLUX-1024^2 self-attention (bf16, B=1, H=24,
N=4608, D=128, no mask).  The metric is attention TFLOP/s = 4*B*H*N^2*D / t.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (4·B·H·N²·D/s) and % of MFMA peak, 1 MI355X"
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3, "int8qk": 5000.0}
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "attention_fa_fwd_04_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def source_hash() -> str:
    """Hash of the kernel sources: HBM-traffic counters taken from an older
    build are not reported against a newer one."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel_key: str):
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kernel_key)
    if not e or e.get("source_hash") != source_hash():
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(w, budget_s: float = 20.0, min_s: float = 10.0) -> dict:
    """The oracle (numpy fp64 naive formula) on the host, over whole heads of
    the same workload: heads in order until about budget_s of work, and the
    whole head list repeated until at least min_s; rate in TFLOP/s."""
    import numpy as np  # noqa: F401
    from attention_fa_fwd_04_amd.workloads import head
    from oracle import attention
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:
        blas_threads = None
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done, t_total, passes = 0, 0.0, 0
    while t_total < min_s and passes < 20:
        passes += 1
        for (b, h) in heads:
            q, k, v = (head(w, t, b, h).double().numpy()[None, None] for t in range(3))
            t0 = time.perf_counter()
            attention.naive(q, k, v, w.scale)
            t_total += time.perf_counter() - t0
            done += 1
            if t_total >= budget_s:
                break
        if t_total >= budget_s:
            break
    flops = 4.0 * done * w.N * w.n_keys * w.D
    cores = len(os.sched_getaffinity(0))
    cpu, blas = "unknown CPU", "unknown BLAS"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu)
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = ", ".join(sorted({f"{p.get('internal_api')} {p.get('version')}" for p in threadpool_info()
                                 if p.get("user_api") == "blas"})) or blas
    except Exception:
        pass
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": blas_threads or cores,
            "kind": "oracle",
            "sample": f"{done} head evaluations ({passes} pass(es) over the {len(heads)} heads) of {w.name} "
                      f"(N={w.N}, Nk={w.n_keys}, D={w.D}), numpy float64 naive formula, {t_total:.1f} s, "
                      f"BLAS {blas} with {blas_threads} threads, host cores {cores}, {cpu}"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the MFMA-only peak probe")
    ap.add_argument("--extra", action="store_true", help="also time the other full-size workloads")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this size (scales HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(heads shard across GPUs without exchange; see the design notes).", file=sys.stderr)
        return 2

    import torch
    import attention_fa_fwd_04_amd as fa
    from attention_fa_fwd_04_amd.workloads import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    fa.lib()
    dev = torch.device("cuda", 0)

    def timed(call, steps, warmup):
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        st = torch.cuda.current_stream(dev)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(st)
        for _ in range(steps):
            call()
        e1.record(st)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) / steps, wall / steps * 1e3

    def measure(w, steps, warmup, split=True):
        if w.merge:
            # two partial results of the layer (seeded) merged into a third buffer
            g = torch.Generator(device="cpu").manual_seed(w.wid)
            shape = (w.B, w.H, w.N, w.D)
            oa, ob = (torch.randn(shape, generator=g).to(w.torch_dtype).to(dev) for _ in range(2))
            la, lb = (torch.randn(shape[:3], generator=g).to(dev) for _ in range(2))
            o, lse = torch.empty_like(oa), torch.empty_like(la)
            return timed(lambda: fa.merge(oa, la, ob, lb, out=o, out_lse=lse), steps, warmup)
        inp = make_inputs(w)
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        kl = None if inp["key_len"] is None else inp["key_len"].to(dev)
        o = torch.empty_like(q)
        if w.quantised:
            size = fa.fa_fwd_int8qk_pv16_workspace_bytes if w.pv16 else fa.fa_fwd_int8qk_workspace_bytes
            ws = torch.empty(size(w.B, w.H, w.N, w.D), dtype=torch.uint8, device=dev)
            pv = "16" if w.pv16 else "fp8"
            call = lambda: fa.fwd_int8qk(q, k, v, key_len=kl, workspace=ws, out=o, pv=pv)  # noqa: E731
        else:
            call = lambda: fa.fwd(q, k, v, key_len=kl, out=o, split=split)  # noqa: E731
        return timed(call, steps, warmup)

    def merge_bytes(w):
        elt = 4 if w.dtype == "f32" else 2
        return 3 * w.B * w.H * w.N * w.D * elt + 3 * w.B * w.H * w.N * 4

    if args.copy_calibration_mib:
        # a plain copy of known size: reads and writes exactly this many bytes
        nbytes = args.copy_calibration_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    w = WORKLOADS[args.workload]
    ev_ms, wall_ms = measure(w, args.steps, args.warmup)
    if w.merge:
        gbs = merge_bytes(w) / (ev_ms * 1e-3) / 1e9
        out = {"metric": "lse merge of two partial attention results, GB/s (bytes read + written / s)",
               "value": round(merge_bytes(w) / (wall_ms * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
               "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 4),
               "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
               "data": "synthetic (seeded)",
               "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "D": w.D},
               "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic_for(f"fa_merge:{w.name}")}}
        print(json.dumps(out), flush=True)
        return 0
    flops = 4.0 * w.B * w.H * w.N * w.n_keys * w.D
    tflops_step = flops / (wall_ms * 1e-3) / 1e12
    tflops_kernel = flops / (ev_ms * 1e-3) / 1e12
    dkey = "int8qk" if w.quantised else w.dtype
    peak = PEAK_TFLOPS[dkey]
    split = (not w.quantised and not w.Nk and not w.key_len and w.dtype != "f32" and
             fa.fa_fwd_workspace_bytes(w.B, w.H, w.N, w.D, fa.FA_BF16 if w.dtype == "bf16" else fa.FA_F16) > 0)
    entry = ("fa_fwd_int8qk_pv16" if w.pv16 else "fa_fwd_int8qk") if w.quantised else \
        ("fa_fwd_cross" if w.Nk else ("fa_fwd_ws" if split else "fa_fwd"))
    kernel_key = f"{entry}:{w.name}"
    out = {
        "metric": METRIC,
        "value": round(tflops_step, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8/fp8 (bf16 in/out)" if w.quantised else w.dtype,
        "data": "synthetic (seeded N(0,1) tensors of the workload's shape)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "Nk": w.n_keys, "D": w.D,
                   "mask": "key_len" if w.key_len else "none", "causal": False, "entry": entry},
        "roofline": {"bound": "mfma", "achieved": round(tflops_kernel, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops_kernel / peak, 4),
                     "traffic": traffic_for(kernel_key)},
    }
    # The sustained MFMA rate of the kernel's data type from an MFMA-only
    # probe: the fraction of what the part holds under load, next to the
    # fraction of the published peak.
    if not args.no_probe and w.dtype != "f32":
        kinds = {"int8": 2, "fp8": 1} if w.quantised else {"bf16" if w.dtype == "bf16" else "f16": 0}
        try:
            mp = {name: round(fa.mfma_peak(kind, device=dev), 1) for name, kind in kinds.items()}
        except Exception as e:          # the probe is a side measurement: never lose the bench line
            print(f"bench.py: MFMA probe failed: {e}", file=sys.stderr)
            mp = None
        out["roofline"]["measured_peak"] = mp
        if mp and not w.quantised:
            out["roofline"]["frac_of_measured_peak"] = round(tflops_kernel / next(iter(mp.values())), 4)
    # Q and O once, K and V once: with few keys (cross-attention on a short
    # text sequence) moving these bytes takes longer than the MFMA work
    elt = 4 if w.dtype == "f32" else 2
    io_bytes = 2.0 * w.B * w.H * (w.N + w.n_keys) * w.D * elt
    if io_bytes / (PEAK_HBM_GBS * 1e9) > flops / (peak * 1e12):
        gbs = io_bytes / (ev_ms * 1e-3) / 1e9
        out["roofline"].update({"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)})
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    if args.extra:
        extra = {}
        if split:
            u_ms, _ = measure(w, 20, 3, split=False)
            extra[w.name + " (fa_fwd, no split)"] = {"ms": round(u_ms, 4), "tflops": round(flops / (u_ms * 1e-3) / 1e12, 2)}
        for wid in (3, 4, 5, 6, 7, 9):
            wx = WORKLOADS[wid]
            if wx.merge:
                e_ms, _ = measure(wx, 50, 3)
                gb = merge_bytes(wx) / (e_ms * 1e-3) / 1e9
                extra[wx.name] = {"ms": round(e_ms, 4), "GB/s": round(gb, 1), "hbm_frac": round(gb / PEAK_HBM_GBS, 3)}
                continue
            fl = 4.0 * wx.B * wx.H * wx.N * wx.n_keys * wx.D
            try:
                e_ms, _ = measure(wx, 3 if wid in (4, 5) else 10, 1)
                io = 2.0 * wx.B * wx.H * (wx.N + wx.n_keys) * wx.D * (4 if wx.dtype == "f32" else 2)
                extra[wx.name] = {"ms": round(e_ms, 3), "tflops": round(fl / (e_ms * 1e-3) / 1e12, 2),
                                  "GB/s": round(io / (e_ms * 1e-3) / 1e9, 1)}
            except fa.FAError as e:
                extra[wx.name] = {"error": str(e)}
            if wx.quantised:
                wb = wx.with_shape(quantised=False)
                b_ms, _ = measure(wb, 3, 1)
                extra[wx.name]["bf16_same_inputs_ms"] = round(b_ms, 3)
                extra[wx.name]["bf16_same_inputs_tflops"] = round(fl / (b_ms * 1e-3) / 1e12, 2)
                p_ms, _ = measure(wx.with_shape(pv16=True), 3, 1)
                extra[wx.name]["int8qk_pv16_ms"] = round(p_ms, 3)
                extra[wx.name]["int8qk_pv16_tops"] = round(fl / (p_ms * 1e-3) / 1e12, 2)
        out["extra"] = extra
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
