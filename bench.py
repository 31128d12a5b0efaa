"""Attention-forward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2..9] [--no-cpu-baseline]
                    [--no-extra] [--extra]

One step is one pass of the hot path over one batch: a single fa_fwd call
(16-bit and fp32 workloads) or a single fa_fwd_int8qk call (the quantised
workload, prepass kernels included).  Inputs are seeded synthetic tensors
already resident in device memory.  Prints ONE JSON line.

The default workload is the largest single-GPU configuration: a video-DiT
720p self-attention layer at the HunyuanVideo shape (bf16, B=1, H=24,
N=119056, D=128, no mask, 4 outlier K channels scaled by 8).  The metric is
attention TFLOP/s = 4*B*H*N^2*D / t.  Unless --no-extra is given the line
also carries, under "extra", the FLUX-1024^2 layer, the SD1.5 768^2 layer
with its key lengths (nominal and effective rates) and the Wan 2.1 layer
through the INT8-QK / FP8-PV entry point next to the bf16 kernel, the
INT8-QK / 16-bit-PV form and Q smoothing on the same inputs, each comparison
timed in interleaved rounds (medians); --extra adds the cross-attention,
window-attention and merge workloads.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
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


def _code_only(text: str) -> str:
    """Source text without comments and blank runs: what the compiler sees."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(" ".join(l.split()) for l in text.splitlines() if l.strip())


def source_hash() -> str:
    """Hash of the kernel sources' code (comments ignored): HBM-traffic
    counters taken from an older build are not reported against a newer
    one."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(name.encode() + _code_only(f.read()).encode())
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


def _host_info():
    cores = len(os.sched_getaffinity(0))
    cpu, blas, blas_threads = "unknown CPU", "unknown BLAS", None
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu)
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        blas_threads = max((p.get("num_threads", 1) for p in info), default=1)
        blas = ", ".join(sorted({f"{p.get('internal_api')} {p.get('version')}" for p in info
                                 if p.get("user_api") == "blas"})) or blas
    except Exception:
        pass
    return cores, cpu, blas, blas_threads


def cpu_baseline(w, budget_s: float = 20.0, min_s: float = 10.0) -> dict:
    """The oracle on the host on a bounded sample of the same workload, rate
    in TFLOP/s of the metric (4 flop per query-key-channel).

    Where a whole head's fp64 score matrix is small (N * Nk * 8 bytes at
    most 1 GiB), whole heads through the naive formula, heads in order until
    about budget_s of work and the head list repeated until at least min_s.
    Otherwise sampled query rows: seeded rows of every head through the
    definition for selected rows (attention.rows; the quantised workload:
    the exact emulation, sage.emulate_rows, with the head's quantisation),
    as many per head as make about (min_s + budget_s) / 2 over all heads at
    the rate the first head showed, in passes until at least min_s; the
    rate is per row against all keys, and the full layer's time is a linear
    extrapolation from it."""
    import numpy as np
    from attention_fa_fwd_04_amd.workloads import T_ROWS, _rng, head, key_lengths
    from oracle import attention, sage
    cores, cpu, blas, blas_threads = _host_info()
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    kl = key_lengths(w)
    whole = w.N * w.n_keys * 8 <= (1 << 30) and not w.quantised
    t_total, t_quant, done, key_work, heads_done, passes = 0.0, 0.0, 0, 0.0, 0, 0
    rows_per_head = 64
    target = 0.5 * (min_s + budget_s)
    while t_total < min_s and passes < 50:
        passes += 1
        for (b, h) in heads:
            q, k, v = (head(w, t, b, h).double().numpy() for t in range(3))
            key_len = None if kl is None else int(kl[b])
            if whole:
                t0 = time.perf_counter()
                attention.rows(q, k, v, w.scale, key_len=key_len)
                t_total += time.perf_counter() - t0
                n = w.N
            else:
                ids = np.sort(_rng(w.wid, T_ROWS, 1000 + passes, b, h).choice(w.N, rows_per_head, replace=False))
                if heads_done == 0:             # untimed warm-up of the BLAS threads
                    attention.rows(q[ids[:8]], k, v, w.scale, key_len=key_len)
                t0 = time.perf_counter()
                if w.quantised:
                    qz = sage.quantise_head(q, k, v)
                    t_quant += time.perf_counter() - t0
                    sage.emulate_rows(q, k, v, ids, w.scale, 64, key_len=key_len, qz=qz,
                                      pv="bf16" if w.pv16 else "fp8")
                else:
                    attention.rows(q[ids], k, v, w.scale, key_len=key_len)
                dt = time.perf_counter() - t0
                t_total += dt
                n = len(ids)
                if heads_done == 0:             # size the sample from the first head's rate
                    per_row = max(dt - (t_quant if w.quantised else 0.0), 1e-6) / n
                    rows_per_head = int(min(max(target / len(heads) / per_row, 16), w.N // 2))
            done += n
            heads_done += 1
            key_work += n * (w.n_keys if key_len is None else key_len)   # valid keys of the rows done
            if t_total >= budget_s:
                break
        if t_total >= budget_s:
            break
    flops = 4.0 * key_work * w.D
    out = {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": blas_threads or cores, "kind": "oracle"}
    host = f"BLAS {blas} with {blas_threads} threads, host cores {cores}, {cpu}"
    if whole:
        out["sample"] = (f"{heads_done} head evaluations ({passes} pass(es) over the {len(heads)} heads) of "
                         f"{w.name} (N={w.N}, Nk={w.n_keys}, D={w.D}), numpy float64 naive formula, "
                         f"{t_total:.1f} s, {host}")
    else:
        rows_s = done / (t_total - t_quant)
        full_rows = w.B * w.H * w.N
        extrap = full_rows / rows_s + (t_quant / heads_done * len(heads) if w.quantised else 0.0)
        what = ("the exact INT8/FP8 emulation (sage.emulate_rows, float64 scores, quantisation of each "
                "head included)" if w.quantised else "the float64 definition for selected rows (attention.rows)")
        out["sample"] = (f"{done} query rows (seeded rows of each of the {len(heads)} heads, {rows_per_head} per "
                         f"head after the first, {passes} pass(es)) of {w.name} (N={w.N}, Nk={w.n_keys}, D={w.D}) against all "
                         f"keys, through {what}, {t_total:.1f} s; {rows_s:.1f} rows/s; linear extrapolation to "
                         f"the full layer's {full_rows} rows: {extrap:.0f} s; {host}")
        out["rows_per_s"] = round(rows_s, 2)
        out["extrapolated_full_layer_s"] = round(extrap, 1)
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the MFMA-only peak probe")
    ap.add_argument("--no-extra", action="store_true", help="time the chosen workload only")
    ap.add_argument("--extra", action="store_true",
                    help="also time the cross-attention, window-attention and merge workloads")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this size (scales HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(heads shard across GPUs without exchange; see the design notes).", file=sys.stderr)
        return 2

    import torch
    import attention_fa_fwd_04_amd as fa
    from attention_fa_fwd_04_amd.workloads import WORKLOADS, key_lengths, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    fa.lib()
    dev = torch.device("cuda", 0)

    def timed(call, steps, warmup):
        """(event-timed ms per call on the stream the kernels run on, wall ms per call)"""
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

    cache = {}

    def device_inputs(w):
        """Device copies of a workload's seeded inputs (one set held at a time;
        workloads 5 and 8 share theirs, so INT8 and bf16 see the same tensors)."""
        key = (w.wid, w.B, w.H, w.N, w.n_keys, w.D, w.dtype)
        if key not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            inp = make_inputs(w, threads=len(os.sched_getaffinity(0)))
            cache[key] = {n: (None if inp[n] is None else inp[n].to(dev)) for n in ("q", "k", "v", "key_len")}
            del inp
        return cache[key]

    def measure(w, steps, warmup, split=True, quantised=None, pv16=None, smooth=False):
        quantised = w.quantised if quantised is None else quantised
        pv16 = w.pv16 if pv16 is None else pv16
        if w.merge:
            # two partial results of the layer (seeded) merged into a third buffer
            g = torch.Generator(device="cpu").manual_seed(w.wid)
            shape = (w.B, w.H, w.N, w.D)
            oa, ob = (torch.randn(shape, generator=g).to(w.torch_dtype).to(dev) for _ in range(2))
            la, lb = (torch.randn(shape[:3], generator=g).to(dev) for _ in range(2))
            o, lse = torch.empty_like(oa), torch.empty_like(la)
            return timed(lambda: fa.merge(oa, la, ob, lb, out=o, out_lse=lse), steps, warmup)
        d = device_inputs(w)
        q, k, v, kl = d["q"], d["k"], d["v"], d["key_len"]
        o = torch.empty_like(q)
        if quantised:
            if smooth:
                nbytes = fa.fa_fwd_int8qk_smooth_workspace_bytes(w.B, w.H, w.N, w.D, 1 if pv16 else 0)
            else:
                size = fa.fa_fwd_int8qk_pv16_workspace_bytes if pv16 else fa.fa_fwd_int8qk_workspace_bytes
                nbytes = size(w.B, w.H, w.N, w.D)
            ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            pv = "16" if pv16 else "fp8"
            call = lambda: fa.fwd_int8qk(q, k, v, key_len=kl, workspace=ws, out=o, pv=pv,  # noqa: E731
                                         smooth_q=smooth)
        else:
            call = lambda: fa.fwd(q, k, v, key_len=kl, out=o, split=split)  # noqa: E731
        return timed(call, steps, warmup)

    def interleaved(w, variants, rounds, steps, warmup):
        """Median event-timed ms of each variant (measure() keyword sets), the
        variants alternating round by round (order reversed every other round)
        so that clock drift under load does not favour whichever runs first."""
        res = [[] for _ in variants]
        for r in range(rounds):
            order = range(len(variants)) if r % 2 == 0 else reversed(range(len(variants)))
            for i in order:
                res[i].append(measure(w, steps, warmup, **variants[i])[0])
        return [statistics.median(x) for x in res]

    def merge_bytes(w):
        elt = 4 if w.dtype == "f32" else 2
        return 3 * w.B * w.H * w.N * w.D * elt + 3 * w.B * w.H * w.N * 4

    def layer_flops(w):
        return 4.0 * w.B * w.H * w.N * w.n_keys * w.D

    def takes_split(w):
        return (not w.quantised and not w.Nk and not w.key_len and w.dtype != "f32" and
                fa.fa_fwd_workspace_bytes(w.B, w.H, w.N, w.D, fa.FA_BF16 if w.dtype == "bf16" else fa.FA_F16) > 0)

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
    flops = layer_flops(w)
    tflops_step = flops / (wall_ms * 1e-3) / 1e12
    tflops_kernel = flops / (ev_ms * 1e-3) / 1e12
    dkey = "int8qk" if w.quantised else w.dtype
    peak = PEAK_TFLOPS[dkey]
    split = takes_split(w)
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
                     "traffic": traffic_for(kernel_key), "kernel_ms": round(ev_ms, 4)},
    }
    if w.key_len:
        eff = 4.0 * w.H * w.D * w.N * float(key_lengths(w).sum())
        out["config"]["effective_tflops"] = round(eff / (ev_ms * 1e-3) / 1e12, 2)
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

    extra = {}
    if not args.no_extra:
        if split:
            s_ms, u_ms = interleaved(w, [{}, {"split": False}], 6, 20, 3)
            extra[w.name + " (fa_fwd_ws vs fa_fwd, interleaved)"] = {
                "split_ms": round(s_ms, 4), "no_split_ms": round(u_ms, 4),
                "no_split_tflops": round(flops / (u_ms * 1e-3) / 1e12, 2)}
        for wid in (2, 3, 5):
            wx = WORKLOADS[wid]
            if wid == args.workload:
                continue
            fl = layer_flops(wx)
            big = wx.N > 50000
            steps, warm = (5, 1) if big else (50, 5)
            if wx.quantised:
                # the three forms on the same device inputs, interleaved
                e_ms, b_ms, p_ms, s_ms = interleaved(wx, [{}, {"quantised": False}, {"pv16": True}, {"smooth": True}],
                                                     2, 3, 1)
                rec = {"int8qk_ms": round(e_ms, 4), "int8qk_tops": round(fl / (e_ms * 1e-3) / 1e12, 2),
                       "entry": "fa_fwd_int8qk (prepass kernels included)",
                       "bf16_same_inputs_ms": round(b_ms, 3),
                       "bf16_same_inputs_tflops": round(fl / (b_ms * 1e-3) / 1e12, 2),
                       "int8qk_speedup_vs_bf16": round(b_ms / e_ms, 3),
                       "int8qk_pv16_ms": round(p_ms, 3),
                       "int8qk_pv16_tops": round(fl / (p_ms * 1e-3) / 1e12, 2),
                       "int8qk_pv16_speedup_vs_bf16": round(b_ms / p_ms, 3),
                       "int8qk_smooth_ms": round(s_ms, 3),
                       "int8qk_smooth_speedup_vs_bf16": round(b_ms / s_ms, 3)}
            elif takes_split(wx):
                e_ms, u_ms = interleaved(wx, [{}, {"split": False}], 6, steps, warm)
                rec = {"ms": round(e_ms, 4), "tflops": round(fl / (e_ms * 1e-3) / 1e12, 2), "entry": "fa_fwd_ws",
                       "fa_fwd_no_split_ms": round(u_ms, 4),
                       "fa_fwd_no_split_tflops": round(fl / (u_ms * 1e-3) / 1e12, 2),
                       "timing": "interleaved rounds, medians"}
            else:
                e_ms, _ = measure(wx, steps, warm)
                rec = {"ms": round(e_ms, 4), "tflops": round(fl / (e_ms * 1e-3) / 1e12, 2)}
            if wx.key_len:
                eff = 4.0 * wx.H * wx.D * wx.N * float(key_lengths(wx).sum())
                rec["effective_tflops"] = round(eff / (e_ms * 1e-3) / 1e12, 2)
            extra[wx.name] = rec
    if args.extra:
        for wid in (4, 6, 7, 9):
            wx = WORKLOADS[wid]
            if wid == args.workload:
                continue
            if wx.merge:
                e_ms, _ = measure(wx, 50, 3)
                gb = merge_bytes(wx) / (e_ms * 1e-3) / 1e9
                extra[wx.name] = {"ms": round(e_ms, 4), "GB/s": round(gb, 1), "hbm_frac": round(gb / PEAK_HBM_GBS, 3)}
                continue
            fl = layer_flops(wx)
            e_ms, _ = measure(wx, 3 if wx.N > 50000 else 10, 1)
            io = 2.0 * wx.B * wx.H * (wx.N + wx.n_keys) * wx.D * (4 if wx.dtype == "f32" else 2)
            extra[wx.name] = {"ms": round(e_ms, 3), "tflops": round(fl / (e_ms * 1e-3) / 1e12, 2),
                              "GB/s": round(io / (e_ms * 1e-3) / 1e9, 1)}
    if extra:
        out["extra"] = extra
    cache.clear()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
