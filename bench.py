#!/usr/bin/env python3
"""Benchmark of the exact tiled attention forward pass on one MI355X.

One step = one forward pass (the whole hot path: Q tile load, K/V tile stream,
QKᵀ, masks, online softmax, P·V, epilogue) over one batch of a named
synthetic workload, launched through the C ABI on torch's current stream with
the inputs already resident in HBM.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]
                    [--no-cpu-baseline] [--no-extra]

value = 4·B·H·N²·d / time (TFLOP/s, the metric as written) for the headline
workload (B=4, H=8, N=1024, d=64, bf16, non-causal).  The three long
bf16 workloads are timed too and reported under "workloads" with both the
nominal and the algorithmic (causal: N(N+1)/2 pairs, padded: N·Σkey_len
pairs) rates and their fraction of the bf16 MFMA peak.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (4·B·H·N²·d) and % of bf16 MFMA peak, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix, published
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published
HEADLINE = 2


def nominal_flops(w):
    return 4.0 * w.B * w.H * w.N * w.N * w.d


def algorithmic_flops(w, key_lens):
    """Work the method must do: 4·d flops per admissible (query, key) pair."""
    if w.causal:
        pairs = w.B * w.H * w.N * (w.N + 1) / 2
    elif key_lens is not None:
        pairs = w.H * w.N * float(sum(int(x) for x in key_lens))
    else:
        pairs = w.B * w.H * w.N * w.N
    return 4.0 * w.d * pairs


def algorithmic_bytes(w):
    """Compulsory HBM bytes of one launch: read Q, K, V once, write O and LSE."""
    e = 2 if w.dtype == "bf16" else 4
    return (2 * w.B * w.H * w.N * w.d + 2 * w.B * w.Hkv * w.N * w.d) * e + 4 * w.B * w.H * w.N


# the sources that decide what the forward bf16 kernel does and how it is launched
FORWARD_SOURCES = ("attn_api.hip", "attn_common.h", "attn_fwd_bf16.hip")


def kernel_source_hash():
    h = hashlib.sha256()
    for name in FORWARD_SOURCES:
        with open(os.path.join(ROOT, "exact_tiled_attention_14_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload_id):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when they are absent or were taken on another version of the kernels."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    ent = rec.get("workloads", {}).get(str(workload_id))
    return None if ent is None else ent.get("bytes_per_launch")


def stored_mfma_util(workload_id):
    """Matrix-core busy fraction and effective shader clock of the forward
    kernel from the committed rocprofv3 counter runs (SQ_VALU_MFMA_BUSY_CYCLES,
    SQ_BUSY_CYCLES), or None when absent or taken on another kernel version."""
    path = os.path.join(ROOT, "profiles", "mfma_util.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    ent = rec.get("workloads", {}).get(str(workload_id))
    return None if ent is None else {"mfma_busy": ent["mfma_busy"], "clock_ghz": ent["clock_ghz"]}


class Runner:
    """Inputs of one workload resident on the GPU and a raw C-ABI launch."""

    def __init__(self, w, dev):
        import torch

        import exact_tiled_attention_14_amd as attn
        from workloads import make_inputs

        self.w = w
        q, k, v, kl = make_inputs(w)
        self.key_lens_host = None if kl is None else kl.tolist()
        self.q, self.k, self.v = q.to(dev), k.to(dev), v.to(dev)
        self.kl = None if kl is None else kl.to(dev)
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        self.stream = torch.cuda.current_stream(dev)
        self.fn = attn.attn_fwd_bf16 if w.dtype == "bf16" else attn.attn_fwd_f32
        self.args = (self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.o.data_ptr(),
                     self.lse.data_ptr(), w.B, w.H, w.Hkv, w.N, w.d, w.scale, int(w.causal),
                     None if self.kl is None else self.kl.data_ptr(), self.stream.cuda_stream)

    def launch(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError(f"attention launch failed with status {st}")

    def prepare_backward(self):
        """Forward outputs, a seeded dout and the gradient buffers (bf16 only)."""
        import torch

        import exact_tiled_attention_14_amd as attn

        w = self.w
        self.launch()
        g = torch.Generator().manual_seed(1000 + w.seed)
        self.dout = torch.randn(self.q.shape, generator=g).to(torch.bfloat16).to(self.q.device)
        self.dq = torch.empty_like(self.q)
        self.dk = torch.empty_like(self.k)
        self.dv = torch.empty_like(self.v)
        self.delta = torch.empty((2, w.B, w.H, w.N), dtype=torch.float32, device=self.q.device)
        self.bwd_args = (self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.o.data_ptr(),
                         self.dout.data_ptr(), self.lse.data_ptr(), self.dq.data_ptr(), self.dk.data_ptr(),
                         self.dv.data_ptr(), self.delta.data_ptr(), w.B, w.H, w.Hkv, w.N, w.d, w.scale,
                         int(w.causal), None if self.kl is None else self.kl.data_ptr(), self.stream.cuda_stream)
        self.bwd_fn = attn.attn_bwd_bf16

    def launch_backward(self):
        st = self.bwd_fn(*self.bwd_args)
        if st != 0:
            raise RuntimeError(f"backward launch failed with status {st}")

    def time(self, steps, warmup, fn=None):
        """Average milliseconds per launch over `steps` back-to-back launches,
        bracketed by HIP events recorded on the launch stream."""
        import torch

        fn = fn or self.launch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(self.stream)
        for _ in range(steps):
            fn()
        end.record(self.stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps


class Fp8Runner(Runner):
    """A workload's fp8 form (attn_fwd_fp8: e4m3 q, k and V transposed, one
    descale factor each) resident on the GPU."""

    def __init__(self, w, dev):
        import torch

        import exact_tiled_attention_14_amd as attn
        from workloads import make_fp8

        self.w = w
        q8, k8, _, vt8, ds, kl = make_fp8(w.B, w.H, w.Hkv, w.N, w.d, seed=100 + w.seed, padded=w.padded)
        self.key_lens_host = None if kl is None else kl.tolist()
        self.q, self.k, self.vt = q8.to(dev), k8.to(dev), vt8.to(dev)
        self.kl = None if kl is None else kl.to(dev)
        self.o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        self.stream = torch.cuda.current_stream(dev)
        self.fn = attn.attn_fwd_fp8
        self.args = (self.q.data_ptr(), self.k.data_ptr(), self.vt.data_ptr(), self.o.data_ptr(),
                     self.lse.data_ptr(), ds[0], ds[1], ds[2], w.B, w.H, w.Hkv, w.N, w.d, w.scale, int(w.causal),
                     None if self.kl is None else self.kl.data_ptr(), self.stream.cuda_stream)


class VarlenRunner(Runner):
    """The packed variable-length batch (attn_fwd_varlen_bf16) resident on the GPU."""

    def __init__(self, spec, dev):
        import torch

        import exact_tiled_attention_14_amd as attn
        from workloads import make_varlen, varlen_lengths

        self.spec = spec
        self.lengths = varlen_lengths(spec["B"], spec["N"] // 2, spec["N"], spec["seed"])
        q, k, v, cu = make_varlen(self.lengths, spec["H"], spec["Hkv"], spec["d"], seed=spec["seed"])
        total = q.shape[0]
        self.q, self.k, self.v, self.cu = q.to(dev), k.to(dev), v.to(dev), cu.to(dev)
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((spec["H"], total), dtype=torch.float32, device=dev)
        self.stream = torch.cuda.current_stream(dev)
        self.fn = attn.attn_fwd_varlen_bf16
        scale = float(1.0 / math.sqrt(spec["d"]))
        self.args = (self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.o.data_ptr(),
                     self.lse.data_ptr(), self.cu.data_ptr(), spec["B"], spec["H"], spec["Hkv"], total,
                     spec["N"], spec["d"], scale, int(spec["causal"]), self.stream.cuda_stream)

    def algorithmic_flops(self):
        s = self.spec
        pairs = sum(n * (n + 1) / 2 if s["causal"] else n * n for n in self.lengths)
        return 4.0 * s["d"] * s["H"] * pairs


class SplitKVRunner(Runner):
    """The split-KV shape (attn_fwd_splitkv_bf16) resident on the GPU, with
    its workspace; ``launch_one`` times the same problem as one key range."""

    def __init__(self, spec, dev, splits=None):
        import torch

        import exact_tiled_attention_14_amd as attn

        self.spec = spec
        s = spec
        g = torch.Generator("cpu").manual_seed(s["seed"])
        q = torch.randn((s["B"], s["H"], s["Nq"], s["d"]), generator=g).to(torch.bfloat16)
        k = torch.randn((s["B"], s["Hkv"], s["Nk"], s["d"]), generator=g).to(torch.bfloat16)
        v = torch.randn((s["B"], s["Hkv"], s["Nk"], s["d"]), generator=g).to(torch.bfloat16)
        self.q, self.k, self.v = q.to(dev), k.to(dev), v.to(dev)
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((s["B"], s["H"], s["Nq"]), dtype=torch.float32, device=dev)
        self.splits = s["splits"] if splits is None else splits
        self.nbytes = attn.attn_splitkv_workspace_bytes(s["B"], s["H"], s["Nq"], s["d"], self.splits)
        self.ws = torch.empty(max(self.nbytes, 16), dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream(dev)
        self.fn = attn.attn_fwd_splitkv_bf16
        scale = float(1.0 / math.sqrt(s["d"]))
        self.args = (self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.o.data_ptr(),
                     self.lse.data_ptr(), s["B"], s["H"], s["Hkv"], s["Nq"], s["Nk"], s["d"], scale,
                     int(s["causal"]), s["Nk"] - s["Nq"], 0, None, self.splits, self.ws.data_ptr(), self.nbytes,
                     self.stream.cuda_stream)

    def algorithmic_flops(self):
        s = self.spec
        nq, nk = s["Nq"], s["Nk"]
        pairs = nq * (nk - nq) + nq * (nq + 1) / 2 if s["causal"] else nq * nk
        return 4.0 * s["d"] * s["H"] * s["B"] * pairs


def cpu_baseline(w, budget_s=10.0):
    """The fp64 oracle, as it stands, on this host's cores over a bounded sample
    of the workload: whole (b, h) heads, all query rows, in order, repeating
    passes over the workload until about ``budget_s`` seconds are spent.
    Reported in the metric's unit (TFLOP/s of the nominal 4·N²·d count per
    head)."""
    import numpy as np

    import oracle
    from workloads import as_f64, make_inputs

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    q, k, v, kl = make_inputs(w)
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    group = w.H // w.Hkv
    heads = 0
    t0 = time.perf_counter()
    done = False
    while not done:
        for b in range(w.B):
            for h in range(w.H):
                g = h // group
                oracle.attention(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1],
                                 w.scale, causal=w.causal,
                                 key_lens=None if kl is None else [int(kl[b])])
                heads += 1
                if time.perf_counter() - t0 >= budget_s:
                    done = True
                    break
            if done:
                break
    dt = time.perf_counter() - t0
    flops = 4.0 * heads * w.N * w.N * w.d
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{heads} (b,h) head passes ({heads / (w.B * w.H):.2f} x the {w.B * w.H}-head "
                      f"workload), all {w.N} query rows each, fp64 numpy, {dt:.1f} s wall",
            "seconds": round(dt, 2)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip timing the other bf16 workloads")
    ap.add_argument("--no-backward", action="store_true", help="skip timing the backward pass")
    ap.add_argument("--no-varlen", action="store_true", help="skip timing the packed variable-length batch")
    ap.add_argument("--no-splitkv", action="store_true", help="skip timing the split-KV shape")
    ap.add_argument("--no-fp8", action="store_true", help="skip timing the fp8 forward")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 3 device-to-device copies of MIB MiB (a plain copy kernel of known "
                         "traffic, to calibrate the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): the forward pass "
              "has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from workloads import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))
        return
    w = WORKLOADS[args.workload]

    r = Runner(w, dev)
    ms = r.time(args.steps, args.warmup)
    nom = nominal_flops(w)
    alg = algorithmic_flops(w, r.key_lens_host)
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    achieved = alg / (ms * 1e-3) / 1e12
    traffic = stored_traffic(args.workload)

    line = {
        "metric": METRIC,
        "value": round(nom / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded i.i.d. N(0,1) q/k/v; no dataset)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "causal": w.causal, "padded": w.padded, "scale": w.scale},
        "frac_of_bf16_peak": round(achieved / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "algorithmic_bytes": algorithmic_bytes(w),
                     "algorithmic_flops": alg,
                     "counters": stored_mfma_util(args.workload)},
    }

    if not args.no_extra:
        extra = {}
        for wid in (3, 4, 5):
            if wid == args.workload:
                continue
            ww = WORKLOADS[wid]
            rr = Runner(ww, dev)
            steps = max(10, min(args.steps, 100))
            m = rr.time(steps, max(3, args.warmup // 4))
            a = algorithmic_flops(ww, rr.key_lens_host)
            extra[str(wid)] = {
                "workload": ww.name, "ms": round(m, 4), "steps": steps,
                "nominal_tflops": round(nominal_flops(ww) / (m * 1e-3) / 1e12, 2),
                "algorithmic_tflops": round(a / (m * 1e-3) / 1e12, 2),
                "frac_of_bf16_peak": round(a / (m * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                "traffic": stored_traffic(wid),
                "counters": stored_mfma_util(wid),
            }
            del rr
        line["workloads"] = extra

    if not args.no_backward:
        # backward pass (dq, dk, dv): algorithmic flops = 2.5 x the forward's
        # (five products per admissible (query, key) pair instead of two)
        bwd = {}
        for wid in (2, 3, 4, 5):
            ww = WORKLOADS[wid]
            if ww.dtype != "bf16":
                continue
            rr = Runner(ww, dev)
            rr.prepare_backward()
            steps = max(5, min(args.steps, 30))
            m = rr.time(steps, 3, fn=rr.launch_backward)
            a = 2.5 * algorithmic_flops(ww, rr.key_lens_host)
            bwd[str(wid)] = {"workload": ww.name, "ms": round(m, 4), "steps": steps,
                             "algorithmic_tflops": round(a / (m * 1e-3) / 1e12, 2),
                             "frac_of_bf16_peak": round(a / (m * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
            del rr
        line["backward"] = bwd

    if not args.no_varlen:
        from workloads import VARLEN

        vr = VarlenRunner(VARLEN, dev)
        steps = max(5, min(args.steps, 30))
        m = vr.time(steps, 3)
        a = vr.algorithmic_flops()
        line["varlen"] = {"workload": VARLEN["name"], "lengths": vr.lengths, "ms": round(m, 4), "steps": steps,
                          "algorithmic_tflops": round(a / (m * 1e-3) / 1e12, 2),
                          "frac_of_bf16_peak": round(a / (m * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del vr

    if not args.no_fp8:
        # fp8 forms of the long workloads (same shapes, masks and key lengths)
        fp8 = {}
        for wid in (4, 5):
            ww = WORKLOADS[wid]
            fr = Fp8Runner(ww, dev)
            steps = max(10, min(args.steps, 50))
            m = fr.time(steps, 3)
            a = algorithmic_flops(ww, fr.key_lens_host)
            fp8[str(wid)] = {"workload": ww.name.replace("bf16", "fp8 e4m3"), "ms": round(m, 4), "steps": steps,
                             "algorithmic_tflops": round(a / (m * 1e-3) / 1e12, 2),
                             "frac_of_fp8_peak": round(a / (m * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)}
            del fr
        line["fp8"] = fp8

    if not args.no_splitkv:
        from workloads import SPLITKV

        res = {"workload": SPLITKV["name"]}
        for splits in (1, SPLITKV["splits"]):
            sr = SplitKVRunner(SPLITKV, dev, splits=splits)
            steps = max(10, min(args.steps, 50))
            m = sr.time(steps, 3)
            a = sr.algorithmic_flops()
            res["one_range" if splits == 1 else f"{splits}_ranges"] = {
                "ms": round(m, 4), "steps": steps, "algorithmic_tflops": round(a / (m * 1e-3) / 1e12, 2),
                "frac_of_bf16_peak": round(a / (m * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
            del sr
        line["splitkv"] = res

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)

    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
