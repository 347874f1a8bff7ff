#!/usr/bin/env python3
"""Benchmark of the exact tiled attention forward pass on one MI355X.

One step = one forward pass (the whole hot path: Q tile load, K/V tile stream,
QKᵀ, masks, online softmax, P·V, epilogue) over one batch of a named
synthetic workload, launched through the C ABI on torch's current stream with
the inputs already resident in HBM.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 5]
                    [--repeats 5] [--no-cpu-baseline] [--no-extra] ...

The headline is the grouped-query padded workload (B=2, 32 query heads over 8
kv heads, N=8192, d=128, bf16, key lengths uniform on N/2..N): the largest
algorithmic work of the five workloads.  value = 4·B·H·N²·d / time (TFLOP/s,
the metric as written); the roofline entry uses the algorithmic count (padded:
N·Σkey_len pairs; causal: N(N+1)/2 pairs per head).  Time per step is the
median over ``--repeats`` timed regions of exactly ``--steps`` back-to-back
launches each, bracketed by HIP events on the launch stream.  The other four
workloads are timed the same way (each region at least ~25 ms) and reported
under "workloads", with the fraction of the bf16 MFMA peak (fp32 matrix peak
for the fp32 workload) and the HBM rate of the committed rocprofv3 traffic
counters against 8 TB/s.
"""

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (4·B·H·N²·d) and % of bf16 MFMA peak, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix, published
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
HEADLINE = 5
MIN_REGION_MS = 25.0        # each timed region of a non-headline measurement lasts at least this long


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


def peak_of(w):
    return PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS


# the sources that decide what the forward kernels do and how they are launched
FORWARD_SOURCES = ("attn_api.hip", "attn_common.h", "attn_fwd_bf16.hip", "attn_fwd_f32.hip")


def kernel_source_hash():
    h = hashlib.sha256()
    for name in FORWARD_SOURCES:
        with open(os.path.join(ROOT, "exact_tiled_attention_14_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def _stored(fname, workload_id):
    """Entry of a committed rocprofv3 summary for this workload, or None when
    absent or taken on another version of the kernels."""
    try:
        with open(os.path.join(ROOT, "profiles", fname)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("workloads", {}).get(str(workload_id))


def stored_traffic(workload_id):
    """HBM bytes per launch (FETCH_SIZE and WRITE_SIZE, calibrated on a copy kernel)."""
    ent = _stored("hbm_traffic.json", workload_id)
    return None if ent is None else ent.get("bytes_per_launch")


def stored_mfma_util(workload_id):
    """Matrix-core busy fraction and effective shader clock (SQ_VALU_MFMA_BUSY_CYCLES,
    SQ_BUSY_CYCLES)."""
    ent = _stored("mfma_util.json", workload_id)
    return None if ent is None else {"mfma_busy": ent["mfma_busy"], "clock_ghz": ent["clock_ghz"]}


def hbm_entry(traffic, ms, alg_bytes):
    """HBM rates of one launch against the 8 TB/s peak: from the counted traffic
    (when stored for this kernel version) and from the compulsory bytes."""
    s = ms * 1e-3
    out = {"algorithmic_bytes": alg_bytes, "algorithmic_gbs": round(alg_bytes / s / 1e9, 1),
           "traffic_bytes": traffic, "traffic_gbs": None, "peak_gbs": PEAK_HBM_GBS, "traffic_frac": None}
    if traffic is not None:
        out["traffic_gbs"] = round(traffic / s / 1e9, 1)
        out["traffic_frac"] = round(traffic / s / 1e9 / PEAK_HBM_GBS, 4)
    return out


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

    def outputs(self, heads, rows=None):
        """GPU O and LSE of the given (b, h) heads (all rows, or the given ones), on the CPU."""
        outs = []
        for b, h in heads:
            o = self.o[b, h] if rows is None else self.o[b, h, rows]
            l_ = self.lse[b, h] if rows is None else self.lse[b, h, rows]
            outs.append((o.cpu(), l_.cpu()))
        return outs

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

    def region(self, steps, fn):
        """Milliseconds per launch over one timed region of `steps`
        back-to-back launches, bracketed by HIP events recorded on the launch
        stream (the device is idle on both sides)."""
        import torch

        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(self.stream)
        for _ in range(steps):
            fn()
        end.record(self.stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    def time(self, steps, warmup, repeats=5, fn=None, min_region_ms=0.0):
        """Median milliseconds per launch over `repeats` timed regions.

        Each region holds exactly `steps` launches, raised (for the secondary
        measurements, min_region_ms > 0) until one region lasts at least
        min_region_ms.  Returns (median ms, steps per region, all region ms)."""
        fn = fn or self.launch
        for _ in range(warmup):
            fn()
        if min_region_ms > 0:
            probe = self.region(max(1, min(steps, 5)), fn)
            steps = max(steps, min(5000, int(math.ceil(min_region_ms / max(probe, 1e-4)))))
        ms = [self.region(steps, fn) for _ in range(repeats)]
        return statistics.median(ms), steps, ms


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


class Fp8PrepRunner(Runner):
    """The fp8 preparation of a workload's bf16 q, k, v on the GPU, as one
    step: amax and rotated quantisation of q and of k (one random-sign
    Hadamard rotation for both), amax and transposed quantisation of V (six
    C-ABI calls, nine kernels, no host synchronisation in between)."""

    def __init__(self, w, dev):
        import torch

        import exact_tiled_attention_14_amd as attn
        from workloads import make_inputs

        self.w = w
        q, k, v, _ = make_inputs(w)
        self.q, self.k, self.v = q.to(dev), k.to(dev), v.to(dev)
        self.signs = attn.hadamard_signs(w.d, seed=w.seed, device=dev)
        self.q8 = torch.empty(self.q.shape, dtype=torch.float8_e4m3fn, device=dev)
        self.k8 = torch.empty(self.k.shape, dtype=torch.float8_e4m3fn, device=dev)
        self.n16 = (w.N + 15) // 16 * 16
        self.vt8 = torch.empty((w.B, w.Hkv, w.d, self.n16), dtype=torch.float8_e4m3fn, device=dev)
        self.scal = torch.zeros(3 * 8, dtype=torch.float32, device=dev)
        self.stream = torch.cuda.current_stream(dev)
        self.attn = attn

    def launch(self):
        a, w, st, sp = self.attn, self.w, self.stream.cuda_stream, self.signs.data_ptr()
        rq, rk = w.B * w.H * w.N, w.B * w.Hkv * w.N
        sc = [self.scal[8 * i:].data_ptr() for i in range(3)]
        ds = [self.scal[8 * i + 4:].data_ptr() for i in range(3)]
        codes = (a.attn_fp8_amax(self.q.data_ptr(), sp, rq, w.d, sc[0], st),
                 a.attn_fp8_quantize(self.q.data_ptr(), sp, rq, w.d, sc[0], self.q8.data_ptr(), ds[0], st),
                 a.attn_fp8_amax(self.k.data_ptr(), sp, rk, w.d, sc[1], st),
                 a.attn_fp8_quantize(self.k.data_ptr(), sp, rk, w.d, sc[1], self.k8.data_ptr(), ds[1], st),
                 a.attn_fp8_amax(self.v.data_ptr(), None, rk, w.d, sc[2], st),
                 a.attn_fp8_quantize_vt(self.v.data_ptr(), w.B * w.Hkv, w.N, w.d, sc[2], self.vt8.data_ptr(), ds[2],
                                        st))
        if any(c != 0 for c in codes):
            raise RuntimeError(f"fp8 preparation failed with status {codes}")

    def bytes(self):
        """(compulsory bytes: every bf16 input read once and every fp8 byte
        written once; bytes of the two passes: the inputs read twice)."""
        w = self.w
        n_in = (w.B * w.H + 2 * w.B * w.Hkv) * w.N * w.d
        n_out = (w.B * w.H + w.B * w.Hkv) * w.N * w.d + w.B * w.Hkv * w.d * self.n16
        return 2 * n_in + n_out, 4 * n_in + n_out


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
    its workspace; splits=1 times the same problem as one key range."""

    def __init__(self, spec, dev, splits=None):
        import torch

        import exact_tiled_attention_14_amd as attn
        from workloads import make_splitkv

        self.spec = spec
        s = spec
        q, k, v = make_splitkv(s)
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


def host_cores():
    """Cores this process may run on (the affinity mask, not the machine's count)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(w, wid, gpu_heads, parity_samples, budget_s=15.0):
    """The fp64 oracle, as it stands, on this host's cores.

    Timing: whole (b, h) heads of the headline workload (all query rows, keys
    cut at the sequence's key length), in order, until about ``budget_s``
    seconds are spent, with the BLAS pool set to every core of the affinity
    mask.  Reported in the metric's unit (TFLOP/s of the nominal 4·N²·d count
    per head).

    The heads it computes are also compared with the GPU's output for them
    (``gpu_heads``: {(b, h): (o, lse)} read back after the timed runs), and
    ``parity_samples`` ({workload id: (workload, inputs, rows, heads, gpu
    outputs)}) adds a bounded row sample of every other workload: max |ΔO|
    and |ΔLSE| per workload against the oracle, the quantities the tests
    bound.  Returns (baseline entry, parity entry)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from workloads import as_f64, make_inputs

    cores = host_cores()
    tol_o = {"bf16": 1.5e-2, "f32": 1e-5}

    def errors(o_g, l_g, O, L):
        fin = np.isfinite(L)
        el = float(np.max(np.abs(as_f64(l_g)[fin] - L[fin]))) if fin.any() else 0.0
        return float(np.max(np.abs(as_f64(o_g) - O))), el

    def entry(ww, what, eo, el):
        return {"rows": what, "max_abs_dO": eo, "max_abs_dLSE": el, "tol_O": tol_o[ww.dtype], "tol_LSE": 1e-3,
                "ok": bool(eo <= tol_o[ww.dtype] and el <= 1e-3)}

    q, k, v, kl = make_inputs(w)
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    group = w.H // w.Hkv
    order = [(b, h) for b in range(w.B) for h in range(w.H)]
    checked = 0
    err_o = err_l = 0.0
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        heads = 0
        while time.perf_counter() - t0 < budget_s:
            b, h = order[heads % len(order)]
            g = h // group
            O, L = oracle.attention(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1], w.scale,
                                    causal=w.causal, key_lens=None if kl is None else [int(kl[b])])
            if heads < len(order) and (b, h) in gpu_heads:
                eo, el = errors(*gpu_heads[(b, h)], O[0, 0], L[0, 0])
                err_o, err_l = max(err_o, eo), max(err_l, el)
                checked += 1
            heads += 1
        dt = time.perf_counter() - t0
        parity = {str(wid): entry(w, f"{checked} whole heads x {w.N} rows", err_o, err_l)}
        for sid, (ww, inputs, rows, hs, outs) in sorted(parity_samples.items()):
            sq, sk, sv, skl = inputs
            sq, sk, sv = as_f64(sq), as_f64(sk), as_f64(sv)
            eo = el = 0.0
            for (b, h), (o_g, l_g) in zip(hs, outs):
                g = h // (ww.H // ww.Hkv)
                O, L = oracle.attention(sq[b:b + 1, h:h + 1], sk[b:b + 1, g:g + 1], sv[b:b + 1, g:g + 1], ww.scale,
                                        causal=ww.causal, key_lens=None if skl is None else [int(skl[b])],
                                        rows=rows)
                e1, e2 = errors(o_g, l_g, O[0, 0], L[0, 0])
                eo, el = max(eo, e1), max(el, e2)
            parity[str(sid)] = entry(ww, f"{len(hs)} heads x {len(rows)} rows", eo, el)
    flops = 4.0 * heads * w.N * w.N * w.d
    base = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{heads} whole (b,h) heads of the {w.B * w.H}-head workload '{w.name}', all {w.N} query "
                      f"rows each against the sequence's keys, fp64 numpy with {cores} BLAS threads, "
                      f"{dt:.1f} s wall",
            "seconds": round(dt, 2)}
    return base, parity


def parity_rows(N, n=96, seed=0):
    """Rows checked by the bench's parity sample: both ends, tile edges and random rows."""
    import numpy as np

    fixed = {0, 1, 127, 128, 255, 256, N // 2, N - 129, N - 2, N - 1}
    rng = np.random.default_rng(seed)
    rnd = set(rng.choice(N, size=min(n, N), replace=False).tolist())
    return np.array(sorted(r for r in fixed | rnd if 0 <= r < N))


def rate(flops, ms):
    return flops / (ms * 1e-3) / 1e12


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--repeats", type=int, default=5, help="timed regions per measurement (median reported)")
    ap.add_argument("--workload", type=int, default=HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip timing the other workloads")
    ap.add_argument("--no-backward", action="store_true", help="skip timing the backward pass")
    ap.add_argument("--no-varlen", action="store_true", help="skip timing the packed variable-length batch")
    ap.add_argument("--no-splitkv", action="store_true", help="skip timing the split-KV shape")
    ap.add_argument("--no-fp8", action="store_true", help="skip timing the fp8 forward")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 3 device-to-device copies of MIB MiB (a plain copy kernel of known "
                         "traffic, to calibrate the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): this build runs on a single "
              "MI355X and has no multi-GPU path; run with --gpus 1", file=sys.stderr)
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
    want_parity = not args.no_cpu_baseline

    r = Runner(w, dev)
    ms, steps, all_ms = r.time(args.steps, args.warmup, args.repeats)
    nom = nominal_flops(w)
    alg = algorithmic_flops(w, r.key_lens_host)
    peak = peak_of(w)
    achieved = rate(alg, ms)
    traffic = stored_traffic(args.workload)
    gpu_heads = {}
    if want_parity:
        heads = [(b, h) for b in range(w.B) for h in range(w.H)][:24]
        gpu_heads = dict(zip(heads, r.outputs(heads)))
    del r

    line = {
        "metric": METRIC,
        "value": round(rate(nom, ms), 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded i.i.d. N(0,1) q/k/v, key lengths uniform on N/2..N; no dataset)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "causal": w.causal, "padded": w.padded, "scale": w.scale},
        "timing": {"repeats": args.repeats, "steps_per_region": steps, "region_ms_per_step": [round(x, 5)
                                                                                               for x in all_ms],
                   "statistic": "median of the regions"},
        "frac_of_bf16_peak": round(achieved / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "algorithmic_flops": alg,
                     "hbm": hbm_entry(traffic, ms, algorithmic_bytes(w)),
                     "counters": stored_mfma_util(args.workload)},
    }

    parity_samples = {}
    if not args.no_extra:
        extra = {}
        for wid in sorted(WORKLOADS):
            if wid == args.workload:
                continue
            ww = WORKLOADS[wid]
            rr = Runner(ww, dev)
            m, st, allm = rr.time(args.steps, max(3, args.warmup // 2), args.repeats, min_region_ms=MIN_REGION_MS)
            a = algorithmic_flops(ww, rr.key_lens_host)
            pk = peak_of(ww)
            tr = stored_traffic(wid)
            extra[str(wid)] = {
                "workload": ww.name, "ms": round(m, 5), "steps_per_region": st, "repeats": args.repeats,
                "region_ms": [round(x, 5) for x in allm],
                "nominal_tflops": round(rate(nominal_flops(ww), m), 2),
                "algorithmic_tflops": round(rate(a, m), 2),
                "peak_tflops": pk,
                "frac_of_peak": round(rate(a, m) / pk, 4),
                "peak_kind": "bf16 MFMA" if ww.dtype == "bf16" else "fp32 matrix",
                "hbm": hbm_entry(tr, m, algorithmic_bytes(ww)),
                "counters": stored_mfma_util(wid),
            }
            if want_parity:
                from workloads import make_inputs

                rows = parity_rows(ww.N, seed=wid)
                hs = [(0, 0), (ww.B - 1, ww.H - 1)]
                parity_samples[wid] = (ww, make_inputs(ww), rows, hs, rr.outputs(hs, rows=torch.as_tensor(rows)))
            del rr
        line["workloads"] = extra

    if not args.no_backward:
        # backward pass (dq, dk, dv): algorithmic flops = 2.5 x the forward's
        # (five products per admissible (query, key) pair instead of two)
        bwd = {}
        for wid in sorted(WORKLOADS):
            ww = WORKLOADS[wid]
            if ww.dtype != "bf16":
                continue
            rr = Runner(ww, dev)
            rr.prepare_backward()
            m, st, _ = rr.time(max(5, min(args.steps, 30)), 3, args.repeats, fn=rr.launch_backward,
                               min_region_ms=MIN_REGION_MS)
            a = 2.5 * algorithmic_flops(ww, rr.key_lens_host)
            bwd[str(wid)] = {"workload": ww.name, "ms": round(m, 4), "steps_per_region": st,
                             "algorithmic_tflops": round(rate(a, m), 2),
                             "frac_of_bf16_peak": round(rate(a, m) / PEAK_BF16_TFLOPS, 4)}
            del rr
        line["backward"] = bwd

    if not args.no_varlen:
        from workloads import VARLEN

        vr = VarlenRunner(VARLEN, dev)
        m, st, _ = vr.time(max(5, min(args.steps, 30)), 3, args.repeats, min_region_ms=MIN_REGION_MS)
        a = vr.algorithmic_flops()
        line["varlen"] = {"workload": VARLEN["name"], "lengths": vr.lengths, "ms": round(m, 4),
                          "steps_per_region": st, "algorithmic_tflops": round(rate(a, m), 2),
                          "frac_of_bf16_peak": round(rate(a, m) / PEAK_BF16_TFLOPS, 4)}
        del vr

    if not args.no_fp8:
        # fp8 forms of the long workloads (same shapes, masks and key lengths)
        fp8 = {}
        for wid in (4, 5):
            ww = WORKLOADS[wid]
            fr = Fp8Runner(ww, dev)
            m, st, _ = fr.time(max(10, min(args.steps, 50)), 3, args.repeats, min_region_ms=MIN_REGION_MS)
            a = algorithmic_flops(ww, fr.key_lens_host)
            fp8[str(wid)] = {"workload": ww.name.replace("bf16", "fp8 e4m3"), "ms": round(m, 4),
                             "steps_per_region": st, "algorithmic_tflops": round(rate(a, m), 2),
                             "frac_of_fp8_peak": round(rate(a, m) / PEAK_FP8_TFLOPS, 4)}
            del fr
            # the preparation (incoherent-processing rotation and quantisation) of the
            # same shape's bf16 inputs: HBM-bound, against 8 TB/s
            pr = Fp8PrepRunner(ww, dev)
            m, st, _ = pr.time(max(10, min(args.steps, 50)), 3, args.repeats, min_region_ms=MIN_REGION_MS)
            compulsory, passes = pr.bytes()
            fp8[str(wid)]["prep"] = {
                "what": ("rotate + amax + quantise q and k, amax + transposed quantise of v "
                         "(6 C-ABI calls, 9 kernels)"),
                "ms": round(m, 4), "steps_per_region": st,
                "compulsory_bytes": compulsory, "compulsory_gbs": round(compulsory / (m * 1e-3) / 1e9, 1),
                "two_pass_bytes": passes, "two_pass_gbs": round(passes / (m * 1e-3) / 1e9, 1),
                "frac_of_hbm_peak": round(passes / (m * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
            del pr
        line["fp8"] = fp8

    if not args.no_splitkv:
        from workloads import SPLITKV

        res = {"workload": SPLITKV["name"]}
        for splits in (1, SPLITKV["splits"]):
            sr = SplitKVRunner(SPLITKV, dev, splits=splits)
            m, st, _ = sr.time(max(10, min(args.steps, 50)), 3, args.repeats, min_region_ms=MIN_REGION_MS)
            a = sr.algorithmic_flops()
            res["one_range" if splits == 1 else f"{splits}_ranges"] = {
                "ms": round(m, 4), "steps_per_region": st, "algorithmic_tflops": round(rate(a, m), 2),
                "frac_of_bf16_peak": round(rate(a, m) / PEAK_BF16_TFLOPS, 4)}
            del sr
        line["splitkv"] = res

    if want_parity:
        base, parity = cpu_baseline(w, args.workload, gpu_heads, parity_samples)
        line["cpu_baseline"] = base
        line["parity"] = parity

    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
