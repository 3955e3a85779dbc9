#!/usr/bin/env python3
"""Forward-pass throughput of the MI355X GPT-2 library.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload small]

One step = one gpt2_forward (encoder, 12 blocks, final LayerNorm, logits GEMM,
vocabulary softmax) over one batch of synthetic tokens, with weights, tokens,
workspace and outputs already resident in HBM. Prints ONE JSON line.

Besides the end-to-end rate it times every kernel of one forward with HIP
events (the same launches gpt2_forward makes, issued one entry at a time on
the same stream) to report the dominant kernel against its roofline, and it
times the CPU oracle on a bounded sample of the same workload.
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

import numpy as np  # noqa: E402

PEAK = {  # MI355X published peaks
    "hbm_GBps": 8000.0,
    "f32_mfma_TFLOPs": 157.3,
    "bf16_mfma_TFLOPs": 2500.0,
}
METRIC = "fwd tokens/s GPT-2 124M B4 T1024; MFMA util % GEMM/attn; HBM GB/s elementwise"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="small",
                    help="small (fp32 B4 T1024, default), small_bf16_b4, small_bf16_b8, medium, decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=192)
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--profile-kernel", action="store_true",
                    help="counter-collection mode: launch only the logits GEMM (3x) and a "
                         "256 MiB device copy (calibration), print their names and sizes")
    return ap.parse_args()


class Bench:
    def __init__(self, w):
        import torch
        import transformer_forward_pass_gpt_amd as G
        from transformer_forward_pass_gpt_amd import inputs as I
        self.torch, self.G, self.I, self.w = torch, G, I, w
        G.load_library()
        self.es = 2 if w.dtype == I.BF16 else 4
        self.tdtype = torch.bfloat16 if w.dtype == I.BF16 else torch.float32
        self.cfg = G.make_config(w.L, w.C, w.NH, w.V, w.Vp, w.maxT, w.dtype, w.ln_eps)
        params = I.make_params(w)
        self.params_np = params
        if w.dtype == I.BF16:
            self.params = torch.from_numpy(I.to_bf16_bits(params).view(np.int16)).cuda().view(torch.bfloat16)
        else:
            self.params = torch.from_numpy(params).cuda()
        self.tokens_np = I.make_tokens(w)
        self.tokens = torch.from_numpy(self.tokens_np).cuda()
        B, T = w.B, w.T
        self.logits = torch.empty((B, T, w.Vp), dtype=self.tdtype, device="cuda")
        self.probs = torch.empty_like(self.logits)
        self.ws = torch.empty(G.workspace_bytes(self.cfg, B, T), dtype=torch.uint8, device="cuda")

    def step(self):
        self.G.gpt2_forward(self.logits, self.probs, self.tokens, self.params, self.cfg, self.ws)

    # ------------------------------------------------------------ per-kernel timing
    def kernel_timing(self, reps=3):
        """Issue one forward entry by entry, HIP events around each launch on
        the current stream; returns per-launch records (median over reps)."""
        torch, G, I, w = self.torch, self.G, self.I, self.w
        B, T, C, L, NH = w.B, w.T, w.C, w.L, w.NH
        N = B * T
        es = self.es
        offs = I.param_offsets(L, C, w.maxT, w.Vp)

        def P(name, l=None):
            o, shp = offs[name]
            n = int(np.prod(shp))
            t = self.params[o:o + n].view(*shp)
            return t if l is None else t[l]

        mk = lambda *s: torch.empty(s, dtype=self.tdtype, device="cuda")  # noqa: E731
        x, ln, qkv, att, tmp, fc = mk(N, C), mk(N, C), mk(N, 3 * C), mk(N, C), mk(N, C), mk(N, 4 * C)
        logits = self.logits.view(N, w.Vp)
        probs = self.probs.view(N, w.Vp)
        s = torch.cuda.current_stream()
        recs = []

        def timed(kind, name, fn, flops=0.0, nbytes=0.0, site=None):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            fn()
            b.record(s)
            recs.append([kind, name, flops, nbytes, a, b, site or name])

        # GEMM launches are named by the kernel configuration the library picks
        gemm = lambda out, inp, wt, bias, M, K, Nc, Nalg, tag: timed(  # noqa: E731
            "gemm", G.matmul_kernel_config(M, K, Nc, w.dtype),
            lambda: G.matmul_forward(out, inp, wt, bias), 2.0 * M * Nalg * K, 0.0, "gemm_" + tag)
        all_runs = []
        for _ in range(reps):
            recs.clear()
            timed("hbm", "encoder", lambda: G.encoder_forward(x.view(B, T, C), self.tokens, P("wte"), P("wpe")),
                  0.0, 4 * N + 2 * N * C * es + T * C * es)
            for l in range(L):
                timed("hbm", "layernorm", lambda: G.layernorm_forward(ln, x, P("ln1_g", l), P("ln1_b", l), w.ln_eps),
                      0.0, 2 * N * C * es + 2 * C * es)
                gemm(qkv, ln, P("qkv_w", l), P("qkv_b", l), N, C, 3 * C, 3 * C, "qkv")
                timed("mfma", "attention", lambda: G.attention_forward(att.view(B, T, C), qkv.view(B, T, 3 * C), NH),
                      4.0 * B * NH * (C // NH) * T * (T + 1) / 2, 0.0)
                gemm(tmp, att, P("attproj_w", l), P("attproj_b", l), N, C, C, C, "attproj")
                timed("hbm", "residual", lambda: G.residual_forward(x, x, tmp), 0.0, 3 * N * C * es)
                timed("hbm", "layernorm", lambda: G.layernorm_forward(ln, x, P("ln2_g", l), P("ln2_b", l), w.ln_eps),
                      0.0, 2 * N * C * es + 2 * C * es)
                gemm(fc, ln, P("fc_w", l), P("fc_b", l), N, C, 4 * C, 4 * C, "fc")
                timed("hbm", "gelu", lambda: G.gelu_forward(fc, fc), 0.0, 2 * N * 4 * C * es)
                gemm(tmp, fc, P("fcproj_w", l), P("fcproj_b", l), N, 4 * C, C, C, "fcproj")
                timed("hbm", "residual", lambda: G.residual_forward(x, x, tmp), 0.0, 3 * N * C * es)
            timed("hbm", "layernorm", lambda: G.layernorm_forward(ln, x, P("lnf_g"), P("lnf_b"), w.ln_eps),
                  0.0, 2 * N * C * es + 2 * C * es)
            gemm(logits, ln, P("wte"), None, N, C, w.Vp, w.V, "logits")
            timed("hbm", "softmax", lambda: G.softmax_forward(probs, logits, w.V), 0.0,
                  N * w.V * es + N * w.Vp * es)
            torch.cuda.synchronize()
            all_runs.append([r[:4] + [r[4].elapsed_time(r[5]), r[6]] for r in recs])
        out = []
        for i in range(len(all_runs[0])):
            ms = float(np.median([run[i][4] for run in all_runs]))
            out.append(all_runs[0][i][:4] + [ms, all_runs[0][i][5]])
        return out


def summarize_kernels(recs, dtype_bf16, key=1):
    """Group launch records by kernel name (key=1) or by call site (key=5)."""
    groups = {}
    for r in recs:
        kind, fl, nb, ms = r[0], r[2], r[3], r[4]
        name = r[key]
        g = groups.setdefault(name, {"kind": kind, "calls": 0, "ms": 0.0, "flops": 0.0, "bytes": 0.0})
        g["calls"] += 1
        g["ms"] += ms
        g["flops"] += fl
        g["bytes"] += nb
    mpeak = PEAK["bf16_mfma_TFLOPs"] if dtype_bf16 else PEAK["f32_mfma_TFLOPs"]
    table = {}
    for name, g in groups.items():
        sec = g["ms"] / 1e3
        row = {"calls": g["calls"], "total_ms": round(g["ms"], 4), "avg_us": round(g["ms"] / g["calls"] * 1e3, 2)}
        if g["kind"] in ("gemm", "mfma"):
            tf = g["flops"] / sec / 1e12
            row.update({"TFLOPs": round(tf, 2), "frac_peak": round(tf / mpeak, 4)})
        else:
            gbs = g["bytes"] / sec / 1e9
            row.update({"GBps": round(gbs, 1), "frac_peak": round(gbs / PEAK["hbm_GBps"], 4)})
        table[name] = row
    dom = max(groups, key=lambda k: groups[k]["ms"])
    g = groups[dom]
    per_launch_s = g["ms"] / g["calls"] / 1e3
    if g["kind"] in ("gemm", "mfma"):
        roof = {"bound": "mfma", "kernel": dom, "achieved": round(g["flops"] / g["calls"] / per_launch_s / 1e12, 3),
                "peak": mpeak, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "kernel": dom, "achieved": round(g["bytes"] / g["calls"] / per_launch_s / 1e9, 1),
                "peak": PEAK["hbm_GBps"], "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["avg_launch_us"] = round(per_launch_s * 1e6, 2)
    roof["launches_per_step"] = g["calls"]
    roof["traffic"] = load_traffic(dom)
    return table, roof


def load_traffic(kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None if
    there is none for this kernel or its source changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
        ent = data.get(kernel)
        if not ent:
            return None
        if ent.get("source_sha1") != source_sha1():
            return None
        return ent.get("bytes_per_launch")
    except Exception:
        return None


def source_sha1():
    h = hashlib.sha1()
    csrc = os.path.join(ROOT, "transformer_forward_pass_gpt_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def profile_kernel(b):
    """Launch the vocabulary GEMM three times and one plain device-to-device
    copy of 256 MiB, for hardware-counter runs (rocprofv3 --pmc FETCH_SIZE /
    WRITE_SIZE): the copy reads and writes a known number of bytes, which
    calibrates the counters."""
    torch, G, I, w = b.torch, b.G, b.I, b.w
    N = w.B * w.T
    o, shp = I.param_offsets(w.L, w.C, w.maxT, w.Vp)["wte"]
    wte = b.params[o:o + int(np.prod(shp))].view(*shp)
    ln = torch.randn(N, w.C, device="cuda").to(b.tdtype)
    logits = b.logits.view(N, w.Vp)
    for _ in range(3):
        G.matmul_forward(logits, ln, wte, None)
    src = torch.ones(64 << 20, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"gemm_kernel": G.matmul_kernel_config(N, w.C, w.Vp, w.dtype),
                      "gemm_shape": [N, w.C, w.Vp], "copy_bytes_each_way": 256 << 20}))


def cpu_baseline(b, ntok):
    """The oracle, single-threaded, on the first ntok positions of sequence 0
    (by the causal invariant, exactly those positions of the full workload)."""
    import oracle
    w = b.w
    tok = b.tokens_np[:1, :ntok]
    t0 = time.perf_counter()
    oracle.forward(tok, b.params_np, w.L, w.C, w.NH, w.V, w.Vp, w.maxT, w.ln_eps)
    dt = time.perf_counter() - t0
    return {"value": round(ntok / dt, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "sequence 0, positions 0..%d of the same workload (%d tokens, %.1f s, "
                      "single-threaded C oracle)" % (ntok - 1, ntok, dt)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; --gpus %d is not supported "
              "(data parallelism over sequences needs no collective, see the design notes)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    from transformer_forward_pass_gpt_amd import inputs as I
    w = I.WORKLOADS[args.workload]
    if w.decode_pos >= 0:
        raise SystemExit("decode workload: use bench_decode (not yet wired)")
    torch.cuda.set_device(0)
    b = Bench(w)
    if args.profile_kernel:
        profile_kernel(b)
        return
    for _ in range(args.warmup):
        b.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        b.step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = dt / args.steps * 1e3
    tokens = w.B * w.T
    res = {
        "metric": METRIC,
        "value": round(tokens * args.steps / dt, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == I.BF16 else "f32",
        "data": "synthetic (seeded uniform tokens, N(0,0.02) weights)",
        "config": {"workload": "GPT-2 %s %s forward B%d T%d (logits + softmax)" % (
            "124M" if w.C == 768 else "350M", "bf16" if w.dtype == I.BF16 else "fp32", w.B, w.T),
            "B": w.B, "T": w.T, "L": w.L, "C": w.C, "NH": w.NH, "V": w.V, "Vp": w.Vp},
    }
    if not args.no_kernel_timing:
        recs = b.kernel_timing()
        table, roof = summarize_kernels(recs, w.dtype == I.BF16)
        sites, _ = summarize_kernels(recs, w.dtype == I.BF16, key=5)
        res["roofline"] = roof
        res["kernels"] = table
        res["sites"] = sites
        res["kernel_sum_ms"] = round(sum(r[4] for r in recs), 4)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(b, args.cpu_sample_tokens)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
