#!/usr/bin/env python3
"""Forward-pass throughput of the MI355X GPT-2 library.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload small]

One step = one gpt2_forward (encoder, 12 blocks with GELU and the residual
adds fused into the GEMM epilogues, final LayerNorm, logits GEMM, vocabulary
softmax) over one batch of synthetic tokens, with weights, tokens,
workspace and outputs already resident in HBM. Prints ONE JSON line. With
``--workload decode`` a step is one gpt2_decode_step instead: one new token
for each of 32 sequences against a prefilled key/value cache. With ``--mode train`` a step is
one training step without the optimizer: gpt2_train_forward (forward keeping
activations, losses and the logit gradient) then gpt2_backward (every
parameter gradient).

Besides the end-to-end rate it times every kernel of one forward with HIP
events (the same launches gpt2_forward makes, issued one entry at a time on
the same stream, one event between consecutive launches; for the decode step,
whose kernels are shorter than a host launch, queued behind a GPU spin so they
run back to back) to report the dominant kernel against its roofline, and it
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
    ap.add_argument("--mode", default="forward", choices=["forward", "train"],
                    help="train: one step = gpt2_train_forward + gpt2_backward (losses, the logit gradient "
                         "and every parameter gradient; no optimizer)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=192)
    ap.add_argument("--cpu-sample-train-tokens", type=int, default=16,
                    help="train mode: positions of sequence 0 the CPU oracle's training step runs on")
    ap.add_argument("--cpu-sample-seqs", type=int, default=32,
                    help="decode workload: sequences the CPU oracle steps")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--elementwise", action="store_true",
                    help="time the standalone gelu_forward and residual_forward entries (which the forward "
                         "fuses into GEMM epilogues) on this workload's shapes, each launch after a cache "
                         "flush; prints their own JSON line")
    ap.add_argument("--profile-kernel", action="store_true",
                    help="counter-collection mode: launch only the dominant kernel (3x: the logits "
                         "GEMM, or the decode attention) and a 256 MiB device copy (calibration)")
    ap.add_argument("--profile-target", default="vocab",
                    choices=["vocab", "attention", "qkv", "attproj", "fc", "fcproj"],
                    help="with --profile-kernel on a prefill workload: which kernel to launch (the "
                         "vocabulary GEMM, the prefill attention, or one layer-0 projection with its "
                         "forward epilogue), on the workload's shapes")
    return ap.parse_args()


class Bench:
    def __init__(self, w, keep_host_cache=False, train=False):
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
        self.decode = w.decode_pos >= 0
        if self.decode:
            kc, vc = I.make_kv_cache(w)
            self.kcache, self.vcache = self.to_dev(kc), self.to_dev(vc)
            self.kc_np, self.vc_np = (kc, vc) if keep_host_cache else (None, None)
            del kc, vc
            self.logits = torch.empty((B, w.Vp), dtype=self.tdtype, device="cuda")
            ws = G.decode_workspace_bytes(self.cfg, B)
        else:
            self.logits = torch.empty((B, T, w.Vp), dtype=self.tdtype, device="cuda")
            ws = G.workspace_bytes(self.cfg, B, T)
        self.probs = torch.empty_like(self.logits)
        self.ws = torch.empty(ws, dtype=torch.uint8, device="cuda")
        self.train = train
        if train:
            self.targets_np = I.make_targets(w)
            self.targets = torch.from_numpy(self.targets_np).cuda()
            self.acts = torch.empty(G.train_acts_bytes(self.cfg, B, T), dtype=torch.uint8, device="cuda")
            self.tws = torch.empty(G.train_workspace_bytes(self.cfg, B, T), dtype=torch.uint8, device="cuda")
            self.grads = torch.empty_like(self.params)
            self.mean_loss = torch.empty(1, dtype=torch.float32, device="cuda")
            del self.probs, self.ws

    def to_dev(self, a):
        if self.w.dtype == self.I.BF16:
            bits = self.I.to_bf16_bits(a).view(np.int16)
            return self.torch.from_numpy(bits).cuda().view(self.torch.bfloat16)
        return self.torch.from_numpy(a).cuda()

    def step(self):
        if self.train:
            self.G.gpt2_train_forward(self.tokens, self.targets, self.params, self.cfg, self.acts, None,
                                      self.mean_loss)
            self.G.gpt2_backward(self.grads, self.tokens, self.params, self.cfg, self.acts, self.tws)
        elif self.decode:
            self.G.gpt2_decode_step(self.logits, self.probs, self.tokens, self.w.decode_pos, self.kcache,
                                    self.vcache, self.params, self.cfg, self.ws)
        else:
            self.G.gpt2_forward(self.logits, self.probs, self.tokens, self.params, self.cfg, self.ws)

    # ------------------------------------------------------------ per-kernel timing
    def gpu_hold(self, ms):
        """Queue a spin kernel that keeps the stream busy for about `ms`, so the
        launches enqueued behind it run back to back and the HIP events between
        them measure GPU time, not host launch gaps."""
        torch = self.torch
        if not hasattr(self, "_cycles_per_ms"):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(1000)
            a.record()
            torch.cuda._sleep(2_000_000)
            b.record()
            torch.cuda.synchronize()
            cpm = 2_000_000 / max(a.elapsed_time(b), 1e-6)
            # a counter between 10 MHz and 10 GHz; anything else: no hold
            self._cycles_per_ms = cpm if 1e4 <= cpm <= 1e7 else 0.0
        if self._cycles_per_ms:
            torch.cuda._sleep(int(min(ms, 200.0) * self._cycles_per_ms))

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
        x, ln, qkv, att, fc = mk(N, C), mk(N, C), mk(N, 3 * C), mk(N, C), mk(N, 4 * C)
        logits = self.logits.view(N, w.Vp)
        probs = self.probs.view(N, w.Vp)
        s = torch.cuda.current_stream()
        recs = []

        def timed(kind, name, fn, flops=0.0, nbytes=0.0, site=None):
            # consecutive launches share the event between them
            if not recs:
                a = torch.cuda.Event(enable_timing=True)
                a.record(s)
            else:
                a = recs[-1][5]
            fn()
            b = torch.cuda.Event(enable_timing=True)
            b.record(s)
            recs.append([kind, name, flops, nbytes, a, b, site or name])

        # GEMM launches are named by the kernel configuration the library picks
        # (plus the epilogue fused into it)
        def gemm(out, inp, wt, bias, M, K, Nc, Nalg, tag, epi=""):
            if epi == "residual":
                fn = lambda: G.matmul_residual_forward(out, inp, wt, bias, out)  # noqa: E731
            elif epi == "gelu":
                fn = lambda: G.matmul_gelu_forward(out, inp, wt, bias)  # noqa: E731
            else:
                fn = lambda: G.matmul_forward(out, inp, wt, bias)  # noqa: E731
            name = G.matmul_kernel_config(M, K, Nc, w.dtype) + ("+" + epi if epi else "")
            timed("gemm", name, fn, 2.0 * M * Nalg * K, 0.0, "gemm_" + tag + ("+" + epi if epi else ""))
        # Forward kernels run for tens of microseconds or more, longer than a
        # host launch, so the launches queue up by themselves; no GPU spin
        # (it costs the following kernels a few percent of clock).
        all_runs = []
        for _ in range(reps + 1):  # the first pass warms up and is dropped
            recs.clear()
            # a short spin ahead of the pass: the first launch is queued before
            # the first event fires, so it is not charged the host's launch time
            self.gpu_hold(0.1)
            timed("hbm", "encoder", lambda: G.encoder_forward(x.view(B, T, C), self.tokens, P("wte"), P("wpe")),
                  0.0, 4 * N + 2 * N * C * es + T * C * es)
            for l in range(L):
                timed("hbm", "layernorm", lambda: G.layernorm_forward(ln, x, P("ln1_g", l), P("ln1_b", l), w.ln_eps),
                      0.0, 2 * N * C * es + 2 * C * es)
                gemm(qkv, ln, P("qkv_w", l), P("qkv_b", l), N, C, 3 * C, 3 * C, "qkv")
                timed("mfma", "attention", lambda: G.attention_forward(att.view(B, T, C), qkv.view(B, T, 3 * C), NH),
                      4.0 * B * NH * (C // NH) * T * (T + 1) / 2, 0.0)
                gemm(x, att, P("attproj_w", l), P("attproj_b", l), N, C, C, C, "attproj", "residual")
                timed("hbm", "layernorm", lambda: G.layernorm_forward(ln, x, P("ln2_g", l), P("ln2_b", l), w.ln_eps),
                      0.0, 2 * N * C * es + 2 * C * es)
                gemm(fc, ln, P("fc_w", l), P("fc_b", l), N, C, 4 * C, 4 * C, "fc", "gelu")
                gemm(x, fc, P("fcproj_w", l), P("fcproj_b", l), N, 4 * C, C, C, "fcproj", "residual")
            timed("hbm", "layernorm", lambda: G.layernorm_forward(ln, x, P("lnf_g"), P("lnf_b"), w.ln_eps),
                  0.0, 2 * N * C * es + 2 * C * es)
            gemm(logits, ln, P("wte"), None, N, C, w.Vp, w.V, "logits")
            timed("hbm", "softmax", lambda: G.softmax_forward(probs, logits, w.V), 0.0,
                  N * w.V * es + N * w.Vp * es)
            torch.cuda.synchronize()
            all_runs.append([r[:4] + [r[4].elapsed_time(r[5]), r[6]] for r in recs])
        all_runs = all_runs[1:]
        out = []
        for i in range(len(all_runs[0])):
            ms = float(np.median([run[i][4] for run in all_runs]))
            out.append(all_runs[0][i][:4] + [ms, all_runs[0][i][5]])
        return out


    def train_kernel_timing(self, reps=2):
        """The entries of one training step (gpt2_train_forward, then
        gpt2_backward) issued one at a time with HIP events between them, with
        per-layer activation buffers as in the library (so every layer's
        operands are as cold as in the real step). A backward entry may run
        several kernels (the linear backward: operand transposes, two GEMMs,
        the bias reduction); its record is the whole entry, charged its
        algorithmic work: 4MNK for the linear backward (dinp and dW), the four
        products dV, dP, dQ, dK for attention (twice the forward's), bytes read
        and written once for the rest."""
        torch, G, I, w = self.torch, self.G, self.I, self.w
        B, T, C, L, NH, Vp, V = w.B, w.T, w.C, w.L, w.NH, w.Vp, w.V
        N = B * T
        es = self.es
        offs = I.param_offsets(L, C, w.maxT, Vp)

        def view(flat, name, l=None):
            o, shp = offs[name]
            t = flat[o:o + int(np.prod(shp))].view(*shp)
            return t if l is None else t[l]

        P = lambda n, l=None: view(self.params, n, l)  # noqa: E731
        D = lambda n, l=None: view(self.grads, n, l)  # noqa: E731
        mk = lambda *s: torch.empty(s, dtype=self.tdtype, device="cuda")  # noqa: E731
        f32 = lambda *s: torch.empty(s, dtype=torch.float32, device="cuda")  # noqa: E731
        acts = [dict(x=mk(N, C), ln1=mk(N, C), m1=f32(N), r1=f32(N), qkv=mk(N, 3 * C), att=mk(N, C),
                     lse=f32(B, NH, T), res1=mk(N, C), ln2=mk(N, C), m2=f32(N), r2=f32(N), fch=mk(N, 4 * C),
                     fchg=mk(N, 4 * C)) for _ in range(L)]
        xf, lnf, mf, rf = mk(N, C), mk(N, C), f32(N), f32(N)
        logits = self.logits.view(N, Vp)
        losses, mean = f32(N), f32(1)
        dres, dC, d4, dqkv = mk(N, C), mk(N, C), mk(N, 4 * C), mk(N, 3 * C)
        ws = torch.empty(G.train_workspace_bytes(self.cfg, B, T), dtype=torch.uint8, device="cuda")
        s = torch.cuda.current_stream()
        recs = []

        def timed(kind, name, fn, flops=0.0, nbytes=0.0, site=None):
            if not recs:
                a = torch.cuda.Event(enable_timing=True)
                a.record(s)
            else:
                a = recs[-1][5]
            fn()
            b = torch.cuda.Event(enable_timing=True)
            b.record(s)
            recs.append([kind, name, flops, nbytes, a, b, site or name])

        def gemm(out, inp, wt, bias, K, Nc, tag, res=None, Nalg=None):
            name = G.matmul_kernel_config(N, K, Nc, w.dtype) + ("+residual" if res is not None else "")
            fn = ((lambda: G.matmul_residual_forward(out, inp, wt, bias, res)) if res is not None
                  else (lambda: G.matmul_forward(out, inp, wt, bias)))
            timed("gemm", name, fn, 2.0 * N * (Nalg or Nc) * K, 0.0, "gemm_" + tag)

        def mmb(dinp, dw, db, dout, inp, wt, K, Nc, tag, Nalg=None):
            timed("gemm", "matmul_backward", lambda: G.matmul_backward(dinp, dw, db, dout, inp, wt, ws),
                  4.0 * N * (Nalg or Nc) * K, 0.0, "matmul_backward_" + tag)

        ln_bytes = 2 * N * C * es + 2 * C * es + 8 * N
        lnb_bytes = lambda res: (4 if res else 3) * N * C * es + C * es + 2 * C * es + 8 * N  # noqa: E731
        attn_flops = 4.0 * B * NH * (C // NH) * T * (T + 1) / 2
        all_runs = []
        for _ in range(reps + 1):  # the first pass warms up and is dropped
            recs.clear()
            self.gpu_hold(0.1)  # the first launch queues behind it (see kernel_timing)
            timed("hbm", "encoder", lambda: G.encoder_forward(acts[0]["x"].view(B, T, C), self.tokens, P("wte"),
                                                               P("wpe")), 0.0, 4 * N + 2 * N * C * es + T * C * es)
            for l in range(L):
                a = acts[l]
                xn = acts[l + 1]["x"] if l + 1 < L else xf
                timed("hbm", "layernorm", lambda: G.layernorm_forward(a["ln1"], a["x"], P("ln1_g", l), P("ln1_b", l),
                                                                       w.ln_eps, a["m1"], a["r1"]), 0.0, ln_bytes)
                gemm(a["qkv"], a["ln1"], P("qkv_w", l), P("qkv_b", l), C, 3 * C, "qkv")
                timed("mfma", "attention", lambda: G.attention_forward_lse(
                    a["att"].view(B, T, C), a["lse"], a["qkv"].view(B, T, 3 * C), NH), attn_flops, 0.0)
                gemm(a["res1"], a["att"], P("attproj_w", l), P("attproj_b", l), C, C, "attproj", res=a["x"])
                timed("hbm", "layernorm", lambda: G.layernorm_forward(a["ln2"], a["res1"], P("ln2_g", l),
                                                                       P("ln2_b", l), w.ln_eps, a["m2"], a["r2"]),
                      0.0, ln_bytes)
                gemm(a["fch"], a["ln2"], P("fc_w", l), P("fc_b", l), C, 4 * C, "fc")
                timed("hbm", "gelu", lambda: G.gelu_forward(a["fchg"], a["fch"]), 0.0, 2 * N * 4 * C * es)
                gemm(xn, a["fchg"], P("fcproj_w", l), P("fcproj_b", l), 4 * C, C, "fcproj", res=a["res1"])
            timed("hbm", "layernorm", lambda: G.layernorm_forward(lnf, xf, P("lnf_g"), P("lnf_b"), w.ln_eps, mf, rf),
                  0.0, ln_bytes)
            gemm(logits, lnf, P("wte"), None, C, Vp, "logits", Nalg=V)
            timed("hbm", "crossentropy_backward", lambda: G.crossentropy_backward(
                logits, logits, self.targets.view(N), V, 1.0 / N, losses, mean), 0.0, N * V * es + N * Vp * es)
            # backward
            mmb(dC, D("wte"), None, logits, lnf, P("wte"), C, Vp, "logits", Nalg=V)
            timed("hbm", "layernorm_backward", lambda: G.layernorm_backward(
                dres, D("lnf_g"), D("lnf_b"), dC, xf, P("lnf_g"), mf, rf, ws), 0.0, lnb_bytes(False))
            for l in reversed(range(L)):
                a = acts[l]
                mmb(d4, D("fcproj_w", l), D("fcproj_b", l), dres, a["fchg"], P("fcproj_w", l), 4 * C, C, "fcproj")
                timed("hbm", "gelu_backward", lambda: G.gelu_backward(d4, a["fch"], d4), 0.0, 3 * N * 4 * C * es)
                mmb(dC, D("fc_w", l), D("fc_b", l), d4, a["ln2"], P("fc_w", l), C, 4 * C, "fc")
                timed("hbm", "layernorm_backward", lambda: G.layernorm_backward(
                    dres, D("ln2_g", l), D("ln2_b", l), dC, a["res1"], P("ln2_g", l), a["m2"], a["r2"], ws, dres=dres),
                    0.0, lnb_bytes(True))
                mmb(dC, D("attproj_w", l), D("attproj_b", l), dres, a["att"], P("attproj_w", l), C, C, "attproj")
                timed("mfma", "attention_backward", lambda: G.attention_backward(
                    dqkv.view(B, T, 3 * C), dC.view(B, T, C), a["qkv"].view(B, T, 3 * C), a["att"].view(B, T, C),
                    a["lse"], NH, ws), 2.0 * attn_flops, 0.0)
                mmb(dC, D("qkv_w", l), D("qkv_b", l), dqkv, a["ln1"], P("qkv_w", l), C, 3 * C, "qkv")
                timed("hbm", "layernorm_backward", lambda: G.layernorm_backward(
                    dres, D("ln1_g", l), D("ln1_b", l), dC, a["x"], P("ln1_g", l), a["m1"], a["r1"], ws, dres=dres),
                    0.0, lnb_bytes(True))
            timed("hbm", "encoder_backward", lambda: G.encoder_backward(D("wte"), D("wpe"), dres.view(B, T, C),
                                                                         self.tokens), 0.0, 3 * N * C * es)
            torch.cuda.synchronize()
            all_runs.append([r[:4] + [r[4].elapsed_time(r[5]), r[6]] for r in recs])
        all_runs = all_runs[1:]
        out = []
        for i in range(len(all_runs[0])):
            ms = float(np.median([run[i][4] for run in all_runs]))
            out.append(all_runs[0][i][:4] + [ms, all_runs[0][i][5]])
        return out

    def decode_kernel_timing(self, reps=3):
        """The launches of one gpt2_decode_step (batches of at most 32
        sequences), entry by entry, HIP events around each. Every kernel of a
        decode step is bound by HBM (the GEMMs stream their weights once for
        32 rows), so each record carries the algorithmic bytes: operands read
        once, results written once."""
        torch, G, I, w = self.torch, self.G, self.I, self.w
        B, C, L, NH, pos = w.B, w.C, w.L, w.NH, w.decode_pos
        es = self.es
        offs = I.param_offsets(L, C, w.maxT, w.Vp)

        def P(name, l=None):
            o, shp = offs[name]
            n = int(np.prod(shp))
            t = self.params[o:o + n].view(*shp)
            return t if l is None else t[l]

        mk = lambda *s: torch.empty(s, dtype=self.tdtype, device="cuda")  # noqa: E731
        x, ln, qkv, att, fc = mk(B, C), mk(B, C), mk(B, 3 * C), mk(B, C), mk(B, 4 * C)
        aws = torch.empty(G.attention_decode_workspace_bytes(B, C, NH, w.maxT), dtype=torch.uint8,
                          device="cuda")
        s = torch.cuda.current_stream()
        recs = []

        def timed(name, fn, nbytes, site=None):
            # consecutive launches share the event between them
            if not recs:
                a = torch.cuda.Event(enable_timing=True)
                a.record(s)
            else:
                a = recs[-1][5]
            fn()
            b = torch.cuda.Event(enable_timing=True)
            b.record(s)
            recs.append(["hbm", name, 0.0, float(nbytes), a, b, site or name])

        def gemm(out, inp, wt, bias, K, Nc, tag):
            nb = (Nc * K + B * K + B * Nc + (Nc if bias is not None else 0)) * es
            timed(G.matmul_kernel_config(B, K, Nc, w.dtype), lambda: G.matmul_forward(out, inp, wt, bias), nb,
                  "gemm_" + tag)

        att_bytes = (B * (pos + 1) * C * 2 + B * 3 * C + B * C) * es
        s_ap = G.matmul_splitk_count(C, C, w.dtype)
        s_fp = G.matmul_splitk_count(4 * C, C, w.dtype)
        part = torch.empty(max(s_ap, s_fp) * B * C, dtype=torch.float32, device="cuda")
        pap, pfp = part[:s_ap * B * C].view(s_ap, B, C), part[:s_fp * B * C].view(s_fp, B, C)

        def splitk(pt, inp, wt, K, Nc, tag):
            nb = (Nc * K + B * K) * es + pt.numel() * 4
            timed("gemm_%s_splitk%d" % ("bf16" if w.dtype == I.BF16 else "f32", pt.shape[0]),
                  lambda: G.matmul_splitk_forward(pt, inp, wt, pt.shape[0]), nb, "gemm_" + tag)

        def res_ln(pt, bias, g, b_, tag):
            nb = 3 * B * C * es + pt.numel() * 4 + 3 * C * es
            timed("residual_layernorm", lambda: G.residual_layernorm_forward(ln, x, pt, bias, g, b_, w.ln_eps), nb,
                  tag)

        all_runs = []
        host_ms = 50.0
        for _ in range(reps + 1):  # the first pass measures the host enqueue time
            recs.clear()
            self.gpu_hold(1.2 * host_ms)
            t0 = time.perf_counter()
            timed("encoder", lambda: G.encoder_forward(x.view(B, 1, C), self.tokens.view(B, 1), P("wte"),
                                                       P("wpe")[pos:pos + 1]),
                  4 * B + 2 * B * C * es + C * es)
            timed("layernorm", lambda: G.layernorm_forward(ln, x, P("ln1_g", 0), P("ln1_b", 0), w.ln_eps),
                  2 * B * C * es + 2 * C * es)
            for l in range(L):
                gemm(qkv, ln, P("qkv_w", l), P("qkv_b", l), C, 3 * C, "qkv")
                timed("attention_decode", lambda: G.attention_decode_forward(
                    att, qkv, self.kcache[l], self.vcache[l], pos, NH, aws), att_bytes)
                splitk(pap, att, P("attproj_w", l), C, C, "attproj")
                res_ln(pap, P("attproj_b", l), P("ln2_g", l), P("ln2_b", l), "residual_ln2")
                timed(G.matmul_kernel_config(B, C, 4 * C, w.dtype) + "_gelu",
                      lambda: G.matmul_gelu_forward(fc, ln, P("fc_w", l), P("fc_b", l)),
                      (4 * C * C + B * C + B * 4 * C + 4 * C) * es, "gemm_fc_gelu")
                splitk(pfp, fc, P("fcproj_w", l), 4 * C, C, "fcproj")
                last = l == L - 1
                res_ln(pfp, P("fcproj_b", l), P("lnf_g") if last else P("ln1_g", l + 1),
                       P("lnf_b") if last else P("ln1_b", l + 1), "residual_ln1")
            gemm(self.logits, ln, P("wte"), None, C, w.Vp, "logits")
            timed("softmax", lambda: G.softmax_forward(self.probs, self.logits, w.V), B * w.V * es + B * w.Vp * es)
            host_ms = (time.perf_counter() - t0) * 1e3
            torch.cuda.synchronize()
            all_runs.append([r[:4] + [r[4].elapsed_time(r[5]), r[6]] for r in recs])
        all_runs = all_runs[1:]
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
    roof["timing"] = "HIP events between consecutive launches on the launch stream, median of passes"
    roof["launches_per_step"] = g["calls"]
    roof["traffic"] = load_traffic(dom)
    # the same kernel's average duration from the committed rocprofv3 kernel
    # trace (while its sources are unchanged), and the fraction it gives
    rp = load_profile_field(dom, "rocprof_avg_us")
    if rp:
        work = g["flops"] if g["kind"] in ("gemm", "mfma") else g["bytes"]
        scale = 1e12 if g["kind"] in ("gemm", "mfma") else 1e9
        roof["rocprof_avg_launch_us"] = rp
        roof["frac_rocprof"] = round(work / g["calls"] / (rp * 1e-6) / scale / roof["peak"], 4)
    return table, roof


# Source files that define each profiled kernel: a counter run stays valid
# until one of them changes.
KERNEL_SOURCES = {
    "gemm": ("common.h", "gemm.h", "matmul.hip"),
    "attention_decode": ("common.h", "attention.hip"),
    "attention": ("common.h", "attention.hip"),
}


def kernel_sources(kernel):
    return KERNEL_SOURCES["gemm" if kernel.startswith("gemm_") else kernel]


def load_profile_field(kernel, field):
    """A per-kernel figure from the committed rocprofv3 runs (profiles/
    traffic.json), or None if there is none for this kernel or its sources
    changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
        ent = data.get(kernel)
        if not ent:
            return None
        if ent.get("source_sha1") != source_sha1(kernel_sources(kernel)):
            return None
        return ent.get(field)
    except Exception:
        return None


def load_traffic(kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs."""
    return load_profile_field(kernel, "bytes_per_launch")


def source_sha1(files):
    h = hashlib.sha1()
    csrc = os.path.join(ROOT, "transformer_forward_pass_gpt_amd", "csrc")
    for f in sorted(files):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def profile_kernel(b, target="vocab"):
    """Counter-collection mode (rocprofv3 --pmc): launch the workload's dominant
    kernel three times, then one plain 256 MiB device-to-device copy whose known
    bytes calibrate the traffic counters. Forward workloads: the vocabulary GEMM
    (or, by target, the prefill attention over random q, k, v, or one layer-0
    projection on random activations with the forward's epilogue); decode:
    attention over the KV cache of layers 0..2 (one decode_attn launch, plus its
    combine when it splits)."""
    torch, G, I, w = b.torch, b.G, b.I, b.w
    if b.decode:
        B, C, NH = w.B, w.C, w.NH
        qkv = torch.randn(B, 3 * C, device="cuda").to(b.tdtype)
        att = torch.empty(B, C, dtype=b.tdtype, device="cuda")
        aws = torch.empty(G.attention_decode_workspace_bytes(B, C, NH, w.maxT), dtype=torch.uint8, device="cuda")
        for l in range(3):
            G.attention_decode_forward(att, qkv, b.kcache[l], b.vcache[l], w.decode_pos, NH, aws)
        info = {"kernel": "attention_decode", "shape": [B, NH, w.decode_pos + 1, w.hs]}
    elif target == "attention":
        qkv = torch.randn(w.B, w.T, 3 * w.C, device="cuda").to(b.tdtype)
        att = torch.empty(w.B, w.T, w.C, dtype=b.tdtype, device="cuda")
        for _ in range(3):
            G.attention_forward(att, qkv, w.NH)
        info = {"kernel": "attention", "shape": [w.B, w.T, w.C, w.NH]}
    elif target != "vocab":
        N = w.B * w.T
        offs = I.param_offsets(w.L, w.C, w.maxT, w.Vp)

        def par(name):  # layer 0's slice of a stacked parameter
            o, shp = offs[name]
            return b.params[o:o + int(np.prod(shp[1:]))].view(*shp[1:])
        wgt, bias = par(target + "_w"), par(target + "_b")
        OC, K = wgt.shape
        inp = torch.randn(N, K, device="cuda").to(b.tdtype)
        out = torch.empty(N, OC, dtype=b.tdtype, device="cuda")
        res = torch.randn(N, OC, device="cuda").to(b.tdtype)
        for _ in range(3):
            if target == "fc":
                G.matmul_gelu_forward(out, inp, wgt, bias)
            elif target in ("attproj", "fcproj"):
                G.matmul_residual_forward(out, inp, wgt, bias, res)
            else:
                G.matmul_forward(out, inp, wgt, bias)
        info = {"kernel": G.matmul_kernel_config(N, K, OC, w.dtype), "shape": [N, K, OC]}
    else:
        N = w.B * w.T
        o, shp = I.param_offsets(w.L, w.C, w.maxT, w.Vp)["wte"]
        wte = b.params[o:o + int(np.prod(shp))].view(*shp)
        ln = torch.randn(N, w.C, device="cuda").to(b.tdtype)
        logits = b.logits.view(N, w.Vp)
        for _ in range(3):
            G.matmul_forward(logits, ln, wte, None)
        info = {"kernel": G.matmul_kernel_config(N, w.C, w.Vp, w.dtype), "shape": [N, w.C, w.Vp]}
    src = torch.ones(64 << 20, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    info["copy_bytes_each_way"] = 256 << 20
    print(json.dumps(info))


def host_info():
    """The host the CPU baseline ran on: CPU model and logical CPU counts."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    info = {"cpu_model": model, "nproc": os.cpu_count()}
    try:
        info["cpus_allowed"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    return info


def forward_flops_per_token(w, t):
    """Algorithmic flops of one position t (0-based): block GEMMs and logits
    (2 flops per weight, V columns), plus causal attention over t+1 keys."""
    C, L = w.C, w.L
    gemm = 2.0 * L * 12 * C * C + 2.0 * C * w.V
    return gemm + 4.0 * L * C * (t + 1)


def elementwise(b, steps):
    """gelu_forward on [N, 4C] and residual_forward on [N, C] (N = B*T) with
    inputs cold in HBM: a 1 GiB buffer (4x the 256 MiB last-level cache) is
    READ before each launch. A written flush buffer would leave dirty lines
    whose write-back competes with the timed kernel (a plain device copy then
    loses a third of its rate). Algorithmic bytes: GELU 2*N*4C*s (read x,
    write y), residual 3*N*C*s (read a and b, write out). Beside each, a plain
    device-to-device copy moving the same bytes under the same conditions:
    the practical streaming rate at that size."""
    torch, G, w = b.torch, b.G, b.w
    N, C, es = w.B * w.T, w.C, b.es
    g_in = torch.randn(N, 4 * C, device="cuda").to(b.tdtype)
    g_out = torch.empty_like(g_in)
    ra = torch.randn(N, C, device="cuda").to(b.tdtype)
    rb = torch.randn(N, C, device="cuda").to(b.tdtype)
    r_out = torch.empty_like(ra)
    c_in = torch.empty(3 * N * C * es // 2, dtype=torch.uint8, device="cuda")  # copy of 3*N*C*s bytes total
    c_out = torch.empty_like(c_in)
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")

    def timed(fn):
        ts = []
        for i in range(steps + 1):
            flush.sum()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            if i:
                ts.append(e0.elapsed_time(e1) * 1e3)
        return float(np.median(ts))

    res = {}
    for name, fn, cp, nbytes in (("gelu", lambda: G.gelu_forward(g_out, g_in), lambda: g_out.copy_(g_in),
                                  2 * N * 4 * C * es),
                                 ("residual", lambda: G.residual_forward(r_out, ra, rb), lambda: c_out.copy_(c_in),
                                  3 * N * C * es)):
        us, cus = timed(fn), timed(cp)
        gbs = nbytes / us / 1e3
        res[name] = {"n": int(g_in.numel() if name == "gelu" else ra.numel()), "avg_us": round(us, 2),
                     "bytes": nbytes, "GBps": round(gbs, 1), "frac_peak": round(gbs / PEAK["hbm_GBps"], 4),
                     "device_copy_same_bytes_GBps": round(nbytes / cus / 1e3, 1)}
    return res


def cpu_baseline(b, ntok):
    """The oracle, single-threaded, on the first ntok positions of sequence 0
    (by the causal invariant, exactly those positions of the full workload).
    Early positions attend over fewer keys, so their average work per token is
    below the full sequence's; the sample string states by how much."""
    import oracle
    w = b.w
    tok = b.tokens_np[:1, :ntok]
    t0 = time.perf_counter()
    oracle.forward(tok, b.params_np, w.L, w.C, w.NH, w.V, w.Vp, w.maxT, w.ln_eps)
    dt = time.perf_counter() - t0
    f_sample = np.mean([forward_flops_per_token(w, t) for t in range(ntok)])
    f_full = np.mean([forward_flops_per_token(w, t) for t in range(w.T)])
    return {"value": round(ntok / dt, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "host": host_info(),
            "sample": "sequence 0, positions 0..%d of the same workload (%d tokens, %.1f s, single-threaded C "
                      "oracle); these positions carry %.1f%% less arithmetic per token than the average over "
                      "all %d positions, so the rate overstates a whole sequence's by about that"
                      % (ntok - 1, ntok, dt, 100.0 * (1.0 - f_sample / f_full), w.T)}


def cpu_baseline_train(b, ntok):
    """The oracle's forward + backward, single-threaded, on the first ntok
    positions of sequence 0 with their targets (a training step on that
    sample; its gradient is that sample's, not a share of the full batch's)."""
    import oracle
    w = b.w
    tok = b.tokens_np[:1, :ntok]
    tg = b.targets_np[:1, :ntok]
    t0 = time.perf_counter()
    oracle.backward(tok, tg, b.params_np, w.L, w.C, w.NH, w.V, w.Vp, w.maxT, w.ln_eps)
    dt = time.perf_counter() - t0
    return {"value": round(ntok / dt, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle", "host": host_info(),
            "sample": "training step on sequence 0, positions 0..%d with their targets (%d tokens, %.1f s, "
                      "single-threaded C oracle)" % (ntok - 1, ntok, dt)}


def cpu_baseline_decode(b, nseq):
    """The oracle's decode step, single-threaded, for the first nseq of the 32
    sequences (sequences are independent, so this is exactly their share of
    the workload)."""
    import oracle
    w = b.w
    kc = np.ascontiguousarray(b.kc_np[:, :nseq])
    vc = np.ascontiguousarray(b.vc_np[:, :nseq])
    tok = b.tokens_np[:nseq]
    t0 = time.perf_counter()
    oracle.decode_step(tok, w.decode_pos, kc, vc, b.params_np, w.L, w.C, w.NH, w.V, w.Vp, w.maxT, w.ln_eps)
    dt = time.perf_counter() - t0
    return {"value": round(nseq / dt, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle", "host": host_info(),
            "sample": "decode step for sequences 0..%d of the 32 at position %d (%d tokens, %.1f s, "
                      "single-threaded C oracle)" % (nseq - 1, w.decode_pos, nseq, dt)}


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
    decode = w.decode_pos >= 0
    torch.cuda.set_device(0)
    train = args.mode == "train"
    if train and decode:
        print("bench.py: --mode train needs a prefill workload", file=sys.stderr)
        sys.exit(2)
    b = Bench(w, keep_host_cache=decode and not args.no_cpu_baseline, train=train)
    if args.profile_kernel:
        profile_kernel(b, args.profile_target)
        return
    if args.elementwise:
        print(json.dumps({"workload": args.workload, "dtype": "bf16" if w.dtype == I.BF16 else "f32",
                          "timing": "HIP events around each launch, inputs cold in HBM (1 GiB read before each)",
                          "kernels": elementwise(b, args.steps)}), flush=True)
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
    tokens = w.B * (1 if decode else w.T)
    prec = "bf16" if w.dtype == I.BF16 else "fp32"
    size = "124M" if w.C == 768 else "350M"
    if train:
        metric = "train tokens/s GPT-2 %s %s B%d T%d (forward + loss + backward, no optimizer)" % (
            size, prec, w.B, w.T)
        wl = "GPT-2 %s %s training step B%d T%d: forward keeping activations, cross-entropy, backward to " \
             "every parameter gradient" % (size, prec, w.B, w.T)
        data = "synthetic (seeded uniform tokens, next-token targets, N(0,0.02) weights)"
    elif decode:
        metric = "decode tokens/s GPT-2 124M bf16, 32 sequences at position %d; HBM GB/s" % w.decode_pos
        wl = "GPT-2 %s %s decode step, %d sequences, KV cache of %d positions (logits + softmax)" % (
            size, prec, w.B, w.decode_pos)
        data = "synthetic (seeded uniform tokens, N(0,0.02) weights, N(0,1) key/value cache)"
    else:
        metric = METRIC
        wl = "GPT-2 %s %s forward B%d T%d (logits + softmax)" % (size, prec, w.B, w.T)
        data = "synthetic (seeded uniform tokens, N(0,0.02) weights)"
    res = {
        "metric": metric,
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
        "data": data,
        "config": {"workload": wl, "B": w.B, "T": w.T, "L": w.L, "C": w.C, "NH": w.NH, "V": w.V, "Vp": w.Vp},
    }
    if decode:
        res["config"]["pos"] = w.decode_pos
    if not args.no_kernel_timing:
        recs = (b.train_kernel_timing() if train else b.decode_kernel_timing() if decode
                else b.kernel_timing())
        table, roof = summarize_kernels(recs, w.dtype == I.BF16)
        sites, _ = summarize_kernels(recs, w.dtype == I.BF16, key=5)
        res["roofline"] = roof
        res["kernels"] = table
        res["sites"] = sites
        res["kernel_sum_ms"] = round(sum(r[4] for r in recs), 4)
    if train:
        res["mean_loss"] = round(float(b.mean_loss.item()), 6)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = (cpu_baseline_train(b, args.cpu_sample_train_tokens) if train
                               else cpu_baseline_decode(b, args.cpu_sample_seqs) if decode
                               else cpu_baseline(b, args.cpu_sample_tokens))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
