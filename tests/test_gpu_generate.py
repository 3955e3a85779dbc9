"""Greedy KV-cached generation on the GPU: argmax_forward, gpt2_prefill and
gpt2_generate against the CPU oracle (forward, capture of k and v) and
against a host-driven loop over the same GPU entries.

Where floating point decides a token (argmax), the decision is compared in
the kernel's own precision: the GPU's choice must equal numpy's argmax over
the GPU's logits, bit for bit. Against the oracle only what is unique is
compared: at every generated position the GPU's token must be the oracle's
argmax or within the logits tolerance of it (a near-tie may go either way).
"""
import numpy as np
import pytest

import oracle
import transformer_forward_pass_gpt_amd as G
from transformer_forward_pass_gpt_amd import inputs as I

from gpu_util import dev, dev_int, empty, host, max_abs, rel_err

pytestmark = pytest.mark.gpu


def announce(*a):
    print("[case]", *a, flush=True)


def cfg_of(w):
    return G.make_config(w.L, w.C, w.NH, w.V, w.Vp, w.maxT, w.dtype, w.ln_eps)


@pytest.mark.parametrize("dt", [I.F32, I.BF16])
@pytest.mark.parametrize("N,V,Vp", [(5, 256, 256), (64, 50257, 50304), (3, 1000, 1008)])
def test_argmax(dt, N, V, Vp):
    announce("argmax", dt, N, V, Vp)
    import torch
    rng = np.random.default_rng(60 + N)
    x = rng.standard_normal((N, Vp)).astype(np.float32)
    if dt == I.BF16:
        x = I.round_to_bf16(x)
    x[:, V:] = 100.0                      # padding must be ignored
    x[0, 7] = x[0, V - 1] = 50.0          # tie: the lowest index wins
    x[1, :V] = 1.5                        # all equal: index 0
    if N > 2:
        x[2, V - 1] = 60.0                # maximum in the last real column
    tok = torch.full((N,), -1, dtype=torch.int32, device="cuda")
    G.argmax_forward(tok, dev(x, dt), V)
    got = tok.cpu().numpy()
    assert np.array_equal(got, np.argmax(x[:, :V], axis=1))
    assert got[0] == 7 and got[1] == 0


def run_prefill(w, params, tok, B, T):
    import torch
    cfg = cfg_of(w)
    shape = (w.L, B, w.NH, w.maxT, w.hs)
    kc = empty(shape, w.dtype, fill=float("nan"))  # slots >= T must stay untouched
    vc = empty(shape, w.dtype, fill=float("nan"))
    logits = empty((B, w.Vp), w.dtype, fill=float("nan"))
    probs = empty((B, w.Vp), w.dtype, fill=float("nan"))
    ws = torch.empty(G.workspace_bytes(cfg, B, T), dtype=torch.uint8, device="cuda")
    pt = dev(params, w.dtype)
    G.gpt2_prefill(logits, probs, dev_int(tok), kc, vc, pt, cfg, ws)
    return logits, probs, kc, vc, pt, cfg


@pytest.mark.parametrize("name,T", [("tiny_affine", 20), ("tiny_bf16", 32), ("small_bf16_b4", 64)])
def test_prefill(name, T):
    announce("prefill", name, T)
    import torch
    w = I.WORKLOADS[name]
    B = 2
    params = I.make_params(w)
    tok = I.make_tokens(w)[:B, :T].copy()
    logits, probs, kc, vc, pt, cfg = run_prefill(w, params, tok, B, T)
    rl, rp, cap = oracle.forward(tok, params, w.L, w.C, w.NH, w.V, w.Vp, w.maxT, w.ln_eps, capture=True)
    gl = host(logits)
    if w.dtype == I.F32:
        assert max_abs(gl[:, :w.V], rl[:, T - 1, :w.V]) <= 1e-3
        assert rel_err(gl[:, :w.V], rl[:, T - 1, :w.V]) <= 1e-4
        assert max_abs(host(probs), rp[:, T - 1]) <= 1e-6
    else:
        assert rel_err(gl[:, :w.V], rl[:, T - 1, :w.V]) <= 2e-2
        assert rel_err(host(probs), rp[:, T - 1]) <= 2e-2
    # the GPU forward's last row (a different GEMM path for the logits)
    ws = torch.empty(G.workspace_bytes(cfg, B, T), dtype=torch.uint8, device="cuda")
    lf = empty((B, T, w.Vp), w.dtype)
    G.gpt2_forward(lf, None, dev_int(tok), pt, cfg, ws)
    assert rel_err(gl[:, :w.V], host(lf)[:, T - 1, :w.V]) <= (1e-5 if w.dtype == I.F32 else 1e-2)
    # caches: the oracle's k and v at 0..T-1, untouched beyond
    kg, vg = host(kc), host(vc)
    for l in range(w.L):
        q = cap["qkv.%d" % l]
        kr = q[:, :, w.C:2 * w.C].reshape(B, T, w.NH, w.hs).transpose(0, 2, 1, 3)
        vr = q[:, :, 2 * w.C:].reshape(B, T, w.NH, w.hs).transpose(0, 2, 1, 3)
        tol = 1e-5 if w.dtype == I.F32 else 2e-2
        assert rel_err(kg[l, :, :, :T], kr) <= tol and rel_err(vg[l, :, :, :T], vr) <= tol
    assert np.all(np.isnan(kg[:, :, :, T:])) and np.all(np.isnan(vg[:, :, :, T:]))


@pytest.mark.parametrize("name,B,T,n_new", [("tiny_affine", 2, 8, 16), ("tiny_bf16", 3, 5, 20),
                                            ("small_bf16_b4", 2, 16, 8), ("tiny_affine", 40, 4, 6)])
def test_generate_greedy(name, B, T, n_new):
    announce("generate", name, B, T, n_new)
    import torch
    w = I.WORKLOADS[name]
    params = I.make_params(w)
    rng = np.random.default_rng(700 + B)
    prompt = rng.integers(0, w.V, size=(B, T)).astype(np.int32)
    cfg = cfg_of(w)
    pt = dev(params, w.dtype)
    shape = (w.L, B, w.NH, w.maxT, w.hs)
    kc, vc = empty(shape, w.dtype, fill=0.0), empty(shape, w.dtype, fill=0.0)
    out = torch.full((B, n_new), -1, dtype=torch.int32, device="cuda")
    ws = torch.empty(G.generate_workspace_bytes(cfg, B, T), dtype=torch.uint8, device="cuda")
    G.gpt2_generate(out, dev_int(prompt), kc, vc, pt, cfg, ws)
    gen = out.cpu().numpy()
    assert np.all((gen >= 0) & (gen < w.V))

    # the same steps driven from the host, argmax in numpy over the GPU's logits
    kc2, vc2 = empty(shape, w.dtype, fill=0.0), empty(shape, w.dtype, fill=0.0)
    logits = empty((B, w.Vp), w.dtype)
    ws2 = torch.empty(max(G.workspace_bytes(cfg, B, T), G.decode_workspace_bytes(cfg, B)), dtype=torch.uint8,
                      device="cuda")
    G.gpt2_prefill(logits, None, dev_int(prompt), kc2, vc2, pt, cfg, ws2)
    steps = []
    for i in range(n_new):
        if i > 0:
            G.gpt2_decode_step(logits, None, dev_int(steps[-1]), T + i - 1, kc2, vc2, pt, cfg, ws2)
        steps.append(np.argmax(host(logits)[:, :w.V], axis=1).astype(np.int32))
    assert np.array_equal(gen, np.stack(steps, axis=1))

    # oracle, teacher-forced on prompt + generated tokens
    seq = np.concatenate([prompt, gen], axis=1)[:, :T + n_new - 1]
    rl, _, _ = oracle.forward(seq, params, w.L, w.C, w.NH, w.V, w.Vp, w.maxT, w.ln_eps, probs=False)
    ol = rl[:, T - 1:, :w.V]                          # rows that predicted the generated tokens
    chosen = np.take_along_axis(ol, gen[:, :, None], axis=2)[:, :, 0]
    gap = ol.max(axis=2) - chosen                     # 0 where the GPU picked the oracle's argmax
    tol = 2e-3 if w.dtype == I.F32 else 5e-2 * np.abs(ol).max()
    assert np.all(gap <= tol), gap.max()
    print("oracle argmax agreement %.3f" % np.mean(gap == 0))


def test_generate_from_one_token():
    """A one-token prompt: prefill at T = 1, then decode steps from position 1."""
    announce("generate-T1")
    import torch
    w = I.WORKLOADS["tiny_affine"]
    params = I.make_params(w)
    B, n_new = 2, 12
    prompt = np.array([[3], [250]], np.int32)
    cfg = cfg_of(w)
    shape = (w.L, B, w.NH, w.maxT, w.hs)
    kc, vc = empty(shape, w.dtype, fill=0.0), empty(shape, w.dtype, fill=0.0)
    out = torch.full((B, n_new), -1, dtype=torch.int32, device="cuda")
    ws = torch.empty(G.generate_workspace_bytes(cfg, B, 1), dtype=torch.uint8, device="cuda")
    G.gpt2_generate(out, dev_int(prompt), kc, vc, dev(params, w.dtype), cfg, ws)
    gen = out.cpu().numpy()
    seq = np.concatenate([prompt, gen], axis=1)[:, :n_new]
    rl, _, _ = oracle.forward(seq, params, w.L, w.C, w.NH, w.V, w.Vp, w.maxT, w.ln_eps, probs=False)
    ol = rl[:, :, :w.V]
    chosen = np.take_along_axis(ol, gen[:, :, None], axis=2)[:, :, 0]
    assert np.all(ol.max(axis=2) - chosen <= 2e-3)
