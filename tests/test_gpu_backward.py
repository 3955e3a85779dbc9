"""Backward parity: each backward C-ABI entry against the CPU oracle's
backward on the same seeded inputs, at small shapes spanning several tiles and
a ragged tail, and at GPT-2 small's full shapes on sampled outputs the oracle
computes piecewise (row slices, single heads); the whole training step
against the oracle's full-model gradient on the tiny configurations, and by a
central difference of the loss along the gradient at GPT-2 small's size.

Tolerances (floating point):
  cross-entropy backward  fp32 |d| <= 2e-6 dloss;             bf16 <= 2^-8 |ref| + 2e-6 dloss
  gelu backward           fp32 |d| <= 4e-6 |dout| max(1,|x|); bf16 adds 2^-8 |ref|
  layernorm backward      fp32 ||d||/||ref|| <= 1e-5;          bf16 <= 1e-2
  linear backward         fp32 ||d||/||ref|| <= 2e-5;          bf16 <= 1e-2; integer inputs bit-exact
  attention lse           |d| <= 2e-5 max(1, |ref|)
  attention backward      fp32 ||d||/||ref|| <= 2e-5;          bf16 <= 3e-2, for each of dq, dk, dv
                          with ||ref|| floored at 0.1 ||d(qkv)||: at T = 1 dq and dk are exactly 0
                          (dP - D cancels), and both sides leave rounding-level residues there
  encoder backward        fp32 |d| <= 1e-5 max|ref|;           bf16 <= 2^-8 |ref| + 1e-6
  training step           fp32 per-tensor ||d||/||ref|| <= 1e-4; bf16 <= 6e-2 (tiny configs, and
                          GPT-2 small's width, heads and vocabulary with 2 layers and 64 tokens)
"""
import sys

import numpy as np
import pytest

import oracle
import transformer_forward_pass_gpt_amd as G
from transformer_forward_pass_gpt_amd import inputs as I

from gpu_util import dev, dev_int, empty, host, host_bits, max_abs, rel_err, tile_rel_max

pytestmark = pytest.mark.gpu
DT = {"f32": I.F32, "bf16": I.BF16}


def announce(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def ws(nbytes):
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device="cuda")


# ------------------------------------------------------------ cross-entropy
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("N,V,Vp", [(5, 250, 256), (7, 1000, 1008), (4, 50257, 50304), (520, 50257, 50304)])
def test_crossentropy_backward(dt, N, V, Vp):
    announce("crossentropy_backward", dt, N, V, Vp)
    d = DT[dt]
    logits = I.random_tensor(11, (N, Vp), 2.0, d)
    tg = np.random.default_rng(12).integers(0, V, N).astype(np.int32)
    dloss = 1.0 / N
    ref = oracle.crossentropy_backward(logits, tg, V, dloss)
    ref_loss = oracle.crossentropy(logits, tg, V)
    lg = dev(logits, d)
    dl = empty((N, Vp), d)
    losses = empty((N,), I.F32)
    mean = empty((1,), I.F32)
    G.crossentropy_backward(dl, lg, dev_int(tg), V, dloss, losses, mean)
    out = host(dl)
    if d == I.F32:
        assert max_abs(out, ref) <= 2e-6 * dloss
    else:
        assert np.all(np.abs(out - ref) <= 2.0 ** -8 * np.abs(ref) + 2e-6 * dloss)
    assert np.all(out[:, V:] == 0)
    assert np.all(np.abs(host(losses) - ref_loss) <= 1e-5 * np.maximum(1.0, np.abs(ref_loss)))
    assert abs(host(mean)[0] - ref_loss.astype(np.float64).mean()) <= 1e-5 * max(1.0, abs(ref_loss.mean()))
    # in place over the logits: same bits
    G.crossentropy_backward(lg, lg, dev_int(tg), V, dloss)
    assert np.array_equal(host_bits(lg), host_bits(dl))
    if N >= 512:
        # the many-row kernel form (packed bf16 rows) against the few-row one
        few = empty((32, Vp), d)
        G.crossentropy_backward(few, dev(logits[:32], d), dev_int(tg[:32]), V, dloss)
        assert np.array_equal(host_bits(few), host_bits(dl)[:32])


# ------------------------------------------------------------ gelu
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [8, 1000003, 4096 * 3072])
def test_gelu_backward(dt, n):
    announce("gelu_backward", dt, n)
    d = DT[dt]
    x = I.random_tensor(21, n, 2.5, d)
    dy = I.random_tensor(22, n, 1.0, d)
    ref = oracle.gelu_backward(x, dy)
    out = empty((n,), d)
    G.gelu_backward(out, dev(x, d), dev(dy, d))
    got = host(out)
    bound = 4e-6 * np.abs(dy) * np.maximum(1.0, np.abs(x))
    if d == I.BF16:
        bound = bound + 2.0 ** -8 * np.abs(ref)
    assert np.all(np.abs(got - ref) <= bound + 1e-30)
    # in place over dout
    g = dev(dy, d)
    G.gelu_backward(g, dev(x, d), g)
    assert np.array_equal(host_bits(g), host_bits(out))


# ------------------------------------------------------------ layernorm
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("N,C", [(64, 64), (37, 104), (1000, 768), (4096, 768)])
@pytest.mark.parametrize("with_res", [False, True])
def test_layernorm_backward(dt, N, C, with_res):
    announce("layernorm_backward", dt, N, C, with_res)
    d = DT[dt]
    x = I.random_tensor(31, (N, C), 1.0, d) + I.random_tensor(32, (N, 1), 0.5, d)
    x = I.round_to_bf16(x) if d == I.BF16 else x
    gamma = (1.0 + I.random_tensor(33, C, 0.1, I.F32))
    gamma = I.round_to_bf16(gamma) if d == I.BF16 else gamma
    beta = I.random_tensor(34, C, 0.1, d)
    dy = I.random_tensor(35, (N, C), 1.0, d)
    dres = I.random_tensor(36, (N, C), 1.0, d)
    rdx, rdg, rdb = oracle.layernorm_backward(dy, x, gamma, 1e-5)
    if with_res:
        rdx = rdx + dres
    xg, gg = dev(x, d), dev(gamma, d)
    y = empty((N, C), d)
    mean = empty((N,), I.F32)
    rstd = empty((N,), I.F32)
    G.layernorm_forward(y, xg, gg, dev(beta, d), 1e-5, mean, rstd)
    dx = dev(dres, d) if with_res else empty((N, C), d)
    dg = empty((C,), d)
    db = empty((C,), d)
    w = ws(G.layernorm_backward_workspace_size(N, C))
    G.layernorm_backward(dx, dg, db, dev(dy, d), xg, gg, mean, rstd, w, dres=dx if with_res else None)
    tol = 1e-5 if d == I.F32 else 1e-2
    assert rel_err(host(dx), rdx) <= tol
    assert rel_err(host(dg), rdg) <= tol
    assert rel_err(host(db), rdb) <= tol


# ------------------------------------------------------------ linear
def _linear_case(d, N, C, OC, seed, integer=False):
    if integer:
        x = I.random_int_tensor(seed, (N, C), -3, 3)
        wt = I.random_int_tensor(seed + 1, (OC, C), -3, 3)
        dy = I.random_int_tensor(seed + 2, (N, OC), -3, 3)
    else:
        x = I.random_tensor(seed, (N, C), 1.0, d)
        wt = I.random_tensor(seed + 1, (OC, C), 0.02, d)
        dy = I.random_tensor(seed + 2, (N, OC), 1.0, d)
    dx, dw, db = empty((N, C), d), empty((OC, C), d), empty((OC,), d)
    w = ws(G.matmul_backward_workspace_size(N, C, OC, d))
    G.matmul_backward(dx, dw, db, dev(dy, d), dev(x, d), dev(wt, d), w)
    return x, wt, dy, host(dx), host(dw), host(db)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("N,C,OC", [(64, 64, 256), (37, 104, 40), (130, 256, 64), (1, 8, 8), (1000, 104, 200),
                                    (1024, 104, 200), (256, 96, 64), (96, 64, 136), (64, 8, 8), (1024, 8, 16)])
def test_matmul_backward(dt, N, C, OC):
    announce("matmul_backward", dt, N, C, OC)
    d = DT[dt]
    x, wt, dy, dx, dw, db = _linear_case(d, N, C, OC, 41)
    rx, rw, rb = oracle.matmul_backward(dy, x, wt)
    tol = 2e-5 if d == I.F32 else 1e-2
    assert rel_err(dx, rx) <= tol
    assert rel_err(dw, rw) <= tol
    assert rel_err(db, rb) <= tol


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("N,C,OC", [(96, 64, 136), (128, 72, 192)])
def test_matmul_backward_integer_exact(dt, N, C, OC):
    """Small-integer operands: every product and sum is exact in fp32 and the
    results (|x| <= 216 for these seeds) in bf16. (96, 64, 136): contractions
    that are not whole bf16 k-tiles (transposed operands in bf16); (128, 72,
    192): both products on k-major operands read in place in both dtypes."""
    announce("matmul_backward_integer", dt, N, C, OC)
    d = DT[dt]
    x, wt, dy, dx, dw, db = _linear_case(d, N, C, OC, 51, integer=True)
    rx, rw, rb = oracle.matmul_backward(dy, x, wt)
    assert np.array_equal(dx, rx) and np.array_equal(dw, rw) and np.array_equal(db, rb)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("C,OC", [(768, 2304), (3072, 768), (768, 768)])
def test_matmul_backward_gpt2_small_sampled(dt, C, OC):
    """B4 T1024 shapes (the weight gradient in 4, 4 and 8 k-slices for bf16);
    dinp on sampled rows and dweight/dbias on sampled output features, each
    from the oracle on the corresponding slice."""
    announce("matmul_backward_full", dt, C, OC)
    d = DT[dt]
    N = 4096
    x, wt, dy, dx, dw, db = _linear_case(d, N, C, OC, 61)
    rows = np.random.default_rng(62).choice(N, 48, replace=False)
    feats = np.random.default_rng(63).choice(OC, 24, replace=False)
    rx, _, _ = oracle.matmul_backward(dy[rows], x[rows], wt)
    _, rw, rb = oracle.matmul_backward(dy[:, feats], x, wt[feats])
    tol = 2e-5 if d == I.F32 else 1e-2
    assert rel_err(dx[rows], rx) <= tol
    assert rel_err(dw[feats], rw) <= tol
    assert rel_err(db[feats], rb) <= tol


# ------------------------------------------------------------ attention
def _part_err(got, ref, part, C):
    """||got - ref|| over one of dq, dk, dv, relative to that part's norm
    floored at a tenth of the whole gradient's norm."""
    sl = slice(part * C, (part + 1) * C)
    g, r = np.asarray(got[..., sl], np.float64), np.asarray(ref[..., sl], np.float64)
    den = max(np.linalg.norm(r), 0.1 * np.linalg.norm(np.asarray(ref, np.float64)), 1e-300)
    return float(np.linalg.norm(g - r) / den)


def _attn_fwd(qkv, NH, d):
    B, T, C3 = qkv.shape
    q = dev(qkv, d)
    out = empty((B, T, C3 // 3), d)
    lse = empty((B, NH, T), I.F32)
    G.attention_forward_lse(out, lse, q, NH)
    return q, out, lse


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,C,NH", [(2, 32, 64, 4), (1, 77, 64, 2), (2, 200, 128, 2), (1, 1, 64, 1)])
def test_attention_lse(dt, B, T, C, NH):
    announce("attention_lse", dt, B, T, C, NH)
    d = DT[dt]
    qkv = I.random_tensor(71, (B, T, 3 * C), 1.0, d)
    q, out, lse = _attn_fwd(qkv, NH, d)
    ref = oracle.attention_lse(qkv, NH)
    # bf16: the normaliser sums the bf16-rounded probabilities of the P.V
    # product (relative error <= 2^-9), so ln of it moves by <= 2^-9
    tol = 2e-5 * np.maximum(1.0, np.abs(ref)) + (2.0 ** -8 if d == I.BF16 else 0.0)
    assert np.all(np.abs(host(lse) - ref) <= tol)
    plain = empty((B, T, C), d)
    G.attention_forward(plain, q, NH)
    assert np.array_equal(host_bits(plain), host_bits(out))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,C,NH", [(2, 32, 64, 4), (1, 77, 64, 2), (2, 200, 128, 2), (1, 1, 64, 1),
                                      (1, 130, 64, 1), (3, 257, 192, 3)])
def test_attention_backward(dt, B, T, C, NH):
    announce("attention_backward", dt, B, T, C, NH)
    d = DT[dt]
    qkv = I.random_tensor(81, (B, T, 3 * C), 1.0, d)
    dy = I.random_tensor(82, (B, T, C), 1.0, d)
    q, out, lse = _attn_fwd(qkv, NH, d)
    dq = empty((B, T, 3 * C), d)
    w = ws(G.attention_backward_workspace_size(B, T, C, NH))
    G.attention_backward(dq, dev(dy, d), q, out, lse, NH, w)
    ref = oracle.attention_backward(dy, qkv, NH)
    got = host(dq)
    tol = 2e-5 if d == I.F32 else 3e-2
    for part in range(3):  # dq, dk, dv separately
        assert _part_err(got, ref, part, C) <= tol, part


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_attention_backward_gpt2_small_sampled(dt):
    """B4 T1024 NH12: two (batch, head) pairs checked against the oracle run
    on that head alone."""
    announce("attention_backward_full", dt)
    d = DT[dt]
    B, T, C, NH = 4, 1024, 768, 12
    hs = C // NH
    qkv = I.random_tensor(91, (B, T, 3 * C), 1.0, d)
    dy = I.random_tensor(92, (B, T, C), 1.0, d)
    q, out, lse = _attn_fwd(qkv, NH, d)
    dq = empty((B, T, 3 * C), d)
    w = ws(G.attention_backward_workspace_size(B, T, C, NH))
    G.attention_backward(dq, dev(dy, d), q, out, lse, NH, w)
    got = host(dq)
    tol = 2e-5 if d == I.F32 else 3e-2
    for b, h in ((0, 0), (3, 11)):
        cols = [np.arange(p * C + h * hs, p * C + (h + 1) * hs) for p in range(3)]
        sub = qkv[b:b + 1][:, :, np.concatenate(cols)]
        ref = oracle.attention_backward(dy[b:b + 1, :, h * hs:(h + 1) * hs], sub, 1)
        for p in range(3):
            assert rel_err(got[b][:, cols[p]], ref[0][:, p * hs:(p + 1) * hs]) <= tol, (b, h, p)


# ------------------------------------------------------------ encoder
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,C,Vtok,Vp", [(2, 32, 64, 5, 256), (3, 37, 104, 1000, 1008), (4, 1024, 768, 50257, 50304)])
def test_encoder_backward(dt, B, T, C, Vtok, Vp):
    announce("encoder_backward", dt, B, T, C, Vtok)
    d = DT[dt]
    tok = np.random.default_rng(101).integers(0, Vtok, (B, T)).astype(np.int32)
    tok[-1, -8:] = tok[0, 0]  # a repeated id in every case
    dy = I.random_tensor(102, (B, T, C), 1.0, d)
    maxT = T + 3
    pre_te = I.random_tensor(103, (Vp, C), 1.0, d)
    pre_pe = I.random_tensor(104, (maxT, C), 1.0, d)
    rte, rpe = oracle.encoder_backward(dy, tok, Vp, maxT, pre_te, pre_pe)
    te, pe = dev(pre_te, d), dev(pre_pe, d)
    G.encoder_backward(te, pe, dev(dy, d), dev_int(tok))
    for got, ref in ((host(te), rte), (host(pe), rpe)):
        if d == I.F32:
            assert max_abs(got, ref) <= 1e-5 * np.max(np.abs(ref))
        else:
            assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)


# ------------------------------------------------------------ training step
def _cfg(w):
    return G.make_config(w.L, w.C, w.NH, w.V, w.Vp, w.maxT, w.dtype, w.ln_eps)


def _train_step(w, params_np):
    cfg = _cfg(w)
    tok = dev_int(I.make_tokens(w))
    tg = dev_int(I.make_targets(w))
    params = dev(params_np, w.dtype)
    acts = ws(G.train_acts_bytes(cfg, w.B, w.T))
    work = ws(G.train_workspace_bytes(cfg, w.B, w.T))
    grads = empty((params_np.size,), w.dtype)
    losses = empty((w.B * w.T,), I.F32)
    mean = empty((1,), I.F32)
    G.gpt2_train_forward(tok, tg, params, cfg, acts, losses, mean)
    G.gpt2_backward(grads, tok, params, cfg, acts, work)
    return grads, losses, mean


@pytest.mark.parametrize("name", ["tiny", "tiny_affine", "tiny_bf16", "small_2l", "small_2l_bf16"])
def test_training_step_vs_oracle(name):
    announce("train_step", name)
    w = I.WORKLOADS[name]
    params = I.make_params(w)
    grads, losses, mean = _train_step(w, params)
    rg, rloss = oracle.backward(I.make_tokens(w), I.make_targets(w), params, w.L, w.C, w.NH, w.V, w.Vp, w.maxT,
                                w.ln_eps)
    assert abs(host(mean)[0] - rloss) <= (1e-5 if w.dtype == I.F32 else 1e-2) * abs(rloss)
    got = I.views(host(grads), w)
    ref = I.views(rg, w)
    tol = 1e-4 if w.dtype == I.F32 else 6e-2
    for k in ref:
        assert np.all(np.isfinite(got[k])), k
        assert rel_err(got[k], ref[k]) <= tol, (k, rel_err(got[k], ref[k]))
        g2 = got[k].reshape(-1, got[k].shape[-1])
        r2 = ref[k].reshape(-1, ref[k].shape[-1])
        # every 128x128 tile of every gradient tensor (a wrong GEMM tile moves
        # the whole tensor's norm by a few percent only)
        assert tile_rel_max(g2, r2) <= 2 * tol, (k, tile_rel_max(g2, r2))


def test_training_step_gpt2_small_directional_derivative():
    """GPT-2 small fp32 B4 T1024: the loss is ln(V) at this init to within a
    few percent, the step is deterministic, and the derivative of the loss
    along the (normalised) gradient direction, measured by a central difference
    of two training forwards, equals the norm of the computed gradient."""
    announce("train_step_small")
    w = I.WORKLOADS["small"]
    params = I.make_params(w)
    grads, losses, mean = _train_step(w, params)
    g = host(grads).astype(np.float64)
    assert np.all(np.isfinite(g))
    loss0 = float(host(mean)[0])
    assert abs(loss0 - np.log(w.V)) <= 0.05 * np.log(w.V)
    grads2, _, _ = _train_step(w, params)
    assert np.array_equal(host_bits(grads), host_bits(grads2))
    gn = np.linalg.norm(g)
    u = g / gn
    eps = 1e-2 / gn  # a loss change of about 0.01
    cfg = _cfg(w)
    tok = dev_int(I.make_tokens(w))
    tg = dev_int(I.make_targets(w))
    acts = ws(G.train_acts_bytes(cfg, w.B, w.T))
    vals = []
    for sgn in (1.0, -1.0):
        p = (params.astype(np.float64) + sgn * eps * u).astype(np.float32)
        m = empty((1,), I.F32)
        G.gpt2_train_forward(tok, tg, dev(p, w.dtype), cfg, acts, None, m)
        vals.append(float(host(m)[0]))
    fd = (vals[0] - vals[1]) / (2 * eps)
    assert abs(fd - gn) <= 0.02 * gn, (fd, gn)
