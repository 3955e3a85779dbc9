"""GPU parity for the running-max update of the online softmax.

The tiled attention ("Understand FlashAttention (I)", Algorithm 1 of the
FlashAttention paper) keeps a running max m and normaliser l per query and
rescales its partial output by exp(m_old - m_new) whenever a later key block
holds a larger score. With q, k ~ N(0, 1) at head size 64 the scaled scores
have a standard deviation near 1.4 (in log2 units), so a later block almost
never beats the first block's max by a wide margin and a rescale that only
triggers on a large jump (a lazy running max) is never exercised. These inputs
force it:

  wide      q, k small integers in [-6, 6]: scaled scores with a standard
            deviation of ~20 log2 units, so later blocks beat the earlier max by
            many units for a large share of the queries;
  rising    scores that grow along the keys (one head dimension of k grows
            with the key index, at a different rate per head), so the max moves
            again and again along every row;
  dominant  one key per head in a late key block with a score ~65 log2 units
            above the rest, so every query after it rescales by ~2^-65.

q and k are integer-valued, so every score q.k is exact in fp32 and bf16 and
both sides see the same scores; the comparison measures the softmax and P.V
arithmetic only. Each case first checks that the condition that forces a
running max with a slack of up to 8 log2 units to move (a 64-key block whose
max exceeds the max of every earlier key by more than 8) occurs for many
queries, so a later change of the inputs cannot silently stop covering the
branch.

Tolerances:
  forward fp32   max|d| <= 1e-5 (scores exact; exp2 and the scale multiply
                 give a few ulp of relative error per probability, |v| <= ~1.5)
  forward bf16   ||d||/||ref|| <= 1e-2, and elementwise
                 |d| <= 2^-8 (|ref| + max|v|): each probability is rounded to
                 bf16 (relative 2^-9) before P.V while the normaliser sums the
                 unrounded ones, so |d| <= 2^-9 max|v| before the output's own
                 rounding (2^-9 |ref|)
  lse            |d| <= 2e-5 max(1, |ref|), + 2^-8 for bf16 (lse_tol)
  backward       per part (dq, dk, dv) ||d||/||ref|| <= 2e-5 (fp32) / 3e-2 (bf16;
                 the reference carries the first-order effect of the stored
                 bf16 output on D = rowsum(dO o O), see stored_output_term;
                 dq and dk allow twice the error that rounding dS to bf16
                 alone causes where that is larger, see ds_rounding_error)
"""
import sys

import numpy as np
import pytest

import oracle
import transformer_forward_pass_gpt_amd as G
from transformer_forward_pass_gpt_amd import inputs as I

from gpu_util import dev, empty, host, host_bits, max_abs, rel_err

pytestmark = pytest.mark.gpu
DT = {"f32": I.F32, "bf16": I.BF16}
LOG2E = 1.4426950408889634


def announce(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def make_qkv(kind, B, T, C, NH, dtype, seed=0):
    """Seeded qkv [B,T,3C] whose causal scores force the running max to move."""
    hs = C // NH
    rng = np.random.default_rng(1000 + seed)
    v = (rng.standard_normal((B, T, C)) * 0.25).astype(np.float32)
    if kind == "wide":
        q = rng.integers(-6, 7, (B, T, C)).astype(np.float32)
        k = rng.integers(-6, 7, (B, T, C)).astype(np.float32)
    elif kind == "rising":
        q = rng.integers(-1, 2, (B, T, C)).astype(np.float32)
        k = rng.integers(-1, 2, (B, T, C)).astype(np.float32)
        j = np.arange(T, dtype=np.float64)
        for h in range(NH):
            # key growth per position, by head: at T = 1024 and head size 64,
            # 64 keys raise the score by 8.6 or 11.5 log2 units; shorter rows
            # grow faster so their last, partial block still beats the slack
            # (k stays below 256: exact in bf16)
            rate = (0.1875 + 0.0625 * (h % 2)) * max(1.0, 768.0 / T)
            q[:, :, h * hs] = 4.0
            k[:, :, h * hs] = np.floor(j * rate)[None, :].astype(np.float32)
    elif kind == "dominant":
        q = rng.integers(-2, 3, (B, T, C)).astype(np.float32)
        k = rng.integers(-2, 3, (B, T, C)).astype(np.float32)
        for h in range(NH):
            js = min(T - 1, max(64, int(0.7 * T)) + 3 * h)  # after the first key block
            q[:, :, h * hs] = 3.0
            k[:, js, h * hs] = 120.0
    else:
        raise ValueError(kind)
    qkv = np.concatenate([q, k, v], axis=2).astype(np.float32)
    return I.round_to_bf16(qkv) if dtype == I.BF16 else qkv


def rescale_queries(qkv, NH, block=64, slack=8.0):
    """Number of queries for which some key block's max (keys <= the query)
    exceeds the max over all earlier keys by more than `slack` log2 units."""
    B, T, C3 = qkv.shape
    C = C3 // 3
    hs = C // NH
    nb = (T + block - 1) // block
    count = 0
    mask = np.triu(np.ones((T, T), bool), 1)
    for b in range(B):
        for h in range(NH):
            q = qkv[b, :, h * hs:(h + 1) * hs].astype(np.float64)
            k = qkv[b, :, C + h * hs:C + (h + 1) * hs].astype(np.float64)
            s = (q @ k.T) * (LOG2E / np.sqrt(hs))
            s[mask] = -np.inf
            sp = np.full((T, nb * block), -np.inf)
            sp[:, :T] = s
            bm = sp.reshape(T, nb, block).max(axis=2)
            prev = np.maximum.accumulate(bm, axis=1)[:, :-1]
            count += int(np.any(bm[:, 1:] > prev + slack, axis=1).sum())
    return count


SHAPES = [(1, 1024, 768, 12), (2, 300, 256, 4), (1, 77, 128, 2)]
KINDS = ["wide", "rising", "dominant"]


def _need(kind, B, T, NH):
    """Queries that must meet the condition: a share of the queries that have
    more than one key block (wide scores need a few blocks to beat the first)."""
    rows = B * NH * max(0, T - 64)
    if kind == "wide":
        return rows // 5 if T >= 256 else 0
    return max(1, rows // (2 if kind == "rising" else 10))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("B,T,C,NH", SHAPES)
def test_attention_rescale(dt, kind, B, T, C, NH):
    announce("attention-rescale", dt, kind, B, T, C, NH)
    d = DT[dt]
    qkv = make_qkv(kind, B, T, C, NH, d)
    assert rescale_queries(qkv, NH) >= _need(kind, B, T, NH)
    out = empty((B, T, C), d, fill=float("nan"))
    G.attention_forward(out, dev(qkv, d), NH)
    ref = oracle.attention(qkv, NH)
    got = host(out)
    assert np.all(np.isfinite(got))
    if d == I.BF16:
        vmax = float(np.abs(qkv[:, :, 2 * C:]).max())
        assert rel_err(got, ref) <= 1e-2
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * (np.abs(ref) + vmax))
    else:
        assert max_abs(got, ref) <= 1e-5


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("B,T,C,NH", SHAPES)
def test_attention_lse_rescale(dt, kind, B, T, C, NH):
    """The log-sum-exp written by attention_forward_lse after rescales, and
    its output equal to attention_forward's bit for bit."""
    announce("attention-lse-rescale", dt, kind, B, T, C, NH)
    d = DT[dt]
    qkv = make_qkv(kind, B, T, C, NH, d, seed=1)
    q = dev(qkv, d)
    out = empty((B, T, C), d)
    lse = empty((B, NH, T), I.F32, fill=float("nan"))
    G.attention_forward_lse(out, lse, q, NH)
    ref = oracle.attention_lse(qkv, NH)
    got = host(lse)
    assert np.all(np.abs(got - ref) <= lse_tol(d, ref))
    plain = empty((B, T, C), d)
    G.attention_forward(plain, q, NH)
    assert np.array_equal(host_bits(plain), host_bits(out))


def lse_tol(d, ref):
    """fp32: 2e-5 max(1, |lse|). bf16 adds 2^-8: the normaliser sums the
    probabilities as rounded to bf16 for the P.V product (relative error
    <= 2^-9 each, so the sum and its logarithm move by <= 2^-9)."""
    return 2e-5 * np.maximum(1.0, np.abs(ref)) + (2.0 ** -8 if d == I.BF16 else 0.0)


def _part_err(got, ref, part, C):
    g = np.asarray(got[..., part * C:(part + 1) * C], np.float64)
    r = np.asarray(ref[..., part * C:(part + 1) * C], np.float64)
    den = max(np.linalg.norm(r), 0.1 * np.linalg.norm(np.asarray(ref, np.float64)), 1e-300)
    return float(np.linalg.norm(g - r) / den)


def stored_output_term(dy, qkv, out_stored, NH):
    """First-order change of dqkv when D = rowsum(dO o O) is formed from the
    stored (bf16-rounded) forward output instead of the exact one.

    The backward rebuilds dS = P o (dP - D). With D' = D + dD, dS' = dS - P dD,
    so dq_t changes by -dD_t sum_j P_tj k_j / sqrt(hs), dk_j by
    -sum_t P_tj dD_t q_t / sqrt(hs), and dv not at all. The bf16 path stores
    the output in bf16 (the precision of every activation), as the
    FlashAttention backward keeps O; the oracle's D is exact. When the softmax
    is peaked on keys that share a large component along q (rising scores),
    this term is amplified by the ratio of the score level to the spread of
    the scores the softmax selects, and dominates the bf16 error of dq and dk;
    adding it to the oracle's gradient leaves the kernel's own rounding to the
    stated bound. P and the exact output come from the definition in float64."""
    B, T, C3 = qkv.shape
    C = C3 // 3
    hs = C // NH
    corr = np.zeros((B, T, C3), np.float64)
    mask = np.triu(np.ones((T, T), bool), 1)
    for b in range(B):
        for h in range(NH):
            sl = slice(h * hs, (h + 1) * hs)
            q = qkv[b, :, sl].astype(np.float64)
            k = qkv[b, :, C + h * hs:C + (h + 1) * hs].astype(np.float64)
            v = qkv[b, :, 2 * C + h * hs:2 * C + (h + 1) * hs].astype(np.float64)
            s = q @ k.T / np.sqrt(hs)
            s[mask] = -np.inf
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            o_exact = p @ v
            dd = np.sum(dy[b, :, sl].astype(np.float64) * (out_stored[b, :, sl].astype(np.float64) - o_exact), axis=1)
            corr[b, :, sl] = -(dd[:, None] * (p @ k)) / np.sqrt(hs)
            corr[b, :, C + h * hs:C + (h + 1) * hs] = -(p.T @ (dd[:, None] * q)) / np.sqrt(hs)
    return corr


def ds_rounding_error(dy, qkv, NH):
    """Norm-relative error of dq and dk when the exact dS = P o (dP - D) is
    rounded to bf16 once before the products dS K and dS^T Q, everything else
    exact (float64 from the definition).

    The bf16 backward feeds dS to the matrix cores in bf16. dq_t =
    sum_j dS_tj k_j / sqrt(hs) cancels (sum_j dS_tj = 0), so when the keys the
    softmax selects share a large component (scores rising along the keys)
    that rounding is amplified by roughly the scores' total rise, and the
    error of a correct kernel is dominated by it. The tolerance for dq and dk
    is twice this figure where it exceeds the usual bf16 bound."""
    B, T, C3 = qkv.shape
    C = C3 // 3
    hs = C // NH
    mask = np.triu(np.ones((T, T), bool), 1)
    sq = [0.0, 0.0]
    sk = [0.0, 0.0]
    for b in range(B):
        for h in range(NH):
            q = qkv[b, :, h * hs:(h + 1) * hs].astype(np.float64)
            k = qkv[b, :, C + h * hs:C + (h + 1) * hs].astype(np.float64)
            v = qkv[b, :, 2 * C + h * hs:2 * C + (h + 1) * hs].astype(np.float64)
            do = dy[b, :, h * hs:(h + 1) * hs].astype(np.float64)
            s = q @ k.T / np.sqrt(hs)
            s[mask] = -np.inf
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            ds = p * (do @ v.T - np.sum(do * (p @ v), axis=1)[:, None])
            dsr = I.round_to_bf16(ds.astype(np.float32)).astype(np.float64)
            gq, gk = ds @ k, ds.T @ q
            sq[0] += float(np.sum(((dsr - ds) @ k) ** 2))
            sq[1] += float(np.sum(gq ** 2))
            sk[0] += float(np.sum(((dsr - ds).T @ q) ** 2))
            sk[1] += float(np.sum(gk ** 2))
    return np.sqrt(sq[0] / max(sq[1], 1e-300)), np.sqrt(sk[0] / max(sk[1], 1e-300))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("B,T,C,NH", [(1, 1024, 128, 2), (2, 300, 128, 2), (1, 77, 64, 1)])
def test_attention_backward_rescale(dt, kind, B, T, C, NH):
    """attention_backward on the lse and output of a forward that rescaled."""
    announce("attention-backward-rescale", dt, kind, B, T, C, NH)
    d = DT[dt]
    qkv = make_qkv(kind, B, T, C, NH, d, seed=2)
    assert rescale_queries(qkv, NH) >= _need(kind, B, T, NH)
    dy = I.random_tensor(2000 + T, (B, T, C), 1.0, d)
    q = dev(qkv, d)
    out = empty((B, T, C), d)
    lse = empty((B, NH, T), I.F32)
    G.attention_forward_lse(out, lse, q, NH)
    dq = empty((B, T, 3 * C), d, fill=float("nan"))
    import torch
    w = torch.empty(max(1, G.attention_backward_workspace_size(B, T, C, NH)), dtype=torch.uint8, device="cuda")
    G.attention_backward(dq, dev(dy, d), q, out, lse, NH, w)
    ref = oracle.attention_backward(dy, qkv, NH)
    tols = [2e-5] * 3
    if d == I.BF16:
        ref = ref + stored_output_term(dy, qkv, host(out), NH)
        eq, ek = ds_rounding_error(dy, qkv, NH)
        tols = [max(3e-2, 2 * eq), max(3e-2, 2 * ek), 3e-2]
    got = host(dq)
    assert np.all(np.isfinite(got))
    for part in range(3):
        assert _part_err(got, ref, part, C) <= tols[part], (part, _part_err(got, ref, part, C), tols[part])
