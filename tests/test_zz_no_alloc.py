"""gpt2_decode_step_noalloc (the decode step on the library's own device
scratch, for callers that cannot allocate) against gpt2_decode_step with a
caller workspace: the same kernels on the same inputs, so logits,
probabilities and the updated caches must agree bit for bit. Two calls in a
row, the second on fewer sequences, so stale scratch contents from the first
call cannot leak into the second."""
import sys

import numpy as np
import pytest

import transformer_forward_pass_gpt_amd as G
from transformer_forward_pass_gpt_amd import inputs as I

from gpu_util import dev, dev_int, empty, host_bits

pytestmark = pytest.mark.gpu


def announce(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _step_both(w, params, cfg, tok, pos, kc, vc, with_probs=True):
    """One step through each entry, each on its own copy of the caches."""
    import torch
    B = tok.shape[0]
    outs = []
    for noalloc in (False, True):
        tk, tv = dev(kc, w.dtype), dev(vc, w.dtype)
        logits = empty((B, w.Vp), w.dtype, fill=float("nan"))
        probs = empty((B, w.Vp), w.dtype, fill=float("nan")) if with_probs else None
        if noalloc:
            G.gpt2_decode_step_noalloc(logits, probs, dev_int(tok), pos, tk, tv, params, cfg)
        else:
            ws = torch.empty(G.decode_workspace_bytes(cfg, B), dtype=torch.uint8, device="cuda")
            G.gpt2_decode_step(logits, probs, dev_int(tok), pos, tk, tv, params, cfg, ws)
        torch.cuda.synchronize()
        outs.append((host_bits(logits), host_bits(probs) if with_probs else None, host_bits(tk), host_bits(tv)))
    return outs


@pytest.mark.parametrize("name", ["decode", "tiny"])
def test_decode_noalloc_matches_workspace_entry(name):
    announce("decode-noalloc", name)
    w = I.WORKLOADS[name]
    cfg = G.make_config(w.L, w.C, w.NH, w.V, w.Vp, w.maxT, w.dtype, w.ln_eps)
    params = dev(I.make_params(w), w.dtype)
    hs = w.C // w.NH
    B0 = 32 if name == "decode" else 4
    rng = np.random.default_rng(7)
    # first call: B0 sequences at the last position; second: 7 (or 3) sequences at an earlier one
    for B, pos in ((B0, w.maxT - 1), (7 if name == "decode" else 3, w.maxT // 2)):
        kc = rng.standard_normal((w.L, B, w.NH, w.maxT, hs), dtype=np.float32)
        vc = rng.standard_normal((w.L, B, w.NH, w.maxT, hs), dtype=np.float32)
        if w.dtype == I.BF16:
            kc, vc = I.round_to_bf16(kc), I.round_to_bf16(vc)
        tok = rng.integers(0, w.V, B).astype(np.int32)
        (la, pa, ka, va), (lb, pb, kb, vb) = _step_both(w, params, cfg, tok, pos, kc, vc, with_probs=(B == B0))
        assert np.array_equal(la, lb), (B, pos)
        if pa is not None:
            assert np.array_equal(pa, pb), (B, pos)
        assert np.array_equal(ka, kb) and np.array_equal(va, vb), (B, pos)
        assert not np.any(np.isnan(la.view(np.uint32) if w.dtype == I.F32 else la.astype(np.float32)))
