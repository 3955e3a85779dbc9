"""Oracle runs for the full-size forward checks, started in background threads.

A full-length GPT-2 sequence takes the single-threaded oracle about a minute
(124M) or more (350M). The ctypes call releases the GIL, so the runs proceed
in parallel with each other and with the GPU tests that come before the
full-size ones; each full-size test then waits for its own run.

Which sequence and how many positions each workload checks:
  small, small_bf16_b4   the last sequence, all 1024 positions
  small_bf16_b8          the last sequence, all 1024 positions
  medium                 the last sequence, positions 0..511
Positions are a prefix because the oracle, like the model, is causal: the
first t positions of a full-length run are exactly a run on those t tokens.
"""
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

FULL_CHECK = {"small": 1024, "small_bf16_b4": 1024, "small_bf16_b8": 1024, "medium": 512}

_lock = threading.Lock()
_pool = None
_futures = {}


def _run(name):
    import oracle
    from transformer_forward_pass_gpt_amd import inputs as I
    w = I.WORKLOADS[name]
    params = I.make_params(w)
    tok = I.make_tokens(w)
    seq = w.B - 1
    t_check = FULL_CHECK[name]
    rl, rp, _ = oracle.forward(tok[seq:seq + 1, :t_check], params, w.L, w.C, w.NH, w.V, w.Vp, w.maxT, w.ln_eps)
    return seq, t_check, rl[0], rp[0]


def prefetch(names):
    """Start the oracle runs of these workloads (idempotent)."""
    global _pool
    with _lock:
        if _pool is None:
            _pool = ThreadPoolExecutor(max_workers=len(FULL_CHECK), thread_name_prefix="oracle")
        for n in names:
            if n in FULL_CHECK and n not in _futures:
                _futures[n] = _pool.submit(_run, n)


def get(name):
    """(sequence index, positions, logits [t,Vp], probs [t,Vp]) for a workload."""
    prefetch([name])
    seq, t, rl, rp = _futures[name].result()
    return seq, t, np.asarray(rl), np.asarray(rp)
