"""ctypes wrapper around the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: used by the test suite, the smoke check and the
benchmark's CPU-baseline leg. It imports nothing from the GPU package and the
GPU package imports nothing from here. All arrays are numpy float32/int32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")
_lock = threading.Lock()
_lib = None

CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-std=gnu11", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain C, libm only)."""
    if not force and os.path.exists(_SO) and os.path.getmtime(_SO) >= os.path.getmtime(_SRC):
        return _SO
    tmp = _SO + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], cwd=_HERE)
    os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        build(force=False)
        lib = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        I = ctypes.c_int
        I64 = ctypes.c_int64
        D = ctypes.c_double
        sig = {
            "oracle_encoder": (None, [P, P, P, P, I, I, I]),
            "oracle_layernorm": (None, [P, P, P, P, P, P, I, I, D]),
            "oracle_matmul": (None, [P, P, P, P, I, I, I]),
            "oracle_attention": (None, [P, P, I, I, I, I]),
            "oracle_gelu": (None, [P, P, I64]),
            "oracle_residual": (None, [P, P, P, I64]),
            "oracle_softmax": (None, [P, P, I, I, I]),
            "oracle_crossentropy": (None, [P, P, P, I, I, I]),
            "oracle_param_count": (I64, [I, I, I, I]),
            "oracle_capture_count": (I64, [I, I, I, I]),
            "oracle_forward": (I, [P, P, P, P, I, I, I, I, I, I, D, I, I, P]),
            "oracle_decode_step": (I, [P, P, P, I, P, P, P, I, I, I, I, I, I, D, I]),
            "oracle_crossentropy_backward": (None, [P, P, P, D, I, I, I]),
            "oracle_matmul_backward": (None, [P, P, P, P, P, P, I, I, I]),
            "oracle_layernorm_backward": (None, [P, P, P, P, P, P, I, I, D]),
            "oracle_gelu_backward": (None, [P, P, P, I64]),
            "oracle_attention_lse": (None, [P, P, I, I, I, I]),
            "oracle_attention_backward": (None, [P, P, P, I, I, I, I]),
            "oracle_encoder_backward": (None, [P, P, P, P, I, I, I]),
            "oracle_backward": (I, [P, P, P, P, P, I, I, I, I, I, I, D, I, I]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def _f32(x):
    a = np.ascontiguousarray(x, dtype=np.float32)
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


def encoder(tokens, wte, wpe):
    lib = _load()
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    B, T = tokens.shape
    wte, wpe = _f32(wte), _f32(wpe)
    C = wte.shape[1]
    out = np.empty((B, T, C), np.float32)
    lib.oracle_encoder(_ptr(out), _ptr(tokens), _ptr(wte), _ptr(wpe), B, T, C)
    return out


def layernorm(x, gamma, beta, eps=1e-5, return_stats=False):
    lib = _load()
    x = _f32(x)
    C = x.shape[-1]
    N = x.size // C
    out = np.empty_like(x)
    mean = np.empty(N, np.float32)
    rstd = np.empty(N, np.float32)
    lib.oracle_layernorm(_ptr(out), _ptr(mean), _ptr(rstd), _ptr(x), _ptr(_f32(gamma)),
                         _ptr(_f32(beta)), N, C, float(eps))
    return (out, mean, rstd) if return_stats else out


def matmul(x, weight, bias=None):
    lib = _load()
    x = _f32(x)
    weight = _f32(weight)
    C = x.shape[-1]
    N = x.size // C
    OC = weight.shape[0]
    assert weight.shape == (OC, C)
    b = None if bias is None else _f32(bias)
    out = np.empty(x.shape[:-1] + (OC,), np.float32)
    lib.oracle_matmul(_ptr(out), _ptr(x), _ptr(weight), _ptr(b), N, C, OC)
    return out


def attention(qkv, NH):
    lib = _load()
    qkv = _f32(qkv)
    B, T, C3 = qkv.shape
    C = C3 // 3
    out = np.empty((B, T, C), np.float32)
    lib.oracle_attention(_ptr(out), _ptr(qkv), B, T, C, NH)
    return out


def gelu(x):
    lib = _load()
    x = _f32(x)
    out = np.empty_like(x)
    lib.oracle_gelu(_ptr(out), _ptr(x), x.size)
    return out


def residual(a, b):
    lib = _load()
    a, b = _f32(a), _f32(b)
    out = np.empty_like(a)
    lib.oracle_residual(_ptr(out), _ptr(a), _ptr(b), a.size)
    return out


def softmax(logits, V):
    lib = _load()
    logits = _f32(logits)
    Vp = logits.shape[-1]
    N = logits.size // Vp
    out = np.empty_like(logits)
    lib.oracle_softmax(_ptr(out), _ptr(logits), N, V, Vp)
    return out


def crossentropy(logits, targets, V):
    """Per-row losses [N] = log-sum-exp over v < V minus the target's logit."""
    lib = _load()
    logits = _f32(logits)
    Vp = logits.shape[-1]
    N = logits.size // Vp
    targets = np.ascontiguousarray(targets, dtype=np.int32).reshape(N)
    assert np.all((targets >= 0) & (targets < V))
    out = np.empty(N, np.float32)
    lib.oracle_crossentropy(_ptr(out), _ptr(logits), _ptr(targets), N, V, Vp)
    return out


def param_count(L, C, maxT, Vp):
    return int(_load().oracle_param_count(L, C, maxT, Vp))


def forward(tokens, params, L, C, NH, V, Vp, maxT, eps=1e-5, probs=True, capture=False):
    """Returns (logits [B,T,Vp], probs or None, capture dict or None)."""
    lib = _load()
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    B, T = tokens.shape
    params = _f32(params)
    assert params.size == param_count(L, C, maxT, Vp)
    logits = np.empty((B, T, Vp), np.float32)
    pr = np.empty((B, T, Vp), np.float32) if probs else None
    capbuf = np.empty(int(lib.oracle_capture_count(L, C, B, T)), np.float32) if capture else None
    rc = lib.oracle_forward(_ptr(logits), _ptr(pr), _ptr(tokens), _ptr(params), L, C, NH, V, Vp,
                            maxT, float(eps), B, T, _ptr(capbuf))
    if rc != 0:
        raise RuntimeError("oracle_forward failed with code %d" % rc)
    cap = None
    if capture:
        N = B * T
        cap = {}
        off = 0

        def take(name, width):
            nonlocal off
            cap[name] = capbuf[off:off + N * width].reshape(B, T, width)
            off += N * width

        take("encoder", C)
        for l in range(L):
            for nm, wd in (("ln1", C), ("qkv", 3 * C), ("attn", C), ("attproj", C), ("res1", C),
                           ("ln2", C), ("fc", 4 * C), ("gelu", 4 * C), ("fcproj", C), ("res2", C)):
                take("%s.%d" % (nm, l), wd)
        take("lnf", C)
        assert off == capbuf.size
    return logits, pr, cap


def decode_step(tokens, pos, kcache, vcache, params, L, C, NH, V, Vp, maxT, eps=1e-5, probs=True):
    """kcache/vcache [L,B,NH,maxT,hs] float32, updated in place at pos.
    Returns (logits [B,Vp], probs or None)."""
    lib = _load()
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    B = tokens.shape[0]
    assert kcache.dtype == np.float32 and kcache.flags.c_contiguous
    assert vcache.dtype == np.float32 and vcache.flags.c_contiguous
    params = _f32(params)
    logits = np.empty((B, Vp), np.float32)
    pr = np.empty((B, Vp), np.float32) if probs else None
    rc = lib.oracle_decode_step(_ptr(logits), _ptr(pr), _ptr(tokens), int(pos), _ptr(kcache),
                                _ptr(vcache), _ptr(params), L, C, NH, V, Vp, maxT, float(eps), B)
    if rc != 0:
        raise RuntimeError("oracle_decode_step failed with code %d" % rc)
    return logits, pr


# ------------------------------------------------------------------ backward


def crossentropy_backward(logits, targets, V, dloss):
    """dlogits [N,Vp] = dloss * (softmax - onehot(target)) on v < V, 0 in the padding."""
    lib = _load()
    logits = _f32(logits)
    Vp = logits.shape[-1]
    N = logits.size // Vp
    targets = np.ascontiguousarray(targets, dtype=np.int32).reshape(N)
    assert np.all((targets >= 0) & (targets < V))
    out = np.empty_like(logits)
    lib.oracle_crossentropy_backward(_ptr(out), _ptr(logits), _ptr(targets), float(dloss), N, V, Vp)
    return out


def matmul_backward(dout, x, weight):
    """Returns (dinp [N,C], dweight [OC,C], dbias [OC]) for out = x W^T + b."""
    lib = _load()
    dout, x, weight = _f32(dout), _f32(x), _f32(weight)
    OC, C = weight.shape
    N = x.size // C
    assert dout.size == N * OC
    dinp = np.empty(x.shape, np.float32)
    dw = np.empty((OC, C), np.float32)
    db = np.empty(OC, np.float32)
    lib.oracle_matmul_backward(_ptr(dinp), _ptr(dw), _ptr(db), _ptr(dout), _ptr(x), _ptr(weight), N, C, OC)
    return dinp, dw, db


def layernorm_backward(dout, x, gamma, eps=1e-5):
    """Returns (dinp, dgamma, dbeta)."""
    lib = _load()
    dout, x, gamma = _f32(dout), _f32(x), _f32(gamma)
    C = x.shape[-1]
    N = x.size // C
    dinp = np.empty_like(x)
    dg = np.empty(C, np.float32)
    db = np.empty(C, np.float32)
    lib.oracle_layernorm_backward(_ptr(dinp), _ptr(dg), _ptr(db), _ptr(dout), _ptr(x), _ptr(gamma), N, C,
                                  float(eps))
    return dinp, dg, db


def gelu_backward(x, dout):
    lib = _load()
    x, dout = _f32(x), _f32(dout)
    out = np.empty_like(x)
    lib.oracle_gelu_backward(_ptr(out), _ptr(x), _ptr(dout), x.size)
    return out


def attention_lse(qkv, NH):
    """lse [B,NH,T] of the causal scaled scores."""
    lib = _load()
    qkv = _f32(qkv)
    B, T, C3 = qkv.shape
    out = np.empty((B, NH, T), np.float32)
    lib.oracle_attention_lse(_ptr(out), _ptr(qkv), B, T, C3 // 3, NH)
    return out


def attention_backward(dout, qkv, NH):
    """dqkv [B,T,3C] for y = attention(qkv) and the incoming dout [B,T,C]."""
    lib = _load()
    qkv, dout = _f32(qkv), _f32(dout)
    B, T, C3 = qkv.shape
    out = np.empty_like(qkv)
    lib.oracle_attention_backward(_ptr(out), _ptr(dout), _ptr(qkv), B, T, C3 // 3, NH)
    return out


def encoder_backward(dout, tokens, Vp, maxT, dwte=None, dwpe=None):
    """Accumulates into (copies of) dwte [Vp,C] and dwpe [maxT,C] (zeros if None)."""
    lib = _load()
    dout = _f32(dout)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    B, T = tokens.shape
    C = dout.shape[-1]
    dwte = np.zeros((Vp, C), np.float32) if dwte is None else _f32(dwte).copy()
    dwpe = np.zeros((maxT, C), np.float32) if dwpe is None else _f32(dwpe).copy()
    lib.oracle_encoder_backward(_ptr(dwte), _ptr(dwpe), _ptr(dout), _ptr(tokens), B, T, C)
    return dwte, dwpe


def backward(tokens, targets, params, L, C, NH, V, Vp, maxT, eps=1e-5):
    """Gradient of the mean cross-entropy w.r.t. the flat parameters.
    Returns (grads [P] float32, mean loss)."""
    lib = _load()
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    targets = np.ascontiguousarray(targets, dtype=np.int32)
    B, T = tokens.shape
    assert targets.shape == (B, T) and np.all((targets >= 0) & (targets < V))
    params = _f32(params)
    assert params.size == param_count(L, C, maxT, Vp)
    grads = np.empty_like(params)
    loss = np.zeros(1, np.float32)
    rc = lib.oracle_backward(_ptr(grads), _ptr(loss), _ptr(tokens), _ptr(targets), _ptr(params), L, C, NH, V,
                             Vp, maxT, float(eps), B, T)
    if rc != 0:
        raise RuntimeError("oracle_backward failed with code %d" % rc)
    return grads, float(loss[0])
