"""GPT-2 forward pass on AMD MI355X (gfx950): Python binding of libgpt2fwd.so.

Thin ctypes marshalling over the C ABI declared in include/gpt2fwd.h: every
function takes torch tensors that already live on the GPU, passes their
device pointers and the current HIP stream, and raises on a nonzero status.
All compute happens in the HIP kernels; there is no CPU or PyTorch fallback:
if the library is missing, every call raises.

The library is loaded on first use, so ``transformer_forward_pass_gpt_amd.inputs``
can be imported on a machine without a GPU or a built library.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgpt2fwd.so")

F32 = 0
BF16 = 1

OK = 0
ERR_INVALID_ARGUMENT = -1
ERR_UNSUPPORTED = -2
ERR_HIP = -3
ERR_WORKSPACE_TOO_SMALL = -4

EXPORTS = (
    "encoder_forward", "layernorm_forward", "matmul_forward", "attention_forward",
    "gelu_forward", "residual_forward", "softmax_forward", "gpt2_param_count",
    "gpt2_workspace_bytes", "gpt2_forward", "attention_decode_workspace_bytes",
    "attention_decode_forward", "gpt2_decode_workspace_bytes", "gpt2_decode_step",
    "gpt2_status_string", "gpt2_last_hip_error", "matmul_kernel_config",
    "matmul_splitk_forward", "matmul_splitk_count", "matmul_gelu_forward", "residual_layernorm_forward",
    "matmul_residual_forward", "argmax_forward", "gpt2_prefill", "gpt2_generate_workspace_bytes",
    "gpt2_generate", "crossentropy_forward",
    "crossentropy_backward", "gelu_backward", "layernorm_backward_workspace_size", "layernorm_backward",
    "matmul_backward_workspace_size", "matmul_backward", "attention_forward_lse",
    "attention_backward_workspace_size", "attention_backward", "encoder_backward", "gpt2_train_acts_bytes",
    "gpt2_train_workspace_bytes", "gpt2_train_forward", "gpt2_backward", "gpt2_decode_step_noalloc",
    "matmul_logits_stats_forward", "softmax_stats_forward",
)

DECODE_SCRATCH_BYTES = 8 << 20  # GPT2_DECODE_SCRATCH_BYTES of the header


class GPT2Error(RuntimeError):
    def __init__(self, fn, status, lib):
        msg = lib.gpt2_status_string(status).decode()
        if status == ERR_HIP:
            msg += " (hipError %d)" % lib.gpt2_last_hip_error()
        super().__init__("%s failed: %s [%d]" % (fn, msg, status))
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int), ("C", ctypes.c_int), ("NH", ctypes.c_int),
                ("V", ctypes.c_int), ("Vp", ctypes.c_int), ("maxT", ctypes.c_int),
                ("dtype", ctypes.c_int), ("ln_eps", ctypes.c_float)]


_lock = threading.Lock()
_lib = None


def load_library(path: str = LIB_PATH):
    """Load libgpt2fwd.so and declare the signatures. Raises if it is missing."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError("libgpt2fwd.so not built (%s); run "
                               "`python -m transformer_forward_pass_gpt_amd.build`" % path)
        lib = ctypes.CDLL(path)
        P, I, I64, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        CP = ctypes.POINTER(Config)
        sig = {
            "encoder_forward": (I, [P, P, P, P, I, I, I, I, P]),
            "layernorm_forward": (I, [P, P, P, P, P, P, I, I, F, I, P]),
            "matmul_forward": (I, [P, P, P, P, I, I, I, I, P]),
            "attention_forward": (I, [P, P, I, I, I, I, I, P]),
            "gelu_forward": (I, [P, P, I64, I, P]),
            "residual_forward": (I, [P, P, P, I64, I, P]),
            "softmax_forward": (I, [P, P, I, I, I, I, P]),
            "gpt2_param_count": (I64, [CP]),
            "gpt2_workspace_bytes": (I64, [CP, I, I]),
            "gpt2_forward": (I, [P, P, P, P, CP, I, I, P, I64, P]),
            "attention_decode_workspace_bytes": (I64, [I, I, I, I]),
            "attention_decode_forward": (I, [P, P, P, P, I, I, I, I, I, I, P, I64, P]),
            "gpt2_decode_workspace_bytes": (I64, [CP, I]),
            "gpt2_decode_step": (I, [P, P, P, I, P, P, P, CP, I, P, I64, P]),
            "gpt2_status_string": (ctypes.c_char_p, [I]),
            "gpt2_last_hip_error": (I, []),
            "matmul_kernel_config": (ctypes.c_char_p, [I, I, I, I]),
            "matmul_splitk_forward": (I, [P, P, P, I, I, I, I, I, P]),
            "matmul_splitk_count": (I, [I, I, I]),
            "matmul_gelu_forward": (I, [P, P, P, P, I, I, I, I, P]),
            "matmul_residual_forward": (I, [P, P, P, P, P, I, I, I, I, P]),
            "argmax_forward": (I, [P, P, I, I, I, I, P]),
            "crossentropy_forward": (I, [P, P, P, P, P, I, I, I, I, P]),
            "gpt2_prefill": (I, [P, P, P, P, P, P, CP, I, I, P, I64, P]),
            "gpt2_generate_workspace_bytes": (I64, [CP, I, I]),
            "gpt2_generate": (I, [P, P, I, P, P, P, CP, I, I, P, I64, P]),
            "residual_layernorm_forward": (I, [P, P, P, I, P, P, P, I, I, F, I, P]),
            "crossentropy_backward": (I, [P, P, P, P, P, F, I, I, I, I, P]),
            "gelu_backward": (I, [P, P, P, I64, I, P]),
            "layernorm_backward_workspace_size": (I64, [I, I]),
            "layernorm_backward": (I, [P, P, P, P, P, P, P, P, P, I, I, I, P, I64, P]),
            "matmul_backward_workspace_size": (I64, [I, I, I, I]),
            "matmul_backward": (I, [P, P, P, P, P, P, I, I, I, I, P, I64, P]),
            "attention_forward_lse": (I, [P, P, P, I, I, I, I, I, P]),
            "attention_backward_workspace_size": (I64, [I, I, I, I]),
            "attention_backward": (I, [P, P, P, P, P, I, I, I, I, I, P, I64, P]),
            "encoder_backward": (I, [P, P, P, P, I, I, I, I, P]),
            "gpt2_train_acts_bytes": (I64, [CP, I, I]),
            "gpt2_train_workspace_bytes": (I64, [CP, I, I]),
            "gpt2_train_forward": (I, [P, P, P, P, P, CP, I, I, P, I64, P]),
            "gpt2_backward": (I, [P, P, P, CP, I, I, P, I64, P, I64, P]),
            "gpt2_decode_step_noalloc": (I, [P, P, P, I, P, P, P, CP, I, P]),
            "matmul_logits_stats_forward": (I, [P, P, P, P, I, I, I, I, I, P]),
            "softmax_stats_forward": (I, [P, P, P, I, I, I, I, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


# ------------------------------------------------------------------ helpers
def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("tensor dtype must be float32 or bfloat16, got %s" % t.dtype)


def _tdt(code):
    torch = _torch()
    return torch.bfloat16 if code == BF16 else torch.float32


def _chk(t, name, dtype=None, numel=None, ndim=None, min_numel=None, optional=False):
    """Shape and dtype check of one tensor argument, before any pointer is
    taken: a caller mistake becomes a ValueError here rather than an
    out-of-bounds access on the GPU."""
    if t is None:
        if optional:
            return
        raise ValueError("%s is required" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dimensions, got shape %s" % (name, ndim, tuple(t.shape)))
    if numel is not None and t.numel() != numel:
        raise ValueError("%s must hold %d elements, got %d (shape %s)" % (name, numel, t.numel(), tuple(t.shape)))
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError("%s must hold at least %d elements, got %d" % (name, min_numel, t.numel()))


def _int32(t, name, numel=None, ndim=None, optional=False):
    _chk(t, name, dtype=_torch().int32, numel=numel, ndim=ndim, optional=optional)


def _f32t(t, name, numel=None, ndim=None, min_numel=None, optional=False):
    _chk(t, name, dtype=_torch().float32, numel=numel, ndim=ndim, min_numel=min_numel, optional=optional)


def _last(t, name):
    if t.dim() < 1:
        raise ValueError("%s must have at least one dimension" % name)
    return t.shape[-1]


def _dev(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _stream(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(fn, status):
    if status != OK:
        raise GPT2Error(fn, status, load_library())


def make_config(L, C, NH, V, Vp, maxT, dtype, ln_eps=1e-5) -> Config:
    return Config(L, C, NH, V, Vp, maxT, dtype, ln_eps)


# ------------------------------------------------------------------ per-step entries
def encoder_forward(out, tokens, wte, wpe, stream=None):
    """out [B,T,C] = wte[tokens] + wpe[:T]; tokens int32 [B,T]."""
    lib = load_library()
    _int32(tokens, "tokens", ndim=2)
    B, T = tokens.shape
    dt = _dtype_code(out)
    _chk(wte, "wte", dtype=out.dtype, ndim=2)
    C = wte.shape[1]
    _chk(wpe, "wpe", dtype=out.dtype, ndim=2)
    if wpe.shape[1] != C or wpe.shape[0] < T:
        raise ValueError("wpe must be [>=%d, %d], got %s" % (T, C, tuple(wpe.shape)))
    _chk(out, "out", numel=B * T * C)
    _check("encoder_forward", lib.encoder_forward(
        _dev(out, "out"), _dev(tokens, "tokens"), _dev(wte, "wte"), _dev(wpe, "wpe"),
        B, T, C, dt, _stream(stream)))
    return out


def layernorm_forward(out, inp, gamma, beta, eps=1e-5, mean=None, rstd=None, stream=None):
    """out = LayerNorm(inp) over the last dimension; mean, rstd fp32 [N] (optional)."""
    lib = load_library()
    dt = _dtype_code(inp)
    C = _last(inp, "inp")
    N = inp.numel() // C if C else 0
    _chk(out, "out", dtype=inp.dtype, numel=inp.numel())
    _chk(gamma, "gamma", dtype=inp.dtype, numel=C)
    _chk(beta, "beta", dtype=inp.dtype, numel=C)
    _f32t(mean, "mean", numel=N, optional=True)
    _f32t(rstd, "rstd", numel=N, optional=True)
    _check("layernorm_forward", lib.layernorm_forward(
        _dev(out, "out"), _dev(mean, "mean"), _dev(rstd, "rstd"), _dev(inp, "inp"),
        _dev(gamma, "gamma"), _dev(beta, "beta"), N, C, float(eps), dt, _stream(stream)))
    return out


def _linear_args(inp, weight, bias):
    """(N, C, OC) of a linear layer, with weight [OC,C] and bias [OC] checked."""
    C = _last(inp, "inp")
    N = inp.numel() // C if C else 0
    _chk(weight, "weight", dtype=inp.dtype, ndim=2)
    if weight.shape[1] != C:
        raise ValueError("weight must be [OC, %d], got %s" % (C, tuple(weight.shape)))
    OC = weight.shape[0]
    _chk(bias, "bias", dtype=inp.dtype, numel=OC, optional=True)
    return N, C, OC


def matmul_forward(out, inp, weight, bias=None, stream=None):
    """out [N,OC] = inp [N,C] @ weight[OC,C]^T + bias."""
    lib = load_library()
    dt = _dtype_code(inp)
    N, C, OC = _linear_args(inp, weight, bias)
    _chk(out, "out", dtype=inp.dtype, numel=N * OC)
    _check("matmul_forward", lib.matmul_forward(
        _dev(out, "out"), _dev(inp, "inp"), _dev(weight, "weight"), _dev(bias, "bias"),
        N, C, OC, dt, _stream(stream)))
    return out


def matmul_kernel_config(N, C, OC, dtype) -> str:
    """Name of the GEMM kernel configuration matmul_forward uses for this shape."""
    return load_library().matmul_kernel_config(N, C, OC, dtype).decode()


def matmul_splitk_forward(part, inp, weight, splits, stream=None):
    """part fp32 [splits,N,OC]: k-range partial sums of inp [N,C] @ weight[OC,C]^T (N <= 32)."""
    lib = load_library()
    dt = _dtype_code(inp)
    N, C, OC = _linear_args(inp, weight, None)
    _f32t(part, "part", numel=int(splits) * N * OC)
    _check("matmul_splitk_forward", lib.matmul_splitk_forward(
        _dev(part, "part"), _dev(inp, "inp"), _dev(weight, "weight"), N, C, OC, int(splits),
        dt, _stream(stream)))
    return part


def matmul_splitk_count(C, OC, dtype) -> int:
    """Split count the decode step uses for a C -> OC projection."""
    return int(load_library().matmul_splitk_count(C, OC, dtype))


def matmul_gelu_forward(out, inp, weight, bias=None, stream=None):
    """out [N,OC] = gelu(inp [N,C] @ weight[OC,C]^T + bias)."""
    lib = load_library()
    dt = _dtype_code(inp)
    N, C, OC = _linear_args(inp, weight, bias)
    _chk(out, "out", dtype=inp.dtype, numel=N * OC)
    _check("matmul_gelu_forward", lib.matmul_gelu_forward(
        _dev(out, "out"), _dev(inp, "inp"), _dev(weight, "weight"), _dev(bias, "bias"),
        N, C, OC, dt, _stream(stream)))
    return out


def matmul_residual_forward(out, inp, weight, bias, res, stream=None):
    """out [N,OC] = res + (inp [N,C] @ weight[OC,C]^T + bias); res may be out."""
    lib = load_library()
    dt = _dtype_code(inp)
    N, C, OC = _linear_args(inp, weight, bias)
    _chk(out, "out", dtype=inp.dtype, numel=N * OC)
    _chk(res, "res", dtype=inp.dtype, numel=N * OC)
    _check("matmul_residual_forward", lib.matmul_residual_forward(
        _dev(out, "out"), _dev(inp, "inp"), _dev(weight, "weight"), _dev(bias, "bias"), _dev(res, "res"),
        N, C, OC, dt, _stream(stream)))
    return out


def residual_layernorm_forward(out, x, part, bias, gamma, beta, eps=1e-5, stream=None):
    """x [N,C] += bias + sum_s part[s] (in place); out = LayerNorm(x)."""
    lib = load_library()
    dt = _dtype_code(x)
    C = _last(x, "x")
    N = x.numel() // C if C else 0
    _f32t(part, "part", ndim=3)
    splits = part.shape[0]
    _f32t(part, "part", numel=splits * N * C)
    _chk(out, "out", dtype=x.dtype, numel=N * C)
    for t, nm in ((bias, "bias"), (gamma, "gamma"), (beta, "beta")):
        _chk(t, nm, dtype=x.dtype, numel=C)
    _check("residual_layernorm_forward", lib.residual_layernorm_forward(
        _dev(out, "out"), _dev(x, "x"), _dev(part, "part"), splits, _dev(bias, "bias"), _dev(gamma, "gamma"),
        _dev(beta, "beta"), N, C, float(eps), dt, _stream(stream)))
    return out


def _qkv_dims(qkv):
    _chk(qkv, "qkv", ndim=3)
    B, T, C3 = qkv.shape
    if C3 % 3:
        raise ValueError("qkv's last dimension must be 3C, got %d" % C3)
    return B, T, C3 // 3


def attention_forward(out, qkv, NH, stream=None):
    """out [B,T,C] from qkv [B,T,3C], causal, NH heads."""
    lib = load_library()
    dt = _dtype_code(qkv)
    B, T, C = _qkv_dims(qkv)
    _chk(out, "out", dtype=qkv.dtype, numel=B * T * C)
    _check("attention_forward", lib.attention_forward(
        _dev(out, "out"), _dev(qkv, "qkv"), B, T, C, NH, dt, _stream(stream)))
    return out


def gelu_forward(out, inp, stream=None):
    lib = load_library()
    dt = _dtype_code(inp)
    _chk(out, "out", dtype=inp.dtype, numel=inp.numel())
    _check("gelu_forward", lib.gelu_forward(_dev(out, "out"), _dev(inp, "inp"), inp.numel(),
                                            dt, _stream(stream)))
    return out


def residual_forward(out, a, b, stream=None):
    lib = load_library()
    dt = _dtype_code(a)
    _chk(b, "b", dtype=a.dtype, numel=a.numel())
    _chk(out, "out", dtype=a.dtype, numel=a.numel())
    _check("residual_forward", lib.residual_forward(_dev(out, "out"), _dev(a, "a"), _dev(b, "b"),
                                                    a.numel(), dt, _stream(stream)))
    return out


def _vocab_dims(logits, V):
    _chk(logits, "logits", ndim=2)
    N, Vp = logits.shape
    if not 0 < V <= Vp:
        raise ValueError("V must lie in [1, %d], got %d" % (Vp, V))
    return N, Vp


def crossentropy_forward(losses, logits, targets, V, probs=None, mean_loss=None, stream=None):
    """losses fp32 [N] (and probs [N,Vp], mean_loss fp32 [1] when given) from logits [N,Vp]."""
    lib = load_library()
    dt = _dtype_code(logits)
    N, Vp = _vocab_dims(logits, V)
    _f32t(losses, "losses", numel=N)
    _f32t(mean_loss, "mean_loss", numel=1, optional=True)
    _chk(probs, "probs", dtype=logits.dtype, numel=N * Vp, optional=True)
    _int32(targets, "targets", numel=N)
    _check("crossentropy_forward", lib.crossentropy_forward(
        _dev(losses, "losses"), _dev(mean_loss, "mean_loss"), _dev(probs, "probs"), _dev(logits, "logits"),
        _dev(targets, "targets"), N, V, Vp, dt, _stream(stream)))
    return losses


def softmax_forward(probs, logits, V, stream=None):
    """probs [N,Vp] = softmax over the first V columns of logits; padding -> 0."""
    lib = load_library()
    dt = _dtype_code(logits)
    Vp = _last(logits, "logits")
    N = logits.numel() // Vp if Vp else 0
    if not 0 < V <= Vp:
        raise ValueError("V must lie in [1, %d], got %d" % (Vp, V))
    _chk(probs, "probs", dtype=logits.dtype, numel=logits.numel())
    _check("softmax_forward", lib.softmax_forward(_dev(probs, "probs"), _dev(logits, "logits"), N,
                                                  V, Vp, dt, _stream(stream)))
    return probs


STAT_COLS = 128  # columns per row-statistics group


def stat_groups(Vp: int) -> int:
    return (Vp + STAT_COLS - 1) // STAT_COLS


def matmul_logits_stats_forward(logits, stats, inp, wte, V, stream=None):
    """logits [N,Vp] = inp [N,C] @ wte[Vp,C]^T and stats fp32 [N, groups, 2]: per row and
    128-column group, the max and the sum of exp(l - max) over the columns < V."""
    lib = load_library()
    dt = _dtype_code(inp)
    N, C, Vp = _linear_args(inp, wte, None)
    if not 0 < V <= Vp:
        raise ValueError("V must lie in [1, %d], got %d" % (Vp, V))
    _chk(logits, "logits", dtype=inp.dtype, numel=N * Vp)
    _f32t(stats, "stats", numel=N * stat_groups(Vp) * 2)
    _check("matmul_logits_stats_forward", lib.matmul_logits_stats_forward(
        _dev(logits, "logits"), _dev(stats, "stats"), _dev(inp, "inp"), _dev(wte, "wte"), N, C, V, Vp, dt,
        _stream(stream)))
    return logits


def softmax_stats_forward(probs, logits, stats, V, stream=None):
    """probs [N,Vp] from logits [N,Vp] and the row statistics of matmul_logits_stats_forward."""
    lib = load_library()
    dt = _dtype_code(logits)
    N, Vp = _vocab_dims(logits, V)
    _chk(probs, "probs", dtype=logits.dtype, numel=N * Vp)
    _f32t(stats, "stats", numel=N * stat_groups(Vp) * 2)
    _check("softmax_stats_forward", lib.softmax_stats_forward(
        _dev(probs, "probs"), _dev(logits, "logits"), _dev(stats, "stats"), N, V, Vp, dt, _stream(stream)))
    return probs


# ------------------------------------------------------------------ model entries
def param_count(cfg: Config) -> int:
    return int(load_library().gpt2_param_count(ctypes.byref(cfg)))


def workspace_bytes(cfg: Config, B: int, T: int) -> int:
    return int(load_library().gpt2_workspace_bytes(ctypes.byref(cfg), B, T))


def _model_args(cfg: Config, params, workspace, ws_bytes):
    """params in the config's dtype holding at least the flat parameter count;
    workspace a byte buffer of at least ws_bytes."""
    n = param_count(cfg)
    if n < 0:
        raise ValueError("invalid model config")
    _chk(params, "params", dtype=_tdt(cfg.dtype), min_numel=n)
    if workspace is not None and _nbytes(workspace) < ws_bytes:
        raise ValueError("workspace must hold at least %d bytes, got %d" % (ws_bytes, _nbytes(workspace)))


def _cache_args(cfg: Config, kcache, vcache, B):
    """kcache, vcache [L,B,NH,maxT,hs] in the config's dtype."""
    hs = cfg.C // cfg.NH
    shape = (cfg.L, B, cfg.NH, cfg.maxT, hs)
    for t, nm in ((kcache, "kcache"), (vcache, "vcache")):
        _chk(t, nm, dtype=_tdt(cfg.dtype))
        if tuple(t.shape) != shape:
            raise ValueError("%s must be %s, got %s" % (nm, shape, tuple(t.shape)))


def gpt2_forward(logits, probs, tokens, params, cfg: Config, workspace, stream=None):
    """logits/probs [B,T,Vp] (probs may be None); tokens int32 [B,T]; params flat."""
    lib = load_library()
    _int32(tokens, "tokens", ndim=2)
    B, T = tokens.shape
    _model_args(cfg, params, workspace, workspace_bytes(cfg, B, T))
    _chk(logits, "logits", dtype=_tdt(cfg.dtype), numel=B * T * cfg.Vp)
    _chk(probs, "probs", dtype=_tdt(cfg.dtype), numel=B * T * cfg.Vp, optional=True)
    _check("gpt2_forward", lib.gpt2_forward(
        _dev(logits, "logits"), _dev(probs, "probs"), _dev(tokens, "tokens"), _dev(params, "params"),
        ctypes.byref(cfg), B, T, _dev(workspace, "workspace"), _nbytes(workspace), _stream(stream)))
    return logits


def attention_decode_workspace_bytes(B, C, NH, maxT) -> int:
    return int(load_library().attention_decode_workspace_bytes(B, C, NH, maxT))


def attention_decode_forward(out, qkv_new, kcache, vcache, pos, NH, workspace, stream=None):
    """out [B,C]; qkv_new [B,3C]; kcache/vcache [B,NH,maxT,hs] for one layer."""
    lib = load_library()
    dt = _dtype_code(qkv_new)
    _chk(qkv_new, "qkv_new", ndim=2)
    B, C3 = qkv_new.shape
    if C3 % 3 or NH <= 0 or (C3 // 3) % NH:
        raise ValueError("qkv_new must be [B, 3C] with C divisible by NH")
    C = C3 // 3
    _chk(kcache, "kcache", dtype=qkv_new.dtype, ndim=4)
    maxT = kcache.shape[2]
    for t, nm in ((kcache, "kcache"), (vcache, "vcache")):
        _chk(t, nm, dtype=qkv_new.dtype)
        if tuple(t.shape) != (B, NH, maxT, C // NH):
            raise ValueError("%s must be %s, got %s" % (nm, (B, NH, maxT, C // NH), tuple(t.shape)))
    _chk(out, "out", dtype=qkv_new.dtype, numel=B * C)
    _check("attention_decode_forward", lib.attention_decode_forward(
        _dev(out, "out"), _dev(qkv_new, "qkv_new"), _dev(kcache, "kcache"), _dev(vcache, "vcache"),
        B, int(pos), maxT, C, NH, dt, _dev(workspace, "workspace"), _nbytes(workspace), _stream(stream)))
    return out


def decode_workspace_bytes(cfg: Config, B: int) -> int:
    return int(load_library().gpt2_decode_workspace_bytes(ctypes.byref(cfg), B))


def gpt2_decode_step(logits, probs, tokens, pos, kcache, vcache, params, cfg: Config, workspace,
                     stream=None):
    """One decode step: tokens int32 [B] at position pos; caches [L,B,NH,maxT,hs]."""
    lib = load_library()
    _int32(tokens, "tokens", ndim=1)
    B = tokens.shape[0]
    _model_args(cfg, params, workspace, decode_workspace_bytes(cfg, B))
    _cache_args(cfg, kcache, vcache, B)
    _chk(logits, "logits", dtype=_tdt(cfg.dtype), numel=B * cfg.Vp)
    _chk(probs, "probs", dtype=_tdt(cfg.dtype), numel=B * cfg.Vp, optional=True)
    _check("gpt2_decode_step", lib.gpt2_decode_step(
        _dev(logits, "logits"), _dev(probs, "probs"), _dev(tokens, "tokens"), int(pos),
        _dev(kcache, "kcache"), _dev(vcache, "vcache"), _dev(params, "params"), ctypes.byref(cfg), B,
        _dev(workspace, "workspace"), _nbytes(workspace), _stream(stream)))
    return logits


def gpt2_decode_step_noalloc(logits, probs, tokens, pos, kcache, vcache, params, cfg: Config, stream=None):
    """gpt2_decode_step with the library's own device scratch instead of a
    workspace (for callers that cannot allocate); calls that overlap on one
    GPU race."""
    lib = load_library()
    _int32(tokens, "tokens", ndim=1)
    B = tokens.shape[0]
    _model_args(cfg, params, None, 0)
    _cache_args(cfg, kcache, vcache, B)
    _chk(logits, "logits", dtype=_tdt(cfg.dtype), numel=B * cfg.Vp)
    _chk(probs, "probs", dtype=_tdt(cfg.dtype), numel=B * cfg.Vp, optional=True)
    _check("gpt2_decode_step_noalloc", lib.gpt2_decode_step_noalloc(
        _dev(logits, "logits"), _dev(probs, "probs"), _dev(tokens, "tokens"), int(pos),
        _dev(kcache, "kcache"), _dev(vcache, "vcache"), _dev(params, "params"), ctypes.byref(cfg), B,
        _stream(stream)))
    return logits


# ------------------------------------------------------------------ generation
def argmax_forward(tokens, logits, V, stream=None):
    """tokens int32 [N] = argmax over v < V of logits [N,Vp] (lowest index on ties)."""
    lib = load_library()
    dt = _dtype_code(logits)
    N, Vp = _vocab_dims(logits, V)
    _int32(tokens, "tokens", numel=N)
    _check("argmax_forward", lib.argmax_forward(_dev(tokens, "tokens"), _dev(logits, "logits"), N, V, Vp,
                                                dt, _stream(stream)))
    return tokens


def gpt2_prefill(logits, probs, tokens, kcache, vcache, params, cfg: Config, workspace, stream=None):
    """Blocks over tokens int32 [B,T], caches [L,B,NH,maxT,hs] filled at 0..T-1; logits/probs [B,Vp]
    of the last position."""
    lib = load_library()
    _int32(tokens, "tokens", ndim=2)
    B, T = tokens.shape
    _model_args(cfg, params, workspace, workspace_bytes(cfg, B, T))
    _cache_args(cfg, kcache, vcache, B)
    _chk(logits, "logits", dtype=_tdt(cfg.dtype), numel=B * cfg.Vp)
    _chk(probs, "probs", dtype=_tdt(cfg.dtype), numel=B * cfg.Vp, optional=True)
    _check("gpt2_prefill", lib.gpt2_prefill(
        _dev(logits, "logits"), _dev(probs, "probs"), _dev(tokens, "tokens"), _dev(kcache, "kcache"),
        _dev(vcache, "vcache"), _dev(params, "params"), ctypes.byref(cfg), B, T, _dev(workspace, "workspace"),
        _nbytes(workspace), _stream(stream)))
    return logits


def generate_workspace_bytes(cfg: Config, B: int, T: int) -> int:
    return int(load_library().gpt2_generate_workspace_bytes(ctypes.byref(cfg), B, T))


def gpt2_generate(out_tokens, prompt, kcache, vcache, params, cfg: Config, workspace, stream=None):
    """Greedy generation: out_tokens int32 [B,n_new] after prompt int32 [B,T]."""
    lib = load_library()
    _int32(prompt, "prompt", ndim=2)
    B, T = prompt.shape
    _int32(out_tokens, "out_tokens", ndim=2)
    if out_tokens.shape[0] != B:
        raise ValueError("out_tokens must be [%d, n_new], got %s" % (B, tuple(out_tokens.shape)))
    n_new = out_tokens.shape[1]
    _model_args(cfg, params, workspace, generate_workspace_bytes(cfg, B, T))
    _cache_args(cfg, kcache, vcache, B)
    _check("gpt2_generate", lib.gpt2_generate(
        _dev(out_tokens, "out_tokens"), _dev(prompt, "prompt"), n_new, _dev(kcache, "kcache"),
        _dev(vcache, "vcache"), _dev(params, "params"), ctypes.byref(cfg), B, T, _dev(workspace, "workspace"),
        _nbytes(workspace), _stream(stream)))
    return out_tokens


# ------------------------------------------------------------------ backward
def _nbytes(t):
    return t.numel() * t.element_size()


def crossentropy_backward(dlogits, logits, targets, V, dloss, losses=None, mean_loss=None, stream=None):
    """dlogits [N,Vp] = dloss * (softmax(logits) - onehot(targets)) on v < V, 0 in the padding
    (dlogits may be logits); optional fp32 losses [N] and their mean [1]."""
    lib = load_library()
    dt = _dtype_code(logits)
    N, Vp = _vocab_dims(logits, V)
    _chk(dlogits, "dlogits", dtype=logits.dtype, numel=N * Vp)
    _int32(targets, "targets", numel=N)
    _f32t(losses, "losses", numel=N, optional=True)
    _f32t(mean_loss, "mean_loss", numel=1, optional=True)
    _check("crossentropy_backward", lib.crossentropy_backward(
        _dev(dlogits, "dlogits"), _dev(losses, "losses"), _dev(mean_loss, "mean_loss"), _dev(logits, "logits"),
        _dev(targets, "targets"), float(dloss), N, V, Vp, dt, _stream(stream)))
    return dlogits


def gelu_backward(dinp, inp, dout, stream=None):
    """dinp = dout * gelu'(inp) (dinp may be dout)."""
    lib = load_library()
    dt = _dtype_code(inp)
    _chk(dout, "dout", dtype=inp.dtype, numel=inp.numel())
    _chk(dinp, "dinp", dtype=inp.dtype, numel=inp.numel())
    _check("gelu_backward", lib.gelu_backward(_dev(dinp, "dinp"), _dev(inp, "inp"), _dev(dout, "dout"),
                                              inp.numel(), dt, _stream(stream)))
    return dinp


def layernorm_backward_workspace_size(N, C) -> int:
    return int(load_library().layernorm_backward_workspace_size(N, C))


def layernorm_backward(dinp, dgamma, dbeta, dout, inp, gamma, mean, rstd, workspace, dres=None, stream=None):
    """dinp = [dres +] LayerNorm backward; dgamma, dbeta (nullable) overwritten; dres may be dinp."""
    lib = load_library()
    dt = _dtype_code(inp)
    C = _last(inp, "inp")
    N = inp.numel() // C if C else 0
    for t, nm in ((dinp, "dinp"), (dout, "dout")):
        _chk(t, nm, dtype=inp.dtype, numel=inp.numel())
    _chk(dres, "dres", dtype=inp.dtype, numel=inp.numel(), optional=True)
    _chk(gamma, "gamma", dtype=inp.dtype, numel=C)
    _chk(dgamma, "dgamma", dtype=inp.dtype, numel=C, optional=True)
    _chk(dbeta, "dbeta", dtype=inp.dtype, numel=C, optional=True)
    _f32t(mean, "mean", numel=N)
    _f32t(rstd, "rstd", numel=N)
    _check("layernorm_backward", lib.layernorm_backward(
        _dev(dinp, "dinp"), _dev(dgamma, "dgamma"), _dev(dbeta, "dbeta"), _dev(dres, "dres"), _dev(dout, "dout"),
        _dev(inp, "inp"), _dev(gamma, "gamma"), _dev(mean, "mean"), _dev(rstd, "rstd"), N, C, dt,
        _dev(workspace, "workspace"), _nbytes(workspace), _stream(stream)))
    return dinp


def matmul_backward_workspace_size(N, C, OC, dtype) -> int:
    return int(load_library().matmul_backward_workspace_size(N, C, OC, dtype))


def matmul_backward(dinp, dweight, dbias, dout, inp, weight, workspace, stream=None):
    """For out = inp [N,C] @ weight[OC,C]^T + b: dinp [N,C], dweight [OC,C], dbias [OC] (each nullable)."""
    lib = load_library()
    dt = _dtype_code(dout)
    _chk(weight, "weight", dtype=dout.dtype, ndim=2)
    OC, C = weight.shape
    if OC == 0 or dout.numel() % OC:
        raise ValueError("dout must be [N, %d], got %s" % (OC, tuple(dout.shape)))
    N = dout.numel() // OC
    _chk(inp, "inp", dtype=dout.dtype, numel=N * C)
    _chk(dinp, "dinp", dtype=dout.dtype, numel=N * C, optional=True)
    _chk(dweight, "dweight", dtype=dout.dtype, numel=OC * C, optional=True)
    _chk(dbias, "dbias", dtype=dout.dtype, numel=OC, optional=True)
    _check("matmul_backward", lib.matmul_backward(
        _dev(dinp, "dinp"), _dev(dweight, "dweight"), _dev(dbias, "dbias"), _dev(dout, "dout"), _dev(inp, "inp"),
        _dev(weight, "weight"), N, C, OC, dt, _dev(workspace, "workspace"), _nbytes(workspace),
        _stream(stream)))
    return dinp


def attention_forward_lse(out, lse, qkv, NH, stream=None):
    """out [B,T,C] and lse fp32 [B,NH,T] (log-sum-exp of each causal score row) from qkv [B,T,3C]."""
    lib = load_library()
    dt = _dtype_code(qkv)
    B, T, C = _qkv_dims(qkv)
    _chk(out, "out", dtype=qkv.dtype, numel=B * T * C)
    _f32t(lse, "lse", numel=B * NH * T)
    _check("attention_forward_lse", lib.attention_forward_lse(
        _dev(out, "out"), _dev(lse, "lse"), _dev(qkv, "qkv"), B, T, C, NH, dt, _stream(stream)))
    return out


def attention_backward_workspace_size(B, T, C, NH) -> int:
    return int(load_library().attention_backward_workspace_size(B, T, C, NH))


def attention_backward(dqkv, dout, qkv, out, lse, NH, workspace, stream=None):
    """dqkv [B,T,3C] from dout [B,T,C] and the forward's qkv, out and lse."""
    lib = load_library()
    dt = _dtype_code(qkv)
    B, T, C = _qkv_dims(qkv)
    _chk(dqkv, "dqkv", dtype=qkv.dtype, numel=B * T * 3 * C)
    _chk(dout, "dout", dtype=qkv.dtype, numel=B * T * C)
    _chk(out, "out", dtype=qkv.dtype, numel=B * T * C)
    _f32t(lse, "lse", numel=B * NH * T)
    _check("attention_backward", lib.attention_backward(
        _dev(dqkv, "dqkv"), _dev(dout, "dout"), _dev(qkv, "qkv"), _dev(out, "out"), _dev(lse, "lse"), B, T, C,
        NH, dt, _dev(workspace, "workspace"), _nbytes(workspace), _stream(stream)))
    return dqkv


def encoder_backward(dwte, dwpe, dout, tokens, stream=None):
    """dwte[tokens[b,t]] += dout[b,t]; dwpe[t] += sum_b dout[b,t] (either may be None)."""
    lib = load_library()
    dt = _dtype_code(dout)
    _int32(tokens, "tokens", ndim=2)
    B, T = tokens.shape
    C = _last(dout, "dout")
    _chk(dout, "dout", numel=B * T * C)
    for t, nm, rows in ((dwte, "dwte", 1), (dwpe, "dwpe", T)):
        _chk(t, nm, dtype=dout.dtype, ndim=2, optional=True)
        if t is not None and (t.shape[1] != C or t.shape[0] < rows):
            raise ValueError("%s must be [>=%d, %d], got %s" % (nm, rows, C, tuple(t.shape)))
    _check("encoder_backward", lib.encoder_backward(
        _dev(dwte, "dwte"), _dev(dwpe, "dwpe"), _dev(dout, "dout"), _dev(tokens, "tokens"), B, T, C,
        dt, _stream(stream)))


def train_acts_bytes(cfg: Config, B: int, T: int) -> int:
    return int(load_library().gpt2_train_acts_bytes(ctypes.byref(cfg), B, T))


def train_workspace_bytes(cfg: Config, B: int, T: int) -> int:
    return int(load_library().gpt2_train_workspace_bytes(ctypes.byref(cfg), B, T))


def gpt2_train_forward(tokens, targets, params, cfg: Config, acts, losses=None, mean_loss=None, stream=None):
    """Forward keeping its activations in acts, then the losses (fp32 [B*T], optional), their mean
    (fp32 [1], optional) and the gradient of the mean loss w.r.t. the logits (kept in acts)."""
    lib = load_library()
    _int32(tokens, "tokens", ndim=2)
    B, T = tokens.shape
    _int32(targets, "targets", numel=B * T)
    _model_args(cfg, params, acts, train_acts_bytes(cfg, B, T))
    _f32t(losses, "losses", numel=B * T, optional=True)
    _f32t(mean_loss, "mean_loss", numel=1, optional=True)
    _check("gpt2_train_forward", lib.gpt2_train_forward(
        _dev(losses, "losses"), _dev(mean_loss, "mean_loss"), _dev(tokens, "tokens"), _dev(targets, "targets"),
        _dev(params, "params"), ctypes.byref(cfg), B, T, _dev(acts, "acts"), _nbytes(acts), _stream(stream)))


def gpt2_backward(grads, tokens, params, cfg: Config, acts, workspace, stream=None):
    """grads (flat, parameter layout) of the mean loss of the preceding gpt2_train_forward."""
    lib = load_library()
    _int32(tokens, "tokens", ndim=2)
    B, T = tokens.shape
    _model_args(cfg, params, workspace, train_workspace_bytes(cfg, B, T))
    _chk(grads, "grads", dtype=_tdt(cfg.dtype), min_numel=param_count(cfg))
    if acts is not None and _nbytes(acts) < train_acts_bytes(cfg, B, T):
        raise ValueError("acts must hold at least %d bytes" % train_acts_bytes(cfg, B, T))
    _check("gpt2_backward", lib.gpt2_backward(
        _dev(grads, "grads"), _dev(tokens, "tokens"), _dev(params, "params"), ctypes.byref(cfg), B, T,
        _dev(acts, "acts"), _nbytes(acts), _dev(workspace, "workspace"), _nbytes(workspace), _stream(stream)))
    return grads
