"""Seeded synthetic workloads for the GPT-2 forward pass.

This module only draws numbers and lays them out. It holds none of the
forward pass's arithmetic, so both the CPU oracle and the GPU library can be
fed from it without sharing any of the method between them.

Workloads (the shapes and inits of the GPT-2 configurations named for this
path; the pages profile GPT-2 small at sequence length 1024 in the llm.c
discussion "State of the Union [April 22, 2024]", kernel summary table):

  tiny      fp32, L=2  C=64   NH=4  V=256   maxT=32,   B=2 T=32
  small     fp32, L=12 C=768  NH=12 V=50257 (Vp 50304), B=4 T=1024
  small_bf16_b8  bf16, same weights as ``small``,   B=8 T=1024
  small_bf16_b4  bf16, same weights as ``small``,   B=4 T=1024
  medium    bf16, L=24 C=1024 NH=16 V=50257 (Vp 50304), B=4 T=1024
  decode    bf16, ``small`` weights, 32 sequences, one new token at
            position 1023 over a prefilled N(0,1) K/V cache

Parameter buffer (one flat tensor, in this order):
  wte [Vp,C], wpe [maxT,C],
  ln1_g [L,C], ln1_b [L,C], qkv_w [L,3C,C], qkv_b [L,3C],
  attproj_w [L,C,C], attproj_b [L,C], ln2_g [L,C], ln2_b [L,C],
  fc_w [L,4C,C], fc_b [L,4C], fcproj_w [L,C,4C], fcproj_b [L,C],
  lnf_g [C], lnf_b [C].
Linear weights are [out_features, in_features] row-major.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Tuple

import numpy as np

F32 = 0
BF16 = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    L: int
    C: int
    NH: int
    V: int
    Vp: int
    maxT: int
    B: int
    T: int
    dtype: int  # F32 or BF16
    token_seed: int
    weight_seed: int
    scale_residual_proj: bool  # attproj/fcproj std 0.02/sqrt(2L)
    random_affine: bool = False  # gamma ~ 1+N(0,0.1), beta ~ N(0,0.1), biases ~ N(0,0.02)
    decode_pos: int = -1  # >= 0: one new token per sequence at this position
    cache_seed: int = 0
    ln_eps: float = 1e-5

    @property
    def hs(self) -> int:
        return self.C // self.NH

    @property
    def N(self) -> int:
        return self.B * (1 if self.decode_pos >= 0 else self.T)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny", 2, 64, 4, 256, 256, 32, 2, 32, F32, 100, 200, False),
        Workload("tiny_affine", 2, 64, 4, 256, 256, 32, 2, 32, F32, 100, 200, False, random_affine=True),
        Workload("tiny_bf16", 2, 64, 4, 256, 256, 32, 2, 32, BF16, 100, 200, False),
        Workload("small", 12, 768, 12, 50257, 50304, 1024, 4, 1024, F32, 101, 201, True),
        Workload("small_bf16_b8", 12, 768, 12, 50257, 50304, 1024, 8, 1024, BF16, 102, 201, True),
        Workload("small_bf16_b4", 12, 768, 12, 50257, 50304, 1024, 4, 1024, BF16, 101, 201, True),
        Workload("medium", 24, 1024, 16, 50257, 50304, 1024, 4, 1024, BF16, 103, 203, True),
        Workload("decode", 12, 768, 12, 50257, 50304, 1024, 32, 1, BF16, 104, 201, True,
                 decode_pos=1023, cache_seed=304),
        # GPT-2 small's width, head size and vocabulary with 2 layers and 64
        # tokens: small enough for the oracle's whole training step
        Workload("small_2l", 2, 768, 12, 50257, 50304, 1024, 1, 64, F32, 105, 205, True),
        Workload("small_2l_bf16", 2, 768, 12, 50257, 50304, 1024, 1, 64, BF16, 105, 205, True),
    ]
}


def param_layout(L: int, C: int, maxT: int, Vp: int) -> List[Tuple[str, Tuple[int, ...]]]:
    """Names and shapes of the flat parameter buffer, in storage order."""
    return [
        ("wte", (Vp, C)), ("wpe", (maxT, C)),
        ("ln1_g", (L, C)), ("ln1_b", (L, C)),
        ("qkv_w", (L, 3 * C, C)), ("qkv_b", (L, 3 * C)),
        ("attproj_w", (L, C, C)), ("attproj_b", (L, C)),
        ("ln2_g", (L, C)), ("ln2_b", (L, C)),
        ("fc_w", (L, 4 * C, C)), ("fc_b", (L, 4 * C)),
        ("fcproj_w", (L, C, 4 * C)), ("fcproj_b", (L, C)),
        ("lnf_g", (C,)), ("lnf_b", (C,)),
    ]


def param_offsets(L: int, C: int, maxT: int, Vp: int) -> Dict[str, Tuple[int, Tuple[int, ...]]]:
    off = 0
    out = {}
    for name, shape in param_layout(L, C, maxT, Vp):
        out[name] = (off, shape)
        off += int(np.prod(shape))
    out["_total"] = (off, ())
    return out


def views(flat: np.ndarray, w: Workload) -> Dict[str, np.ndarray]:
    """Named views into a flat parameter array."""
    offs = param_offsets(w.L, w.C, w.maxT, w.Vp)
    return {k: flat[o:o + int(np.prod(s))].reshape(s) for k, (o, s) in offs.items() if k != "_total"}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs here are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 values of the bf16 numbers nearest to x."""
    return bf16_bits_to_f32(to_bf16_bits(x))


def make_tokens(w: Workload) -> np.ndarray:
    rng = np.random.default_rng(w.token_seed)
    shape = (w.B,) if w.decode_pos >= 0 else (w.B, w.T)
    return rng.integers(0, w.V, size=shape, dtype=np.int64).astype(np.int32)


def make_targets(w: Workload) -> np.ndarray:
    """Next-token targets int32 [B,T]: position t's target is token t+1 of the
    same sequence; the last position's is a seeded uniform draw."""
    tok = make_tokens(w)
    rng = np.random.default_rng(w.token_seed + 7)
    tg = np.empty_like(tok)
    tg[:, :-1] = tok[:, 1:]
    tg[:, -1] = rng.integers(0, w.V, size=tok.shape[0], dtype=np.int64).astype(np.int32)
    return tg


def make_params(w: Workload) -> np.ndarray:
    """fp32 flat parameters. For bf16 workloads the values are already rounded
    to bf16, so the fp32 array holds exactly what the bf16 buffer holds."""
    offs = param_offsets(w.L, w.C, w.maxT, w.Vp)
    total = offs["_total"][0]
    rng = np.random.default_rng(w.weight_seed)
    flat = rng.standard_normal(total, dtype=np.float32)
    flat *= np.float32(0.02)
    p = views(flat, w)
    if w.scale_residual_proj:
        s = np.float32(1.0 / math.sqrt(2 * w.L))
        p["attproj_w"][...] *= s
        p["fcproj_w"][...] *= s
    p["wte"][w.V:, :] = 0.0
    if w.random_affine:
        arng = np.random.default_rng(w.weight_seed + 50)
        for g in ("ln1_g", "ln2_g", "lnf_g"):
            p[g][...] = 1.0 + 0.1 * arng.standard_normal(p[g].shape, dtype=np.float32)
        for b in ("ln1_b", "ln2_b", "lnf_b"):
            p[b][...] = 0.1 * arng.standard_normal(p[b].shape, dtype=np.float32)
        for b in ("qkv_b", "attproj_b", "fc_b", "fcproj_b"):
            p[b][...] = 0.02 * arng.standard_normal(p[b].shape, dtype=np.float32)
    else:
        for g in ("ln1_g", "ln2_g", "lnf_g"):
            p[g][...] = 1.0
        for b in ("ln1_b", "ln2_b", "lnf_b", "qkv_b", "attproj_b", "fc_b", "fcproj_b"):
            p[b][...] = 0.0
    if w.dtype == BF16:
        flat = round_to_bf16(flat)
    return flat


def make_kv_cache(w: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """Prefilled decode cache [L,B,NH,maxT,hs]: positions < decode_pos ~ N(0,1)
    (bf16-rounded for bf16 workloads), positions >= decode_pos are zero."""
    assert w.decode_pos >= 0
    rng = np.random.default_rng(w.cache_seed)
    shape = (w.L, w.B, w.NH, w.maxT, w.hs)
    caches = []
    for _ in range(2):
        c = rng.standard_normal(shape, dtype=np.float32)
        c[:, :, :, w.decode_pos:, :] = 0.0
        if w.dtype == BF16:
            c = round_to_bf16(c)
        caches.append(c)
    return caches[0], caches[1]


def random_tensor(seed: int, shape, std: float = 1.0, dtype: int = F32) -> np.ndarray:
    """Generic seeded N(0, std^2) tensor for per-kernel tests."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)
    return round_to_bf16(x) if dtype == BF16 else x


def random_int_tensor(seed: int, shape, lo: int, hi: int, dtype: int = F32) -> np.ndarray:
    """Small-integer-valued float tensor (exact in fp32 and bf16 for |x| <= 256)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)
