"""Helpers for the GPU parity tests: host<->device transfer with bf16 bit
patterns, and the error measures the tolerances are stated in."""
import numpy as np

from transformer_forward_pass_gpt_amd import inputs as I


def torch_mod():
    import torch
    return torch


def dev(x, dtype):
    """numpy float32 (already bf16-representable for BF16) -> GPU tensor."""
    torch = torch_mod()
    x = np.ascontiguousarray(x)
    if dtype == I.BF16:
        bits = I.to_bf16_bits(x.astype(np.float32)).view(np.int16)
        return torch.from_numpy(bits).cuda().view(torch.bfloat16)
    return torch.from_numpy(x.astype(np.float32)).cuda()


def dev_int(x):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def empty(shape, dtype, fill=None):
    torch = torch_mod()
    t = torch.empty(shape, dtype=torch.bfloat16 if dtype == I.BF16 else torch.float32, device="cuda")
    if fill is not None:
        t.fill_(fill)
    return t


def host(t):
    """GPU tensor -> numpy float32 (bf16 widened exactly)."""
    torch = torch_mod()
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return I.bf16_bits_to_f32(bits)
    return t.cpu().numpy()


def host_bits(t):
    torch = torch_mod()
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy().view(np.uint32)


def rel_err(x, ref):
    """Norm-relative error ||x - ref|| / ||ref|| in double."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300))


def max_abs(x, ref):
    return float(np.max(np.abs(np.asarray(x, np.float64) - np.asarray(ref, np.float64))))


def bf16_round(x):
    return I.round_to_bf16(np.asarray(x, np.float32))


def tile_rel_max(got, ref, rows=128, cols=128):
    """Largest norm-relative error over rows x cols tiles of a 2-D array, each
    tile's norm floored at a tenth of the whole array's rms times the tile's
    size (so near-zero tiles do not dominate): a tile the GEMMs got wrong
    shows up here even when the whole-array norm hardly moves."""
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(r * r))
    worst = 0.0
    for i in range(0, r.shape[0], rows):
        for j in range(0, r.shape[1], cols):
            rt = r[i:i + rows, j:j + cols]
            dt = g[i:i + rows, j:j + cols] - rt
            den = max(np.linalg.norm(rt), 0.1 * rms * np.sqrt(rt.size), 1e-300)
            worst = max(worst, float(np.linalg.norm(dt) / den))
    return worst
