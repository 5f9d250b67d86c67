"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws numbers; it holds none of the attention method's
arithmetic (no pooling, normalisation, rotation, quantisation or scoring).
Values that must live on a number format's grid are drawn on that grid
directly:
  - bf16 inputs: a normal float32 draw whose low 16 mantissa bits are dropped
    (truncation, so the value is exactly a bf16 number);
  - FP4 inputs: uniform E2M1 codes and E8M0 exponents drawn from a range;
  - "grid" inputs: a normal draw clipped to [lo, hi] and snapped to a step.
Seeds: numpy PCG64, 1000 + n for weights and 2000 + n for activations of the
n-th workload, unless a test picks its own.
"""
import numpy as np


def rng(seed):
    return np.random.default_rng(seed)


def normal(g, shape, std=1.0):
    return (g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def bf16_bits(g, shape, std=1.0):
    """Normal draw as bf16 bit patterns (uint16), by truncating float32."""
    x = normal(g, shape, std)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b):
    """Exact widening of bf16 bit patterns to float32 (a format view)."""
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def grid(g, shape, step=0.125, lo=-2.0, hi=2.0):
    """N(0,1) clipped to [lo, hi] and snapped to multiples of step."""
    x = np.clip(g.standard_normal(size=shape), lo, hi)
    return (np.round(x / step) * step).astype(np.float32)


def fp4_rows(g, rows, di, exp_lo=-3, exp_hi=0):
    """Random FP4 rows: codes [rows..., di/2] (two E2M1 codes per byte, even
    element in the low nibble) and E8M0 scales [rows..., di/32] with exponents
    uniform in [exp_lo, exp_hi]."""
    rows = tuple(np.atleast_1d(rows))
    lo = g.integers(0, 16, size=rows + (di // 2,), dtype=np.uint8)
    hi = g.integers(0, 16, size=rows + (di // 2,), dtype=np.uint8)
    codes = (lo | (hi << 4)).astype(np.uint8)
    scales = (g.integers(exp_lo, exp_hi + 1, size=rows + (di // 32,)) + 127).astype(np.uint8)
    return codes, scales


def topk_lists(g, n_visible, k, rows):
    """rows x k block indices: distinct, ascending, drawn from [0, n_visible),
    padded with -1 when n_visible < k."""
    out = np.full((rows, k), -1, np.int32)
    for r in range(rows):
        n = int(n_visible[r]) if np.ndim(n_visible) else int(n_visible)
        take = min(n, k)
        if take > 0:
            out[r, :take] = np.sort(g.choice(n, size=take, replace=False)).astype(np.int32)
    return out


def fp8_records(g, prefix, d, dr, rec_bytes):
    """Random FP8 KV records [prefix..., rec_bytes]: E4M3 codes drawn uniformly
    over the finite codes, bf16 RoPE dims from a normal draw, a positive fp32
    row scale, zero padding (layout of include/csa_attn.h)."""
    prefix = tuple(np.atleast_1d(prefix))
    dn = d - dr
    out = np.zeros(prefix + (rec_bytes,), np.uint8)
    codes = g.integers(0, 254, size=prefix + (dn,), dtype=np.uint8)
    codes = np.where(codes >= 0x7F, codes + 1, codes).astype(np.uint8)      # skip 0x7F (NaN); 0xFF unreachable
    out[..., :dn] = codes
    out[..., dn:dn + 2 * dr] = bf16_bits(g, prefix + (dr,)).view(np.uint8).reshape(prefix + (2 * dr,))
    scale = (np.abs(normal(g, prefix)) * np.float32(0.01) + np.float32(1e-3)).astype(np.float32)
    out[..., dn + 2 * dr:dn + 2 * dr + 4] = scale.view(np.uint8).reshape(prefix + (4,))
    return out


def e4m3_codes(g, shape, std=64.0):
    """FP8 weight codes: a normal draw times std, clipped to +-448 and cast to
    E4M3 by torch's float8_e4m3fn conversion (a format cast), as uint8."""
    import torch
    x = np.clip(normal(g, shape, std), -448.0, 448.0).astype(np.float32)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# E4M3 codes of 0, 0.25, 0.5 and 1 (exponent field 5, 6, 7; mantissa 0)
E4M3_POW2 = np.array([0x00, 0x28, 0x30, 0x38], np.uint8)


def e4m3_pow2_codes(g, shape, p_zero=0.5):
    """FP8 weight codes drawn from {0, +-0.25, +-0.5, +-1}: products with grid
    activations and their fp32 sums stay exact (zero with probability p_zero)."""
    mag = g.integers(1, 4, size=shape)
    mag = np.where(g.random(size=shape) < p_zero, 0, mag)
    sign = (g.integers(0, 2, size=shape) * 0x80).astype(np.uint8)
    return (E4M3_POW2[mag] | np.where(mag > 0, sign, 0)).astype(np.uint8)
