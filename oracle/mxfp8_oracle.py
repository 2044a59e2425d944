"""Plain CPU oracle of the MXFP8 variant of the grouped expert FFN.

TEST INFRASTRUCTURE ONLY. Only the tests and the benchmark's CPU-baseline leg
may import this module. It shares no code with the HIP path.

The pages name an MXFP8 transform of the distributed MoE layer (torchtitan
issue 5554: the shared-expert overlap applies to the layer's BF16 and MXFP8
transforms) without defining the format. The definitions below are the
published OCP Microscaling (MX) format, version 1.0, MXFP8 with E4M3
elements:

  * element E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; no
    infinities; S.1111.111 is NaN; largest magnitude 448 = 1.75 * 2^8;
    smallest normal 2^-6; subnormals m * 2^-9 (m = 1..7);
  * block: 32 consecutive elements along the contraction dimension share one
    scale X = 2^s, stored as an E8M0 byte s + 127;
  * s = floor(log2(max |v|)) - 8 over the block (8 = the exponent of E4M3's
    largest normal), clamped to [-127, 127]; an all-zero block gets s = -127
    (scale byte 0);
  * element code = the E4M3 value nearest v / X, ties to the even mantissa,
    magnitudes beyond 448 saturate to 448.

Readings taken where neither the pages nor the format fix the step (each also
listed in the design notes):
  * saturation (not NaN) on overflow, the usual choice for E4M3 conversions;
  * both GEMM operands are quantized along K (the hidden size D for GEMM 1,
    the intermediate size I for GEMM 2); weights are quantized once, per
    output column, and stored as [N][K] (K contiguous) with scales [N][K/32];
  * the activations entering GEMM 1 are the bf16 rows of x_perm; H is formed
    in fp32 (SiLU(g) * u, gate = the first I columns of gate_up_proj as in
    the bf16 layer), stored as bf16 (round to nearest even), and that bf16 H
    is what GEMM 2 quantizes; Y stays in higher precision (fp32 in the
    kernel, float64 here) as in the bf16 layer.

Arithmetic is float64 (every product and sum of dequantized values is exact
or float64-rounded); rounding points are only the ones listed above.
Pins: the CPU tests pin the E4M3 code table, round-to-nearest-even at every
midpoint, saturation, the block scale rule, the error bound, and the MX GEMM
against numpy's matmul on exactly representable inputs.
"""
from __future__ import annotations

from typing import Dict, Tuple

import numpy as np

__all__ = [
    "E4M3_MAX",
    "BLOCK",
    "e4m3_decode",
    "e4m3_encode",
    "mx_quantize",
    "mx_dequantize",
    "pack_weights",
    "mx_gemm",
    "round_bf16",
    "expert_ffn_mxfp8",
]

E4M3_MAX = 448.0
BLOCK = 32


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 codes (uint8) -> float64 values (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(y) -> np.ndarray:
    """Finite float64 values -> nearest E4M3 codes (ties to even), saturating."""
    y = np.asarray(y, dtype=np.float64)
    sign = np.signbit(y).astype(np.int64) << 7
    a = np.abs(y)
    out = np.zeros(a.shape, dtype=np.int64)
    # Subnormal range (below 2^-6): multiples of 2^-9; rounding up to 8 * 2^-9
    # gives code 8, the smallest normal, as it should.
    sub = a < 2.0 ** -6
    out = np.where(sub, np.rint(np.where(sub, a, 0.0) * 2.0 ** 9).astype(np.int64), out)
    # Normal range: exponent e = floor(log2 a), mantissa rounded to 3 bits.
    nz = ~sub
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.floor(np.log2(np.where(nz, a, 1.0))).astype(np.int64)
        # guard the floor against log2 rounding at exact powers of two
        e = np.where(np.exp2(e.astype(np.float64)) > a, e - 1, e)
        e = np.where(np.exp2((e + 1).astype(np.float64)) <= a, e + 1, e)
        frac = np.where(nz, a / np.exp2(e.astype(np.float64)) - 1.0, 0.0)  # exact: [0, 1)
    qm = np.rint(frac * 8.0).astype(np.int64)  # round half to even
    e = np.where(qm == 8, e + 1, e)
    qm = np.where(qm == 8, 0, qm)
    code_n = ((e + 7) << 3) | qm
    sat = (e > 8) | ((e == 8) & (qm > 6))
    code_n = np.where(sat, 0x7E, code_n)
    out = np.where(nz, code_n, out)
    return (out | sign).astype(np.uint8)


def mx_quantize(v, block: int = BLOCK) -> Tuple[np.ndarray, np.ndarray]:
    """Quantize along the last axis in blocks of 32.

    Returns (codes, scales): codes has v's shape (uint8 E4M3), scales the
    shape [..., K / 32] (uint8 E8M0, s + 127).
    """
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    assert K % block == 0, "K must be a multiple of the block size"
    vb = v.reshape(v.shape[:-1] + (K // block, block))
    amax = np.max(np.abs(vb), axis=-1)
    with np.errstate(divide="ignore"):
        s = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))), -np.inf)
    # guard floor(log2) at exact powers of two
    s = np.where(np.isfinite(s) & (np.exp2(s) > amax), s - 1, s)
    s = np.where(np.isfinite(s) & (np.exp2(s + 1) <= amax), s + 1, s)
    s = np.where(np.isfinite(s), s - 8, -127.0)
    s = np.clip(s, -127, 127).astype(np.int64)
    scaled = vb / np.exp2(s.astype(np.float64))[..., None]
    codes = e4m3_encode(scaled).reshape(v.shape)
    return codes, (s + 127).astype(np.uint8)


def mx_dequantize(codes, scales, block: int = BLOCK) -> np.ndarray:
    """Inverse of mx_quantize: element value times its block's 2^(byte - 127)."""
    vals = e4m3_decode(codes)
    K = vals.shape[-1]
    sc = np.exp2(np.asarray(scales, dtype=np.float64) - 127.0)
    return (vals.reshape(vals.shape[:-1] + (K // block, block)) * sc[..., None]).reshape(vals.shape)


def pack_weights(w) -> Tuple[np.ndarray, np.ndarray]:
    """Stacked weights [n, K, N] -> MXFP8 codes [n, N, K] and scales [n, N, K/32].

    Each output column is quantized along K (the contraction dimension).
    """
    w = np.asarray(w, dtype=np.float64)
    return mx_quantize(np.swapaxes(w, -1, -2))


def mx_gemm(a_codes, a_scales, w_codes, w_scales) -> np.ndarray:
    """Rows [M, K] (MXFP8) times packed columns [N, K] (MXFP8) -> [M, N] float64."""
    return mx_dequantize(a_codes, a_scales) @ mx_dequantize(w_codes, w_scales).T


def round_bf16(v) -> np.ndarray:
    """float64 -> fp32 (nearest even) -> bf16 (nearest even), as float64 values."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def expert_ffn_mxfp8(x_perm, offsets, w_gate_up, w_down) -> Dict[str, np.ndarray]:
    """MXFP8 grouped expert FFN over the ragged expert segments.

    x_perm [M, D] (bf16 values), offsets [n+1], w_gate_up [n, D, 2I],
    w_down [n, I, D] (bf16 values). Returns the quantized operands and Y:
      xq, xs   x_perm quantized along D
      h        bf16 H (as float64 values) [M, I]
      hq, hs   H quantized along I
      y        [M, D] float64
    """
    guq, gus = pack_weights(w_gate_up)   # [n, 2I, D]
    dq, ds = pack_weights(w_down)        # [n, D, I]
    return expert_ffn_mxfp8_packed(x_perm, offsets, guq, gus, dq, ds)


def expert_ffn_mxfp8_packed(x_perm, offsets, guq, gus, dq, ds) -> Dict[str, np.ndarray]:
    """expert_ffn_mxfp8 with the weights already quantized by pack_weights
    (gate_up_proj as guq, gus [n, 2I, D], down_proj as dq, ds [n, D, I])."""
    x = np.asarray(x_perm, dtype=np.float64)
    M, D = x.shape
    n = len(offsets) - 1
    I = guq.shape[1] // 2
    xq, xs = mx_quantize(x)
    h = np.zeros((M, I))
    for e in range(n):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi <= lo:
            continue
        gu = mx_gemm(xq[lo:hi], xs[lo:hi], guq[e], gus[e])  # [rows, 2I]
        gate, up = gu[:, :I], gu[:, I:]
        with np.errstate(over="ignore"):
            silu = gate / (1.0 + np.exp(-gate))
        h[lo:hi] = round_bf16(silu * up)
    hq, hs = mx_quantize(h)
    y = np.zeros((M, D))
    for e in range(n):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            y[lo:hi] = mx_gemm(hq[lo:hi], hs[lo:hi], dq[e], ds[e])
    return dict(xq=xq, xs=xs, h=h, hq=hq, hs=hs, y=y)
