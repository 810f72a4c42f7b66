"""Storage-format encoders for synthetic inputs: bf16, OCP FP8 E4M3, OCP MXFP4.

These turn generated float64 values into the bytes that both the GPU path and
the CPU oracle read.  Encoding happens once, here; each side decodes the bytes
with its own code.

Formats follow the public Open Compute Project specifications:
  * OCP 8-bit Floating Point Specification (OFP8) v1.0: E4M3 with bias 7,
    no infinities, NaN = S.1111.111, largest finite 448.
  * OCP Microscaling Formats (MX) v1.0: MXFP4 = blocks of 32 FP4 (E2M1)
    elements sharing one E8M0 scale; shared exponent = floor(log2(amax)) - 2
    (2 = emax of E2M1); elements round to nearest even and saturate at +-6.

Per-row scaling for FP8 (scale = amax / 448) is this project's choice of
quantisation recipe; the element encoding itself is the OCP one.
"""
from __future__ import annotations

import numpy as np

FP8_E4M3_MAX = 448.0


def bf16_bits(x) -> np.ndarray:
    """Round float values to bfloat16 (round-to-nearest-even), return uint16 bits."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_round(x) -> np.ndarray:
    """float32 values exactly representable in bf16 (RNE of x)."""
    return (bf16_bits(x).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _e4m3_encode_abs(a: np.ndarray) -> np.ndarray:
    """|value| (float64, already <= 448 after saturation) -> 7-bit E4M3 magnitude code."""
    a = np.minimum(a, FP8_E4M3_MAX)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)
    quantum = np.exp2(e - 3)                      # spacing of the 3-bit mantissa grid
    q = np.rint(a / quantum) * quantum            # RNE on the grid of this binade
    q = np.minimum(q, FP8_E4M3_MAX)
    # re-derive fields from the rounded value (rounding may move to the next binade)
    with np.errstate(divide="ignore"):
        e2 = np.floor(np.log2(np.where(q > 0, q, 1.0)))
    normal = q >= 2.0 ** -6
    e2 = np.where(normal, e2, -6)
    exp_field = np.where(normal, e2 + 7, 0).astype(np.int64)
    mant = np.where(normal, q / np.exp2(e2) * 8 - 8, q / 2.0 ** -9)
    code = (exp_field << 3) | np.rint(mant).astype(np.int64)
    code = np.where(q == 0, 0, code)
    return code.astype(np.uint8)


def fp8_e4m3_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """Quantise each row: scale = amax/448 (float32), code = E4M3(x/scale), RNE, saturating.

    Returns (codes uint8 [..., cols], scale float32 [...]).
    """
    x = np.asarray(x, dtype=np.float64)
    amax = np.abs(x).max(axis=-1)
    scale = (amax / FP8_E4M3_MAX).astype(np.float32)
    scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    v = x / scale.astype(np.float64)[..., None]
    code = _e4m3_encode_abs(np.abs(v))
    code = code | np.where(v < 0, 0x80, 0).astype(np.uint8)
    return code.astype(np.uint8), scale


_E2M1_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])  # midpoints of the E2M1 grid


def _e2m1_encode_abs(a: np.ndarray) -> np.ndarray:
    """|value| -> 3-bit E2M1 magnitude code: nearest grid value, ties to the even code,
    saturating at 6."""
    a = np.minimum(a, 6.0)
    code = np.searchsorted(_E2M1_MID, a, side="left")  # a on a midpoint -> the lower code
    on_mid = (code < 7) & (a == _E2M1_MID[np.minimum(code, 6)])
    code = np.where(on_mid & (code % 2 == 1), code + 1, code)
    return code.astype(np.uint8)


def mxfp4_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """Quantise rows to MXFP4.  Row length must be a multiple of 32.

    Returns (packed uint8 [..., cols/2], e8m0 uint8 [..., cols/32]).  Element 2j of
    a row sits in the low nibble of byte j, element 2j+1 in the high nibble.
    """
    x = np.asarray(x, dtype=np.float64)
    cols = x.shape[-1]
    assert cols % 32 == 0
    blk = x.reshape(x.shape[:-1] + (cols // 32, 32))
    amax = np.abs(blk).max(axis=-1)
    with np.errstate(divide="ignore"):
        sexp = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2.0
    sexp = np.where(amax > 0, sexp, 0.0)
    sexp = np.clip(sexp, -127, 127)
    e8m0 = (sexp + 127).astype(np.uint8)
    v = blk / np.exp2(sexp)[..., None]
    code = _e2m1_encode_abs(np.abs(v)) | np.where(v < 0, 8, 0).astype(np.uint8)
    code = code.reshape(x.shape[:-1] + (cols,))
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return packed, e8m0


def kv576_rows(x, rope_dims=64) -> tuple[np.ndarray, np.ndarray]:
    """Rows [..][c] -> production cache rows [..][c + rope_dims] bytes (E4M3 codes of the
    c - rope_dims leading channels with one float32 scale per row, then the rope_dims
    channels as little-endian bf16) and the scales [..]."""
    x = np.asarray(x, dtype=np.float64)
    c = x.shape[-1]
    nq = c - rope_dims
    codes, scale = fp8_e4m3_rows(x[..., :nq])
    tail = bf16_bits(x[..., nq:]).view(np.uint8)
    return np.concatenate([codes, tail], axis=-1), scale
