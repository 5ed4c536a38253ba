"""FP8 MLA latent rows decoded to float64 (TEST INFRASTRUCTURE: oracle only).

The pages' FP8 KV cache keeps one 656-byte record per token (sglang PR 32320,
summary and "Modifications": pages of 656-byte FP8 rows; PR 32779, "Accuracy
Tests" (c): the FP8-native kernel consumes the pool with its scales) and
compare it with the 1152-byte bf16 latent row. The byte layout is not
printed; the reading used here is the one that accounts for all 656 bytes
of a 576-wide row (512 latent + 64 rope):

    bytes   0 .. 511   512 latent values, OCP FP8 E4M3 (e4m3fn)
    bytes 512 .. 527   four little-endian fp32 scales; scale b multiplies
                       latent values 128 b .. 128 b + 127
    bytes 528 .. 655   64 rope values, bf16

The pages' kernel never reads FP8 codes in its products: the pool's rows
reach it already dequantised to bf16, and its matrix products run in bf16
(sglang PR 32779, "Accuracy Tests" (c), which sets it against an FP8-native
kernel that applies the scales itself). So a latent value is dequantised as
the fp32 product fp32(code) * scale, rounded to nearest even, then rounded
to nearest even bf16; the decoded row
is [those 512 values | rope (64)], of which the first 512 also serve as V,
as for the bf16 latent row.

E4M3 (OCP "e4m3fn"): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
bits; exponent field 0 is subnormal (m / 8 * 2^-6); the pattern S.1111.111
is NaN; there are no infinities.
"""
from __future__ import annotations

import numpy as np

from .attention import bf16_to_f64

ROW_BYTES = 656
LATENT = 512
ROPE = 64
BLOCK = 128


def fp8_e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = sign * np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> float64 holding the nearest-even bf16 value (NaN kept)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = bf16_to_f64((r & 0xFFFF).astype(np.uint16))
    return np.where(np.isnan(x), np.nan, out)


def mla_fp8_rows_to_f64(rows: np.ndarray) -> np.ndarray:
    """uint8 [..., 656] records -> float64 [..., 576] rows."""
    r = np.ascontiguousarray(rows, dtype=np.uint8)
    assert r.shape[-1] == ROW_BYTES
    code = fp8_e4m3_to_f64(r[..., :LATENT]).astype(np.float32)        # exact
    scales = r[..., LATENT:LATENT + 16].copy().view("<f4")
    with np.errstate(invalid="ignore", over="ignore"):
        prod = code * np.repeat(scales, BLOCK, axis=-1)                 # fp32, nearest even
    latent = f32_to_bf16_rne(prod)
    rope = bf16_to_f64(r[..., LATENT + 16:].copy().view("<u2"))
    return np.concatenate([latent, rope], axis=-1)
