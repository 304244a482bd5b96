"""MXFP4 (OCP MX e2m1 elements, e8m0 block scales, block 32) dequantisation, float64.

Passages followed:
  * kimi-k3-mlx README, Architecture table, Source-format row: routed experts
    ship as MXFP4, a u8 `weight_packed` plus an e8m0 `weight_scale`, group 32.
  * kimi-k3-mlx README, Tiers section: MLX's mxfp4 mode uses the identical
    encoding -- low-nibble-first codes, e8m0 scales -- so the bytes are reused
    with no arithmetic.
  * K3 open-artifact audit, section 4.3: `w*.weight_packed` is u8 [N, K/2],
    `w*.weight_scale` is u8 [N, K/32] (3584/32 = 112, 3072/32 = 96).

Readings (the pages name the format but print no table):
  * e2m1 is the OCP MX v1.0 element: bit 3 sign, bits 2..1 exponent (bias 1),
    bit 0 mantissa; magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}; code 8 is -0.
  * byte b of a row holds element 2b in its low nibble and element 2b+1 in
    its high nibble ("low bits first").
  * e8m0 byte e means 2**(e - 127); e = 255 is NaN.
  * scale[n, g] applies to elements k of row n with k // 32 == g.
"""
from __future__ import annotations

import numpy as np

GROUP = 32

# e2m1 magnitudes by the 3 low code bits, then the sign bit.
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                        -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0], dtype=np.float64)


def e8m0_to_f64(e: np.ndarray) -> np.ndarray:
    """2**(e-127) for e in 0..254, NaN for 255."""
    e = np.asarray(e).astype(np.int64)
    out = np.ldexp(1.0, e - 127)
    return np.where(e == 255, np.nan, out)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """u8 [..., K/2] -> e2m1 codes u8 [..., K]; element 2b is the low nibble of byte b."""
    packed = np.asarray(packed, dtype=np.uint8)
    codes = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    codes[..., 0::2] = packed & 0x0F
    codes[..., 1::2] = packed >> 4
    return codes


def dequant(packed: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Dequantised weights float64 [..., N, K] = e2m1[code] * 2**(scale - 127)."""
    codes = unpack_codes(packed)
    K = codes.shape[-1]
    if scale.shape[-1] * GROUP != K:
        raise ValueError(f"scale has {scale.shape[-1]} groups for K={K}")
    vals = E2M1_VALUES[codes]
    s = e8m0_to_f64(scale)
    return vals * np.repeat(s, GROUP, axis=-1)
