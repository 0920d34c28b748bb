"""Plain CPU oracle of the sparse MLA forward over an FP8 MLA KV cache (decode).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or run this module; the product path never does.
It shares no code, constants or helpers with the HIP library.

Where it comes from
-------------------
* "feat: add XTuner TileLang sparse MLA backend" (InternLM/lmdeploy PR 4904):
  its Summary rejects the FP8 MLA KV-cache path for the TileLang kernel, its
  per-file overview tests BF16 and FP8 sparse decode behaviour, and the
  DeepSeek-V3.2 configuration defaults the DSA MLA cache to BF16 "with explicit
  FP8 policy still possible elsewhere".
* The pages never lay out an FP8 row. Reading taken here (the published cache
  layout of DeepSeek-V3.2 sparse attention, to which the configuration
  refers): one 656-byte row per key,
      bytes   0 .. 511  512 latent values, float8 e4m3 (bias 7, no infinities,
                        S.1111.111 is NaN), in 4 groups of 128;
      bytes 512 .. 527  4 float32 scales (little endian), one per group;
      bytes 528 .. 655  64 rope values, bfloat16 (little endian).
  The dequantised row is latent[g*128 + i] = e4m3(byte) * scale[g] and
  rope[j] = bf16 value; everything else is the BF16 paged definition on the
  dequantised rows (oracle/sparse_mla_ref.py).

Dequantisation is exact here: e4m3 values and fp32 scales are held exactly
in float64, and so are their products.
"""
from __future__ import annotations

import numpy as np

from .sparse_mla_ref import sparse_mla_fwd_paged_ref

ROW_BYTES = 656
LATENT = 512
GROUP = 128
SCALE_OFF = 512
ROPE_OFF = 528


def e4m3_to_float(codes) -> np.ndarray:
    """float8 e4m3 codes (uint8) -> float64, from the format's definition:
    sign s, exponent e (4 bits, bias 7), mantissa m (3 bits);
    e == 0: (-1)^s * m/8 * 2^-6 (subnormal); e == 15, m == 7: NaN;
    otherwise (-1)^s * (1 + m/8) * 2^(e - 7)."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 15
    m = b & 7
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = s * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, val)


def dequantize_rows(raw) -> np.ndarray:
    """uint8 [..., 656] FP8 MLA rows -> float64 [..., 576] (latent, then rope)."""
    raw = np.ascontiguousarray(np.asarray(raw, dtype=np.uint8))
    assert raw.shape[-1] == ROW_BYTES
    lat = e4m3_to_float(raw[..., :LATENT])
    scales = raw[..., SCALE_OFF:ROPE_OFF].copy().view("<f4").astype(np.float64)   # [..., 4]
    lat = lat * np.repeat(scales, GROUP, axis=-1)
    rope_bits = raw[..., ROPE_OFF:].copy().view("<u2").astype(np.uint32) << 16
    rope = rope_bits.view(np.float32).astype(np.float64)
    return np.concatenate([lat, rope], axis=-1)


def sparse_mla_fwd_paged_fp8_ref(q, kv_pages_fp8, page_table, seq_lens, indices, sm_scale, q_per_seq,
                                 dtype=np.float64):
    """Sparse MLA forward over an FP8 paged cache: dequantise every row, then
    the BF16 paged definition.

    kv_pages_fp8: uint8 [num_pages, page_size, 656]; the other arguments as in
    sparse_mla_fwd_paged_ref.
    """
    kv = dequantize_rows(kv_pages_fp8)
    return sparse_mla_fwd_paged_ref(q, kv, page_table, seq_lens, indices, sm_scale, q_per_seq, dtype=dtype)
