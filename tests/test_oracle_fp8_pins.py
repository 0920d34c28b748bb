"""Pins of the FP8 MLA cache oracle (oracle/fp8_cache_ref.py), independent of
its own code, and planted mistakes that each fail a pin.

The row layout is a reading (stated in the oracle's header): 512 e4m3 latent
values in 4 groups of 128, 4 fp32 scales, 64 bf16 rope values; 656 bytes.

Pins:
* e4m3 decoding of all 256 codes against torch.float8_e4m3fn (a library
  routine), and a hand table of codes;
* one row laid out by hand: each group takes its own scale, the rope is not
  scaled, the byte offsets are 512 and 528;
* reduction to the BF16 path: a cache whose latent values are exactly
  representable in e4m3 with scale 1 gives exactly the BF16 paged oracle's
  result on the same values (which is pinned in test_oracle_pins.py).
"""
from __future__ import annotations

import inspect
import math
import types

import numpy as np
import pytest
import torch

import oracle.fp8_cache_ref as ref
from oracle import sparse_mla_fwd_paged_ref


def pin_e4m3_table(mod):
    codes = np.arange(256, dtype=np.uint8)
    got = mod.e4m3_to_float(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    by_hand = {0x00: 0.0, 0x38: 1.0, 0x7E: 448.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
               0xC6: -3.5, 0x3C: 1.5, 0x40: 2.0, 0x47: 3.75}
    for c, v in by_hand.items():
        assert mod.e4m3_to_float(np.array([c], dtype=np.uint8))[0] == v, hex(c)
    assert math.isnan(mod.e4m3_to_float(np.array([0x7F], dtype=np.uint8))[0])
    assert math.isnan(mod.e4m3_to_float(np.array([0xFF], dtype=np.uint8))[0])


def pin_row_by_hand(mod):
    row = np.zeros(656, dtype=np.uint8)
    row[0] = 0x38        # latent 0 = 1.0 (group 0)
    row[127] = 0x40      # latent 127 = 2.0 (group 0)
    row[128] = 0x38      # latent 128 = 1.0 (group 1)
    row[300] = 0xC6      # latent 300 = -3.5 (group 2)
    row[511] = 0x3C      # latent 511 = 1.5 (group 3)
    row[512:528] = np.array([0.5, 3.0, 0.25, -2.0], dtype="<f4").view(np.uint8)
    rope = np.array([1.0, -2.5] + [0.0] * 62, dtype=np.float32)
    row[528:656] = (rope.view(np.uint32) >> 16).astype("<u2").view(np.uint8)
    got = mod.dequantize_rows(row[None, :])[0]
    want = np.zeros(576)
    want[0], want[127], want[128], want[300], want[511] = 0.5, 1.0, 3.0, -0.875, -3.0
    want[512], want[513] = 1.0, -2.5
    assert np.array_equal(got, want)


def pin_reduces_to_bf16(mod):
    rng = np.random.default_rng(5)
    P, ps, S, Q, H, k = 6, 16, 2, 3, 4, 24
    codes = rng.integers(0, 256, (P, ps, 512)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x30                       # no NaN codes
    lat = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    rope = torch.randn((P, ps, 64), generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    raw = np.zeros((P, ps, 656), dtype=np.uint8)
    raw[..., :512] = codes
    raw[..., 512:528] = np.ones((P, ps, 4), dtype="<f4").view(np.uint8)
    raw[..., 528:] = rope.view(torch.int16).numpy().astype("<i2").view(np.uint8).reshape(P, ps, 128)
    kv = np.concatenate([lat, rope.double().numpy()], axis=-1)
    table = np.array([[3, 0, 5], [1, 4, 2]], dtype=np.int32)
    lens = np.array([40, 33], dtype=np.int32)
    q = torch.randn((S * Q, H, 576), generator=torch.Generator().manual_seed(2)).to(torch.bfloat16).double().numpy()
    idx = np.stack([rng.choice(41, k, replace=False) - 1 for _ in range(S * Q)]).astype(np.int32)
    sm = 0.05
    o8, l8 = mod.sparse_mla_fwd_paged_fp8_ref(q, raw, table, lens, idx, sm, Q)
    ob, lb = sparse_mla_fwd_paged_ref(q, kv, table, lens, idx, sm, Q)
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)


ALL_PINS = [pin_e4m3_table, pin_row_by_hand, pin_reduces_to_bf16]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(ref)


MUTANTS = {
    "exponent bias 8": ("np.exp2(e.astype(np.float64) - 7.0)", "np.exp2(e.astype(np.float64) - 8.0)"),
    "subnormals as normals": ("np.where(e == 0, sub, normal)", "normal"),
    "groups interleaved": ("np.repeat(scales, GROUP, axis=-1)", "np.tile(scales, GROUP)"),
    "scale on the rope too": ("return np.concatenate([lat, rope], axis=-1)",
                              "return np.concatenate([lat, rope * scales[..., :1]], axis=-1)"),
    "rope at byte 512": ("raw[..., ROPE_OFF:].copy()", "raw[..., SCALE_OFF:SCALE_OFF + 128].copy()"),
    "sign ignored": ("s = np.where(b >> 7, -1.0, 1.0)", "s = 1.0"),
    "mantissa over 16": ("normal = (1.0 + m / 8.0)", "normal = (1.0 + m / 16.0)"),
}


def _mutant(old, new):
    src = inspect.getsource(ref)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace("from .sparse_mla_ref import", "from oracle.sparse_mla_ref import")
    mod = types.ModuleType("fp8_mutant")
    exec(compile(src.replace(old, new), "fp8_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_mutant_fails_a_pin(name):
    mod = _mutant(*MUTANTS[name])
    caught = False
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception:
            caught = True
            break
    assert caught, f"no pin catches the mutant: {name}"
