"""Pin of the oracle's fp32 -> bf16 rounding and bf16 -> fp32 widening.

Against a library routine: torch's CPU float32 -> bfloat16 conversion (round
to nearest, ties to even).  NaN is compared by NaN-ness only (payloads are
implementation choices); the oracle's NaN must be 0x7FC0.
"""
import numpy as np
import torch

from oracle import _c


def _patterns():
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    # low halves: exact, just below / at / above the tie, odd / even cases
    lows = np.array([0x0000, 0x0001, 0x3FFF, 0x7FFF, 0x8000, 0x8001, 0xBFFF, 0xFFFF],
                    dtype=np.uint32)
    rng = np.random.default_rng(1234)
    lows = np.concatenate([lows, rng.integers(0, 1 << 16, 8, dtype=np.uint32)])
    return (hi[:, None] | lows[None, :]).reshape(-1)


def test_rne_matches_torch_cpu_cast():
    bits = _patterns()                                   # ~1M patterns, every exponent
    x = bits.view(np.float32)
    ours = _c.f32_to_bf16(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all(ours[nan] == 0x7FC0)


def test_widening_is_exact():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = _c.bf16_to_f32(h)
    ref = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    same = (f.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(f) & np.isnan(ref))
    assert same.all()
    # and the widening is the 16-bit shift: every non-NaN pattern round-trips
    back = _c.f32_to_bf16(f)
    ok = ~np.isnan(f)
    assert np.array_equal(back[ok], h[ok])


def test_special_values():
    x = np.array([0.0, -0.0, np.inf, -np.inf, 1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8,
                  np.float32(3.4028235e38), 1e-45], dtype=np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even wins (1); 1 + 3*2^-8 is a
    # tie between 1 + 2^-7 (odd) and 1 + 2^-6 (even): rounds up; FLT_MAX
    # rounds to +Inf; the smallest subnormal rounds to +0 (below half of the
    # smallest bf16 subnormal 2^-133)
    expect = np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x3F80, 0x3F80, 0x3F82,
                       0x7F80, 0x0000], dtype=np.uint16)
    assert np.array_equal(_c.f32_to_bf16(x), expect)


def test_rne_matches_torch_on_every_fp32_pattern():
    # all 2^32 bit patterns, in chunks of 2^26
    step = 1 << 26
    base = np.arange(step, dtype=np.uint32)
    for start in range(0, 1 << 32, step):
        x = (base + np.uint32(start)).view(np.float32)
        ours = _c.f32_to_bf16(x)
        ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(x)
        assert np.array_equal(ours[~nan], ref[~nan]), hex(start)
        assert np.all(ours[nan] == 0x7FC0), hex(start)
