"""Pins of the oracle's input handling, independent of the oracle's own code.

* ``widen`` (bf16 bit patterns -> float64) against torch's own bfloat16 ->
  float32 conversion, over every one of the 65536 bf16 bit patterns;
* the generator's float64 -> bf16 rounding against torch's float32 ->
  bfloat16 conversion (round to nearest even) on float32-exact values, and
  against hand-worked single roundings of float64 values that a float32
  detour would round twice;
* ``kv_head`` (the GQA map) against the MInference page's statement (section
  5.1, "head 分派与 GQA 映射"): with 32 query heads and 8 KV heads every four
  consecutive query heads share one K/V group, h_kv = floor(h_q / 4).
"""
import numpy as np
import torch

from oracle import minf_oracle as O
from synth import gen


def test_widen_every_bf16_pattern_matches_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = O.widen(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    with np.errstate(invalid="ignore"):
        ref = ref.astype(np.float64)
    nan = np.isnan(ref)
    assert nan.sum() == 2 * 127                       # exponent all ones, mantissa non-zero, both signs
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros and infinities keep their sign
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_widen_f32_is_exact():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(4096).astype(np.float32) * np.float32(1e-30)
    x[:4] = [0.0, -0.0, np.float32(3.4e38), np.float32(1e-45)]
    w = O.widen(x, "f32")
    assert w.dtype == np.float64
    assert np.array_equal(w.astype(np.float32).view(np.uint32), x.view(np.uint32))


def test_generator_rounding_matches_torch_on_f32_values():
    """For float32-exact values torch's conversion rounds once, to nearest
    even; the generator's float64 -> bf16 must agree bit for bit."""
    rng = np.random.default_rng(2)
    b = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    x = b.view(np.float32)
    x = x[np.isfinite(x)]
    # bf16 has float32's exponent range; values within half an ulp of the
    # largest bf16 round to it, larger ones overflow to infinity in both
    ours = gen.f64_to_bf16_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_generator_rounding_is_one_rounding_from_f64():
    """Round to nearest even straight from float64 (bf16 keeps 8 significant
    bits, so the ulp of [1, 2) is 2^-7): 1 + 2^-8 is a tie and goes to the
    even 1.0; a float64 value just above the tie goes up, although its
    float32 rounding is the tie itself; 1 + 3*2^-8 is a tie that goes up to
    the even 1 + 2^-6; the same mirrored for negative values."""
    cases = [
        (1.0 + 2.0 ** -8, 0x3F80),
        (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),
        (1.0 + 2.0 ** -8 - 2.0 ** -40, 0x3F80),
        (1.0 + 3 * 2.0 ** -8, 0x3F82),
        (-(1.0 + 2.0 ** -8 + 2.0 ** -40), 0xBF81),
        (-(1.0 + 3 * 2.0 ** -8), 0xBF82),
        (0.0, 0x0000),
        (2.0 ** -133, 0x0001),                 # the smallest bf16 subnormal
        (2.0 ** -134, 0x0000),                 # half of it: a tie, to the even 0
        (2.0 ** -134 + 2.0 ** -160, 0x0001),   # just above that tie
        (3.0, 0x4040),
    ]
    x = np.array([c[0] for c in cases], dtype=np.float64)
    got = gen.f64_to_bf16_bits(x)
    assert [int(v) for v in got] == [c[1] for c in cases]


def test_kv_head_groups_of_four_query_heads():
    """32 query heads over 8 KV heads: KV head g serves exactly the four
    consecutive query heads 4g .. 4g+3 (MInference page, section 5.1)."""
    groups = {}
    for h in range(32):
        groups.setdefault(O.kv_head(h, 32, 8), []).append(h)
    assert sorted(groups) == list(range(8))
    for g, hs in groups.items():
        assert hs == [4 * g, 4 * g + 1, 4 * g + 2, 4 * g + 3]
    # no sharing without GQA; all heads on one KV head with Hkv = 1
    assert [O.kv_head(h, 4, 4) for h in range(4)] == [0, 1, 2, 3]
    assert {O.kv_head(h, 8, 1) for h in range(8)} == {0}
