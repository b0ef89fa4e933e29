"""Pin of the oracle's input decoder: bf16 bit patterns -> exact float64.

Every GPU parity check feeds the oracle through ``oracle.mla.bf16_bits_to_f64``,
so the decoder is pinned against a library routine (torch's bfloat16 ->
float64 conversion) on all 65,536 patterns, and a plausible slip (reading the
bits as IEEE binary16 instead of bfloat16) is planted to show the pin catches it.
"""

import numpy as np
import torch

from oracle import mla


def all_patterns():
    return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def torch_decode(bits):
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def decoder_mismatches(decode):
    """Patterns whose decoded value differs from torch's (NaN patterns must
    decode to NaN, every other pattern to the same float64, signed zeros and
    infinities included)."""
    bits = all_patterns()
    got = np.asarray(decode(bits), dtype=np.float64)
    ref = torch_decode(bits)
    nan_ref = np.isnan(ref)
    bad = nan_ref != np.isnan(got)
    ok = ~nan_ref & ~np.isnan(got)
    bad |= ok & ((got != ref) | (np.signbit(got) != np.signbit(ref)))
    return int(bad.sum())


def test_bf16_decoder_matches_torch_on_every_pattern():
    assert decoder_mismatches(mla.bf16_bits_to_f64) == 0


def test_bf16_decoder_special_values():
    f = mla.bf16_bits_to_f64
    v = f(np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x7F80, 0xFF80, 0x0001, 0x7F7F, 0x7FC0], np.uint16))
    assert v[0] == 0.0 and not np.signbit(v[0])
    assert v[1] == 0.0 and np.signbit(v[1])
    assert v[2] == 1.0 and v[3] == -1.0
    assert v[4] == np.inf and v[5] == -np.inf
    assert v[6] == 2.0 ** -133                      # smallest subnormal: 2^-126 * 2^-7
    assert v[7] == (2.0 - 2.0 ** -7) * 2.0 ** 127   # largest finite
    assert np.isnan(v[8])


def test_planted_binary16_decode_is_caught():
    """Reading the 16 bits as IEEE half precision (a plausible slip) fails the pin."""
    def as_half(bits):
        return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    assert decoder_mismatches(as_half) > 60000
