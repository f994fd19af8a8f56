"""The seeded input generators: SplitMix64 against its published outputs and a
pure-Python re-derivation, and the value ranges of the synthetic tensors."""
import numpy as np

import synthetic as syn


def test_splitmix64_published_sequence():
    # SplitMix64 seeded with 0 (Steele, Lea & Flood 2014; the reference C
    # implementation distributed with the xoshiro generators).
    got = [int(v) for v in syn.splitmix64(0, 3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_stream_matches_pure_python():
    base = syn.stream_base(123, 7, 511, 2, 1)
    state = base
    ref = []
    for _ in range(50):
        state = (state + syn.GAMMA) & syn.M64
        ref.append(syn.mix64_int(state))
    assert [int(v) for v in syn.splitmix64(base, 50)] == ref
    assert [int(v) for v in syn.splitmix64(base, 10, start=40)] == ref[40:]


def test_codes_bit_order_and_range():
    for bits in (4, 2):
        codes = syn.matrix_codes(0, 3, 1, 0, 16, 256, bits)
        words = syn.splitmix64(syn.stream_base(0, 3, 1, 0, 0), 16 * 256 * bits // 64)
        per = 64 // bits
        flat = codes.ravel()
        for i in (0, 1, per - 1, per, 12345 % flat.size, flat.size - 1):
            assert flat[i] == (int(words[i // per]) >> (bits * (i % per))) & ((1 << bits) - 1)
        hist = np.bincount(flat, minlength=1 << bits)
        assert hist.size == 1 << bits and hist.min() > 0.75 * flat.size / (1 << bits)


def test_scale_bias_ranges():
    s, b = syn.matrix_scale_bias(0, 0, 0, 1, 1024, 4096)
    sf, bf = syn.bf16_bits_to_f32(s), syn.bf16_bits_to_f32(b)
    assert sf.min() >= 0.005 - 1e-4 and sf.max() <= 0.02 + 1e-4
    assert bf.min() >= -0.1 - 1e-3 and bf.max() <= 0.0
    assert abs(sf.mean() - 0.0125) < 2e-4 and abs(bf.mean() + 0.05) < 2e-3


def test_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5], np.float32)
    got = syn.bf16_bits_to_f32(syn.f32_to_bf16_bits(f))
    assert list(got) == [1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5]


def test_distinct_streams():
    a = syn.matrix_codes(0, 0, 0, 0, 4, 64, 4)
    b = syn.matrix_codes(0, 0, 1, 0, 4, 64, 4)
    c = syn.matrix_codes(0, 1, 0, 0, 4, 64, 4)
    d = syn.matrix_codes(1, 0, 0, 0, 4, 64, 4)
    assert not np.array_equal(a, b) and not np.array_equal(a, c) and not np.array_equal(a, d)
