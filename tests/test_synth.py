"""The seeded generator: deterministic, keyed per tensor, and shaped like the named
workloads (distribution sanity only; it holds no quantization arithmetic)."""
import numpy as np

import synth


def test_deterministic_and_keyed():
    a = synth.activations_bf16(3, 5, 64)
    b = synth.activations_bf16(3, 5, 64)
    c = synth.activations_bf16(4, 5, 64)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert not np.array_equal(synth.weight_codes(3, 5, 64, tensor_id=1), synth.weight_codes(3, 5, 64, tensor_id=2))


def test_row_prefix_is_stable():
    # rows come from per-chunk streams, so a smaller request is a prefix of a larger one
    a = synth.activations_bf16(7, 10, 32)
    b = synth.activations_bf16(7, 5000, 32)
    assert np.array_equal(a, b[:10])


def test_distributions():
    x = synth.activations_bf16(1, 256, 1024, outlier_p=0.01)
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    frac_big = np.mean(np.abs(xf) > 8)
    assert 0.005 < frac_big < 0.015
    w = synth.weight_codes(1, 64, 1024)
    assert not np.any((w & 0x7F) == 0x7F)
    mm = synth.masked_rows(3, 10000, 512)
    assert mm.min() == 0 and mm.max() == 512 and abs(mm.mean() - 256) < 8
    e = synth.e8m0_exponents(4, 100, 100)
    assert e.min() == 123 and e.max() == 131
    s = synth.block_scales(1, 100, 100)
    assert abs(np.mean(np.log(s))) < 0.02 and abs(np.std(np.log(s)) - 0.5) < 0.02
