"""The seeded input generator (CPU only)."""
import numpy as np
import torch

import synth


def test_splitmix64_published_vectors():
    # First outputs of a SplitMix64 stream seeded with 0 and with 1234567
    # (the test values published with the algorithm's reference code).
    L = synth.lib()
    assert [L.synth_splitmix64(0, i) for i in range(4)] == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F, 0xF88BB8A8724C81EC]
    assert L.synth_splitmix64(1234567, 0) == 6457827717110365317


def test_independent_of_thread_count():
    a = synth.normal(300_001, 77, synth.BF16, nthreads=1)
    b = synth.normal(300_001, 77, synth.BF16, nthreads=7)
    assert np.array_equal(a, b)
    c = synth.normal(300_001, 77, synth.F32, 2.0, 1000, 0.01, nthreads=3)
    d = synth.normal(300_001, 77, synth.F32, 2.0, 1000, 0.01, nthreads=0)
    assert np.array_equal(c, d)


def test_prefix_property_and_seeds_differ():
    a = synth.normal(1000, 5, synth.F32)
    b = synth.normal(5000, 5, synth.F32)
    assert np.array_equal(a, b[:1000])
    assert not np.array_equal(a, synth.normal(1000, 6, synth.F32))


def test_normal_moments():
    z = synth.normal(2_000_000, 1, synth.F32).astype(np.float64)
    n = z.size
    assert abs(z.mean()) < 5 / np.sqrt(n)
    assert abs(z.var() - 1) < 5 * np.sqrt(2 / n)
    assert abs((z ** 3).mean()) < 5 * np.sqrt(15 / n)
    assert abs((z ** 4).mean() - 3) < 5 * np.sqrt(96 / n)
    assert abs((np.abs(z) < 1).mean() - 0.682689492) < 0.002


def test_bf16_is_rne_of_the_float_values():
    f = synth.normal(100_000, 9, synth.F32, 3.0)
    b = synth.normal(100_000, 9, synth.BF16, 3.0)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)
    assert np.array_equal(synth.bf16_bits_to_f32(b), torch.from_numpy(f).to(torch.bfloat16).float().numpy())


def test_frame_slope_and_weight_scale():
    F, S, C = 64, 50, 32
    x = synth.make_tensor(4, synth.X_GN, F, 10, 5, C, synth.F32, slope=0.3)
    means = x.reshape(F, -1).mean(axis=1)
    assert np.abs(means - 0.3 * np.arange(F) / F).max() < 5 / np.sqrt(S * C)
    w = synth.make_conv_weight(3, 640, synth.F32)
    assert w.shape == (3, 640, 640)
    assert abs(w.astype(np.float64).var() * 3 * 640 - 1) < 0.01
