"""The seeded input generators (CPU only)."""
import numpy as np

import datagen


def test_splitmix64_published_sequence():
    # SplitMix64 seeded with state 0 (Steele, Lea, Flood 2014; the reference
    # implementation's first three outputs).
    w = [int(x) for x in datagen.words(0, 0, 3)]
    assert w == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_based_positions():
    a = datagen.words(5, 0, 100)
    b = datagen.words(5, 37, 20)
    assert np.array_equal(a[37:57], b)


def test_uniform_grid_and_range():
    u = datagen.uniform_pm1(1, 1 << 16).astype(np.float64)
    assert u.min() >= -1.0 and u.max() <= 1.0 - 2.0 ** -23
    assert np.all(u * 2 ** 23 == np.round(u * 2 ** 23))
    assert not np.any(np.signbit(u) & (u == 0))
    assert abs(u.mean()) < 0.02


def test_coarse_grid():
    c = datagen.coarse_pm1(2, 4096).astype(np.float64)
    assert set(np.unique(c * 16).astype(int)) <= set(range(-16, 16))


def test_normal_moments():
    n = datagen.normal01(3, 1 << 18).astype(np.float64)
    assert abs(n.mean()) < 0.01 and abs(n.std() - 1) < 0.01


def test_torch_twin_matches():
    u = datagen.uniform_pm1(9, 5000)
    ut = datagen.uniform_pm1_torch(9, 5000).numpy()
    assert np.array_equal(u, ut)
    n = datagen.normal01(4, 3000)
    nt = datagen.normal01_torch(4, 3000).numpy()
    assert np.allclose(n, nt, rtol=1e-6, atol=1e-6)


def test_page_pattern():
    a = datagen.page_pattern_a(200)
    b = datagen.page_pattern_b(200)
    assert a[96] == np.float32(96) * np.float32(0.01) and a[97] == 0
    assert b[0] == np.float32(-0.5) and b[53] == np.float32(-0.5)


def test_matrix_padding():
    m = datagen.matrix("uniform", 1, 3, 5, ld=8)
    assert m.shape == (3, 8) and np.all(np.isnan(m[:, 5:]))
    assert np.array_equal(m[:, :5].ravel(), datagen.uniform_pm1(1, 15))


def test_torch_twin_of_the_16bit_grid_matches():
    import torch
    for fmt, dt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        want = datagen.matrix16(9, 33, 515, fmt)
        got = datagen.grid16_torch(9, 33, 515, fmt)
        assert got.dtype == dt and got.shape == (33, 515)
        assert np.array_equal(got.view(torch.int16).numpy().view(np.uint16), want), fmt
