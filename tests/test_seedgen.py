"""The seeded generator: published SplitMix64 outputs, RNE rounding against torch's
conversions, determinism and basic distribution checks."""
import numpy as np
import pytest

import seedgen


def test_splitmix64_published_values():
    # SplitMix64 from state 0: first outputs as published with the reference C code.
    w = seedgen.splitmix64_words(0, 0, 0, 3)
    assert [int(x) for x in w] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_stream_offsets_and_keys():
    a = seedgen.splitmix64_words(1003, 2, 0, 100)
    b = seedgen.splitmix64_words(1003, 2, 40, 60)
    np.testing.assert_array_equal(a[40:], b)
    c = seedgen.splitmix64_words(1003, 3, 0, 100)
    assert not np.any(a == c)


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.concatenate([
        seedgen.normal_f64(5, 0, 200000).astype(np.float32) * 37.0,
        np.array([1.0, -1.0, 0.0, -0.0, 1.00390625, 1.01171875, 3.0e38, 1e-40], dtype=np.float32),
        # exact ties: 1 + 2^-8 sits halfway between two bf16 neighbours
        (np.float32(1.0) + np.float32(2.0 ** -8)) * np.array([1, 3, 5, 7], dtype=np.float32),
    ])
    ours = seedgen.round_f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(seedgen.bf16_bits_to_f64(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_draw_dtypes_and_widening():
    torch = pytest.importorskip("torch")
    for dt, tdt in (("bf16", torch.bfloat16), ("fp16", torch.float16), ("fp32", torch.float32)):
        d = seedgen.draw(1001, 0, (2, 3, 5, 8), dt)
        t = d.torch()
        assert t.dtype == tdt and tuple(t.shape) == (2, 3, 5, 8)
        np.testing.assert_array_equal(t.double().numpy(), d.f64)
        x32 = seedgen.normal_f64(1001, 0, 240).astype(np.float32)
        np.testing.assert_array_equal(t.reshape(-1).numpy() if dt == "fp32" else
                                      t.reshape(-1).float().numpy(),
                                      torch.from_numpy(x32).to(tdt).float().numpy())


def test_deterministic_and_scaled():
    a = seedgen.draw(1005, 1, (4, 64), "bf16", mul=0.5)
    b = seedgen.draw(1005, 1, (4, 64), "bf16", mul=0.5)
    np.testing.assert_array_equal(a.stored, b.stored)
    full = seedgen.normal_f64(1005, 1, 256)
    np.testing.assert_array_equal(a.f64.ravel(), seedgen.bf16_bits_to_f64(
        seedgen.round_f32_to_bf16_bits((full * 0.5).astype(np.float32))))


def test_normal_moments():
    x = seedgen.normal_f64(7, 0, 1 << 20)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1.0) < 5e-3
    assert abs(np.mean(x ** 3)) < 1e-2 and abs(np.mean(x ** 4) - 3.0) < 3e-2


def test_choice_rows():
    r = seedgen.choice_rows(1005, 16, 65536, 32)
    assert r.size == 32 and len(set(r.tolist())) == 32 and r.min() >= 0 and r.max() < 65536
    np.testing.assert_array_equal(r, seedgen.choice_rows(1005, 16, 65536, 32))


def test_block_mask_is_seeded_and_has_its_density():
    a = seedgen.block_mask(5, seedgen.TENSOR_MASK, (64, 64), 0.3)
    b = seedgen.block_mask(5, seedgen.TENSOR_MASK, (64, 64), 0.3)
    c = seedgen.block_mask(6, seedgen.TENSOR_MASK, (64, 64), 0.3)
    assert a.dtype == np.uint8 and a.shape == (64, 64)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert set(np.unique(a).tolist()) <= {0, 1}
    assert abs(a.mean() - 0.3) < 0.03


def test_e4m3_rounding_matches_torch():
    """The generator's fp32 -> e4m3 rounding (nearest, ties to even) against torch's
    float8_e4m3fn conversion, and exact widening back."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(20000) * 3, rng.standard_normal(5000) * 0.01,
                        rng.uniform(-448, 448, 5000), np.array([0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10,
                                                                1.0625, 1.1875, 0.0029296875])]).astype(np.float32)
    ours = seedgen.round_f32_to_e4m3_bits(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours & 0x7F, ref & 0x7F)
    nz = (ref & 0x7F) != 0
    np.testing.assert_array_equal(ours[nz], ref[nz])
    back = torch.from_numpy(ours.copy()).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(seedgen.e4m3_bits_to_f64(ours), back)
    d = seedgen.draw(3, 0, (4, 5), "fp8e4m3")
    assert d.stored.dtype == np.uint8 and d.f64.shape == (4, 5)
    with pytest.raises(ValueError):
        seedgen.round_f32_to_e4m3_bits(np.array([500.0], dtype=np.float32))


def test_lengths_are_seeded_and_cover_their_range():
    a = seedgen.lengths(3, seedgen.TENSOR_LENS, 4000, 256, 1024)
    assert a.dtype == np.int32 and a.shape == (4000,)
    assert np.array_equal(a, seedgen.lengths(3, seedgen.TENSOR_LENS, 4000, 256, 1024))
    assert not np.array_equal(a, seedgen.lengths(4, seedgen.TENSOR_LENS, 4000, 256, 1024))
    assert a.min() == 256 and a.max() == 1024
    assert abs(a.mean() - 640) < 15
    assert np.all(seedgen.lengths(1, 9, 50, 7, 7) == 7)
