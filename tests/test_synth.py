"""The seeded input generator: determinism, rounding, structure."""

import numpy as np

import synth


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9,
                  -2.5, 0.0, -0.0, np.inf, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    b = synth.f32_to_bf16_bits(x)
    back = synth.bf16_bits_to_f32(b)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 3*2^-8 ties between 1+2^-7 and 1+2^-6: even is 1 + 2^-6.
    expect = np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 0.0, -0.0, np.inf,
                       1.0 + 2 ** -7], dtype=np.float32)
    np.testing.assert_array_equal(back, expect)
    assert synth.f32_to_bf16_bits(np.array([np.nan], np.float32))[0] == 0x7FC0


def test_bf16_roundtrip_is_exact_on_representable_values():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    f = synth.bf16_bits_to_f32(bits)
    finite = np.isfinite(f)
    np.testing.assert_array_equal(synth.f32_to_bf16_bits(f[finite]), bits[finite])


def test_normal_is_deterministic_and_thread_count_independent(monkeypatch):
    monkeypatch.setattr(synth, "_BLOCK", 257)          # many blocks
    a = synth.normal(5, synth.S_K, (3, 1000), "f32")
    monkeypatch.setattr(synth, "_THREADS", 1)
    b = synth.normal(5, synth.S_K, (3, 1000), "f32")
    np.testing.assert_array_equal(a, b)
    c = synth.normal(6, synth.S_K, (3, 1000), "f32")
    assert not np.array_equal(a, c)
    assert abs(a.mean()) < 0.1 and abs(a.std() - 1) < 0.1
    # Blocks are distinct streams: no two blocks repeat each other.
    assert not np.array_equal(a.reshape(-1)[:257], a.reshape(-1)[257:514])
    # bf16 bits are the rounding of the same float32 samples.
    d = synth.normal(5, synth.S_K, (3, 1000), "bf16")
    np.testing.assert_array_equal(d, synth.f32_to_bf16_bits(a))


def test_symmetric_twin_shares_value_bytes():
    asym = synth.make_case(**{**synth.workload("decode32k_asym"), "ctx_len": 64})
    sym = synth.make_case(**{**synth.workload("decode32k_sym"), "ctx_len": 64})
    np.testing.assert_array_equal(asym.v_cache, sym.v_cache)
    assert asym.k_cache.shape == (1, 4, 64, 64) and sym.k_cache.shape == (1, 16, 64, 128)


def test_ragged_lengths_range_and_seed():
    L = synth.ragged_lengths(3, 1000, 4096, 32768)
    assert L.min() >= 4096 and L.max() <= 32768
    np.testing.assert_array_equal(L, synth.ragged_lengths(3, 1000, 4096, 32768))


def test_outlier_channels_count_and_scaling():
    for d_k, count in ((64, 3), (128, 6)):
        assert len(synth.outlier_channels(4, 4, d_k)) == count
    assert len(synth.outlier_channels(4, 16, 128)) == 21
    kw = {**synth.workload("decode64k_dk64"), "ctx_len": 32, "batch": 1}
    c = synth.make_case(**kw)
    base = synth.make_case(**{**kw, "outlier_frac": 0.0})
    kf, bf = synth.bf16_bits_to_f32(c.k_cache), synth.bf16_bits_to_f32(base.k_cache)
    for h, ch in c.outliers:
        np.testing.assert_array_equal(kf[:, h, :, ch], bf[:, h, :, ch] * 8)
    mask = np.ones(kf.shape, bool)
    for h, ch in c.outliers:
        mask[:, h, :, ch] = False
    np.testing.assert_array_equal(kf[mask], bf[mask])


def test_poisoned_tail():
    c = synth.make_case(1, dtype="bf16", batch=2, n_q=4, n_k=1, n_v=4, d_k=32,
                        d_v=64, ctx_len=[10, 20], l_cap=24, poison_tail=True)
    assert (c.k_cache[0, :, 10:] == 0x7FC0).all() and (c.k_cache[1, :, 20:] == 0x7FC0).all()
    assert not np.isnan(synth.bf16_bits_to_f32(c.v_cache[1, :, :20])).any()
