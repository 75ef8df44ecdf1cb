"""The seeded input generator: determinism, storage rounding, paging structure."""
import numpy as np
import pytest

from synth import (CONFIGS, bf16_bits_to_f32, block_table, f32_to_bf16_bits, generate,
                   pages_per_seq, seq_lens, sequence_rows, small)


def test_bf16_round_nearest_even_edges():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)        # bf16 spacing at 1.0
    vals = np.array([one, one + ulp / 2, one + 3 * ulp / 2, one + ulp / 2 + np.float32(2 ** -20),
                     -one - ulp / 2, np.array([0x7F7F8000], np.uint32).view(np.float32)[0], np.float32(1e-40), np.inf, -np.inf],
                    dtype=np.float32)
    got = bf16_bits_to_f32(f32_to_bf16_bits(vals))
    expect = np.array([1.0, 1.0, 1.0 + 2 * ulp, 1.0 + ulp, -1.0, np.inf, got[6], np.inf, -np.inf],
                      dtype=np.float32)
    assert np.array_equal(got[[0, 1, 2, 3, 4, 7, 8]], expect[[0, 1, 2, 3, 4, 7, 8]])
    assert np.isinf(got[5])            # tie above the largest finite bf16 goes to even: inf
    assert np.isnan(bf16_bits_to_f32(f32_to_bf16_bits(np.array([np.nan], np.float32))))[0]


def test_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    x = (np.random.default_rng(0).standard_normal(200000) * 10.0 ** np.random.default_rng(1)
         .integers(-20, 20, 200000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)


def test_generate_is_deterministic():
    cfg = small(CONFIGS["v2_varlen_b128"], "d", 3, (1, 500))
    a, b = generate(cfg), generate(cfg)
    for f in ("cache", "q_nope", "q_pe", "w_uk", "w_uv", "block_table", "seq_lens"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f


def test_varlen_lengths_pinned():
    L = seq_lens(CONFIGS["v2_varlen_b128"])
    assert L.shape == (128,) and int(L.sum()) == 2169799
    assert int(L.min()) == 1265 and int(L.max()) == 32534
    assert int(pages_per_seq(L, 64).sum()) == 33967


def test_block_table_is_a_bijection():
    for name in ("v2_b64_l8192", "v2_varlen_b128", "v2lite_b32_l4096"):
        cfg = CONFIGS[name]
        L = seq_lens(cfg)
        bt, total = block_table(cfg, L)
        npg = pages_per_seq(L, 64)
        used = np.concatenate([bt[b, :npg[b]] for b in range(cfg.batch)])
        assert used.size == total and np.array_equal(np.sort(used), np.arange(total))
        if not cfg.permute_pages:
            assert np.array_equal(used, np.arange(total))


def test_value_laws():
    cfg = small(CONFIGS["v2_b64_l8192"], "d", 2, 1000)
    wl = generate(cfg)
    rows = bf16_bits_to_f32(sequence_rows(cfg, 1, 1000)).astype(np.float64)
    # latent rows lie on the sphere of radius sqrt(512) up to bf16 rounding
    assert np.allclose(np.sqrt((rows[:, :512] ** 2).mean(1)), 1.0, atol=5e-3)
    assert abs(rows[:, 512:].std() - 1.0) < 0.02
    w = bf16_bits_to_f32(wl.w_uk).astype(np.float64)
    assert abs(w.std() * np.sqrt(512) - 1.0) < 0.01
    # unused slots are zero by default, NaN when poisoned
    p = generate(small(cfg, "d", 1, 70), pad_value=float("nan"))
    tail = bf16_bits_to_f32(p.cache[p.block_table[0, 1], 6:])
    assert np.isnan(tail).all()
