"""Pins of the fp64 oracle against what the pages and mathematics fix.

Each check_* function raises AssertionError on a mismatch; the test_* functions
run them on the oracle as written, and the mutation tests run them on an
oracle with a planted mistake to show that the pins catch it.
"""
import json
import os

import numpy as np
import pytest

import oracle.mla_oracle as O
from synth import CONFIGS, generate, hidden_recipe, sequence_rows, small

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TINY = CONFIGS["tiny_f32"]
RNG = np.random.default_rng(1234)


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def rand_case(n_h=3, d_h=8, d_c=24, d_r=4, L=5, seed=0):
    r = np.random.default_rng(seed)
    return dict(c=r.standard_normal((L, d_c)), k_rope=r.standard_normal((L, d_r)),
                q_nope=r.standard_normal((n_h, d_h)), q_pe=r.standard_normal((n_h, d_r)),
                w_uk=r.standard_normal((n_h * d_h, d_c)) / np.sqrt(d_c),
                w_uv=r.standard_normal((n_h * d_h, d_c)) / np.sqrt(d_c))


# ---------------------------------------------------------------------------
# cache-size closed forms (the pages' own numbers)
# ---------------------------------------------------------------------------
def test_cache_size_closed_forms():
    g = json.load(open(os.path.join(GOLDEN, "cache_size.json")))
    for name in ("v2lite_b32_l4096", "v2_b64_l8192", "v2_varlen_b128", "v2_b8_l131072"):
        cfg = CONFIGS[name]
        assert cfg.d_latent == g["d_latent_over_d_head"] * cfg.d_head
        assert cfg.d_rope == g["d_rope_over_d_head"] * cfg.d_head
        assert cfg.d_latent + cfg.d_rope == g["per_token_elements_over_d_head"] * cfg.d_head == 576
        # GQA with n_g groups caches 2 n_g d_h; equal to MLA's 4.5 d_h at n_g = 2.25
        assert (cfg.d_latent + cfg.d_rope) / (2 * cfg.d_head) == g["gqa_equivalent_groups"]
        assert (cfg.d_latent + cfg.d_rope) * 2 == 1152          # bytes per bf16 row
    v2 = CONFIGS["v2_b64_l8192"]
    assert 2 * v2.n_heads * v2.d_head == 32768                   # MHA per token per layer
    assert TINY.d_latent + TINY.d_rope == 4.5 * TINY.d_head == 72
    # one oracle row is exactly d_c + d_h^R wide
    wl = generate(small(v2, "s", 1, 70))
    assert O.gather_rows(wl.cache, wl.block_table[0], 70, 64).shape == (70, 576)


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------
def check_rope_planar():
    # d = 2: theta_0 = 1, so position m rotates by m radians, counter-clockwise
    x = np.array([0.3, -1.7])
    for m in (0, 1, 5, 131071):
        R = np.array([[np.cos(m), -np.sin(m)], [np.sin(m), np.cos(m)]])
        assert rel(O.rope(x, m, 10000.0), R @ x) < 1e-14


def check_rope_pairing():
    # d = 4, base 1e4: pairs (0,1) at theta 1 and (2,3) at theta 1e4^(-1/2) = 0.01
    m = 7.0
    e2 = np.array([0.0, 0.0, 1.0, 0.0])
    assert rel(O.rope(e2, m, 1e4), [0, 0, np.cos(0.01 * m), np.sin(0.01 * m)]) < 1e-14
    e1 = np.array([0.0, 1.0, 0.0, 0.0])
    assert rel(O.rope(e1, m, 1e4), [-np.sin(m), np.cos(m), 0, 0]) < 1e-14
    assert np.allclose(O.rope_theta(64, 1e4)[[0, 1, 31]], [1.0, 1e4 ** (-2 / 64), 1e4 ** (-62 / 64)],
                       rtol=1e-15)


def check_rope_identities():
    d = 64
    x, y = RNG.standard_normal(d), RNG.standard_normal(d)
    assert np.array_equal(O.rope(x, 0, 1e4), x)                          # R_0 = I
    for m, n in ((3, 11), (100, 7), (131071, 65536)):
        Rm = O.rope_matrix(m, d, 1e4)
        assert np.allclose(Rm @ Rm.T, np.eye(d), atol=1e-14)             # orthogonal
        assert rel(Rm @ x, O.rope(x, m, 1e4)) < 1e-13
        assert abs(np.linalg.norm(O.rope(x, m, 1e4)) - np.linalg.norm(x)) < 1e-12
        # S = Q^T R_m^T R_n K depends only on n - m
        lhs = O.rope(x, m, 1e4) @ O.rope(y, n, 1e4)
        rhs = x @ O.rope(y, n - m, 1e4)
        assert abs(lhs - rhs) < 1e-11 * np.linalg.norm(x) * np.linalg.norm(y)


def test_rope_planar():
    check_rope_planar()


def test_rope_pairing():
    check_rope_pairing()


def test_cache_rows_from_hidden_properties():
    """The cache-write recipe against properties that hold whatever its code:
    the normalised latent keeps the direction of W^DKV h and has mean square
    ms / (ms + eps) (ms that of W^DKV h); without the norm it is W^DKV h; the
    key part is W^KR h at position 0 and has its norm at every position."""
    rng = np.random.default_rng(5)
    T, dm, dc, dr = 6, 40, 16, 8
    h = rng.standard_normal((T, dm))
    w_dkv = rng.standard_normal((dc, dm)) / np.sqrt(dm)
    w_kr = rng.standard_normal((dr, dm)) / np.sqrt(dm)
    pos = np.array([0, 1, 7, 100, 4095, 131071])
    eps = 1e-6
    raw_c = np.einsum("cd,td->tc", w_dkv, h)
    raw_k = np.einsum("rd,td->tr", w_kr, h)
    rows = O.cache_rows_from_hidden(h, w_dkv, w_kr, pos, 1e4, rms_norm=True, eps=eps)
    c, kr = rows[:, :dc], rows[:, dc:]
    ms = (raw_c ** 2).mean(axis=1)
    assert np.allclose((c ** 2).mean(axis=1), ms / (ms + eps), rtol=1e-13, atol=0)
    ratio = c / raw_c
    assert np.all(ratio > 0) and np.allclose(ratio, ratio[:, :1], rtol=1e-12, atol=0)
    assert np.array_equal(kr[0], raw_k[0]) or rel(kr[0], raw_k[0]) < 1e-15
    assert np.allclose(np.linalg.norm(kr, axis=1), np.linalg.norm(raw_k, axis=1), rtol=1e-13, atol=0)
    plain = O.cache_rows_from_hidden(h, w_dkv, w_kr, pos, 1e4, rms_norm=False)
    assert rel(plain[:, :dc], raw_c) < 1e-14
    assert rel(plain[:, dc:], kr) < 1e-14   # the norm of c does not touch the key part
    # one hidden state at several positions: the key part is rotated by the
    # position (it moves away from W^KR h), and the inner product of two
    # encodings depends only on the difference of their positions
    hp = np.repeat(h[:1], 4, axis=0)
    same = O.cache_rows_from_hidden(hp, w_dkv, w_kr, np.array([3, 4, 50, 51]), 1e4, rms_norm=True)[:, dc:]
    assert rel(same[1], raw_k[0]) > 1e-3 and rel(same[0], same[1]) > 1e-3
    assert abs(same[0] @ same[1] - same[2] @ same[3]) < 1e-12 * (raw_k[0] @ raw_k[0])


def check_cache_rows_from_hidden():
    test_cache_rows_from_hidden_properties()


def _cache_rows_norm_over_tokens(h, w_dkv, w_kr, positions, rope_base, rms_norm, eps=1e-6):
    c = np.asarray(h, np.float64) @ np.asarray(w_dkv, np.float64).T
    if rms_norm:
        c = c / np.sqrt((c * c).mean(axis=0, keepdims=True) + eps)
    kr = O.rope(np.asarray(h, np.float64) @ np.asarray(w_kr, np.float64).T, np.asarray(positions), rope_base)
    return np.concatenate([c, kr], axis=1)


def _cache_rows_unrotated(h, w_dkv, w_kr, positions, rope_base, rms_norm, eps=1e-6):
    c = np.asarray(h, np.float64) @ np.asarray(w_dkv, np.float64).T
    if rms_norm:
        c = c / np.sqrt((c * c).mean(axis=1, keepdims=True) + eps)
    return np.concatenate([c, np.asarray(h, np.float64) @ np.asarray(w_kr, np.float64).T], axis=1)


def _cache_rows_first_position(h, w_dkv, w_kr, positions, rope_base, rms_norm, eps=1e-6):
    c = np.asarray(h, np.float64) @ np.asarray(w_dkv, np.float64).T
    if rms_norm:
        c = c / np.sqrt((c * c).mean(axis=1, keepdims=True) + eps)
    kr = O.rope(np.asarray(h, np.float64) @ np.asarray(w_kr, np.float64).T, np.asarray(positions)[0], rope_base)
    return np.concatenate([c, kr], axis=1)


@pytest.mark.parametrize("replacement", [_cache_rows_norm_over_tokens, _cache_rows_unrotated,
                                         _cache_rows_first_position])
def test_planted_cache_row_mistake_is_caught(monkeypatch, replacement):
    monkeypatch.setattr(O, "cache_rows_from_hidden", replacement)
    with pytest.raises(AssertionError):
        check_cache_rows_from_hidden()


def test_rope_identities():
    check_rope_identities()


# ---------------------------------------------------------------------------
# closed forms of the decode step
# ---------------------------------------------------------------------------
def check_single_token():
    # L = 1: softmax weight 1, o_i = W^UV_i c_0, lse = s_00 (query at position 0: R_0 = I)
    k = rand_case(L=1)
    r = O.naive_decode_seq(**k, pos=0, scale=0.25, rope_base=1e4)
    n_h, d_h = k["q_nope"].shape
    for i in range(n_h):
        wv = k["w_uv"][i * d_h:(i + 1) * d_h]
        wk = k["w_uk"][i * d_h:(i + 1) * d_h]
        assert rel(r["o"][i], wv @ k["c"][0]) < 1e-14
        assert rel(r["o_latent"][i], k["c"][0]) < 1e-15
        s = 0.25 * (k["q_nope"][i] @ (wk @ k["c"][0]) + k["q_pe"][i] @ k["k_rope"][0])
        assert abs(r["lse"][i] - s) < 1e-13


def check_equal_scores():
    # zero query: every score is 0, weights 1/L, o_i = W^UV_i mean_j c_j, lse = ln L
    k = rand_case(L=9)
    k["q_nope"][:] = 0
    k["q_pe"][:] = 0
    r = O.naive_decode_seq(**k, pos=4, scale=0.3, rope_base=1e4)
    d_h = k["q_nope"].shape[1]
    mean_c = k["c"].mean(axis=0)
    for i in range(k["q_nope"].shape[0]):
        assert rel(r["o"][i], k["w_uv"][i * d_h:(i + 1) * d_h] @ mean_c) < 1e-13
        assert rel(r["o_latent"][i], mean_c) < 1e-14
        assert abs(r["lse"][i] - np.log(9)) < 1e-14


def check_identical_tokens():
    # all tokens equal (c_j = c, k^R_j = 0): o_i = W^UV_i c whatever the query
    k = rand_case(L=6)
    k["c"][:] = k["c"][0]
    k["k_rope"][:] = 0
    r = O.naive_decode_seq(**k, pos=5, scale=0.2, rope_base=1e4)
    d_h = k["q_nope"].shape[1]
    for i in range(k["q_nope"].shape[0]):
        assert rel(r["o"][i], k["w_uv"][i * d_h:(i + 1) * d_h] @ k["c"][0]) < 1e-13


def check_two_token_rope_part():
    # q^C = 0, query at position 0, q^R = t e_0, k^R_0 = e_0, k^R_1 = 0:
    # s_0 = t / sqrt(d_h + d_h^R), s_1 = 0 -> a_0 = logistic(s_0)
    n_h, d_h, d_c, d_r = 2, 8, 24, 4
    k = rand_case(n_h, d_h, d_c, d_r, L=2)
    k["q_nope"][:] = 0
    k["q_pe"][:] = 0
    k["q_pe"][:, 0] = [1.5, -2.0]
    k["k_rope"][:] = 0
    k["k_rope"][0, 0] = 1.0
    scale = 1 / np.sqrt(d_h + d_r)
    r = O.naive_decode_seq(**k, pos=0, scale=O.softmax_scale(d_h, d_r), rope_base=1e4)
    for i, t in enumerate([1.5, -2.0]):
        s0 = scale * t
        a0 = 1 / (1 + np.exp(-s0))
        wv = k["w_uv"][i * d_h:(i + 1) * d_h]
        assert rel(r["o"][i], a0 * (wv @ k["c"][0]) + (1 - a0) * (wv @ k["c"][1])) < 1e-13
        assert abs(r["lse"][i] - np.log(np.exp(s0) + 1)) < 1e-13


def check_head_rows():
    # head i owns rows i*d_h .. i*d_h+d_h-1 of W^UK and W^UV.  With selection rows
    # W^UK[i d_h + r] = e_{(r + 3i) % d_c} and W^UV[i d_h + r] = e_{(r + 5i) % d_c},
    # q^C_i = t_i e_0 and no RoPE part: s_ij = scale t_i c_j[3i % d_c] and
    # o_i[r] = sum_j a_ij c_j[(r + 5i) % d_c].
    n_h, d_h, d_c, d_r, L = 4, 6, 20, 2, 5
    k = rand_case(n_h, d_h, d_c, d_r, L=L)
    k["w_uk"][:] = 0
    k["w_uv"][:] = 0
    for i in range(n_h):
        for r_ in range(d_h):
            k["w_uk"][i * d_h + r_, (r_ + 3 * i) % d_c] = 1
            k["w_uv"][i * d_h + r_, (r_ + 5 * i) % d_c] = 1
    t = np.array([0.7, -1.1, 2.3, 0.4])
    k["q_nope"][:] = 0
    k["q_nope"][:, 0] = t
    k["q_pe"][:] = 0
    scale = 0.5
    res = O.naive_decode_seq(**k, pos=3, scale=scale, rope_base=1e4)
    for i in range(n_h):
        s = scale * t[i] * k["c"][:, (3 * i) % d_c]
        a = np.exp(s - s.max())
        a /= a.sum()
        expect = np.array([a @ k["c"][:, (r_ + 5 * i) % d_c] for r_ in range(d_h)])
        assert rel(res["o"][i], expect) < 1e-13
        # q~_i = (W^UK_i)^T q^C_i = t_i e_{3i % d_c}
        qt = np.zeros(d_c)
        qt[(3 * i) % d_c] = t[i]
        assert rel(res["q_abs"][i, :d_c], qt) < 1e-15


def test_single_token():
    check_single_token()


def test_equal_scores():
    check_equal_scores()


def test_identical_tokens():
    check_identical_tokens()


def test_two_token_rope_part():
    check_two_token_rope_part()


def test_head_rows():
    check_head_rows()


# ---------------------------------------------------------------------------
# library attention and the absorbed form
# ---------------------------------------------------------------------------
def check_matches_sdpa():
    torch = pytest.importorskip("torch")
    n_h, d_h, d_c, d_r, L = 5, 16, 40, 8, 33
    k = rand_case(n_h, d_h, d_c, d_r, L=L, seed=7)
    pos = 32
    scale = O.softmax_scale(d_h, d_r)
    r = O.naive_decode_seq(**k, pos=pos, scale=scale, rope_base=1e4)
    # keys/values by the pages' definitions, attention by torch's routine (float64, CPU)
    K = np.stack([np.concatenate([k["c"] @ k["w_uk"][i * d_h:(i + 1) * d_h].T, k["k_rope"]], 1)
                  for i in range(n_h)])
    V = np.stack([k["c"] @ k["w_uv"][i * d_h:(i + 1) * d_h].T for i in range(n_h)])
    q = np.concatenate([k["q_nope"], O.rope(k["q_pe"], pos, 1e4)], 1)[:, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None],
        scale=scale)[0, :, 0].numpy()
    assert rel(r["o"], ref) < 1e-13


def test_matches_sdpa():
    check_matches_sdpa()


def check_absorbed_equals_naive_full_recipe(cfg=TINY, delta=0):
    # Tiny workload from hidden states: cache and query derived by the oracle.
    L = cfg.seq_len
    raw = hidden_recipe(cfg, L)
    pos = np.arange(L) + delta
    rows = O.cache_rows_from_hidden(raw["h"], raw["w_dkv"], raw["w_kr"], pos, cfg.rope_base,
                                    rms_norm=cfg.rms_norm_latent)
    qn, qp = O.query_from_hidden(raw["h"][L - 1], raw["w_q"], raw["w_qr"], cfg.n_heads)
    scale = O.softmax_scale(cfg.d_head, cfg.d_rope)
    args = (rows[:, :cfg.d_latent], rows[:, cfg.d_latent:], qn, qp, L - 1 + delta,
            raw["w_uk"], raw["w_uv"], scale, cfg.rope_base)
    nv = O.naive_decode_seq(*args)
    ab = O.absorbed_decode_seq(*args)
    for key in ("o", "o_latent", "lse", "q_abs"):
        assert rel(nv[key], ab[key]) < 1e-12, key
    # o_i = W^UV_i o~_i
    d_h = cfg.d_head
    for i in range(cfg.n_heads):
        assert rel(nv["o"][i], raw["w_uv"][i * d_h:(i + 1) * d_h] @ nv["o_latent"][i]) < 1e-12
    return nv


def test_absorbed_equals_naive_tiny():
    check_absorbed_equals_naive_full_recipe()


def test_absorbed_equals_naive_v2_shape():
    cfg = small(CONFIGS["v2_b64_l8192"], "v2s", 1, 130)
    wl = generate(cfg)
    rows = O.to_f64(O.gather_rows(wl.cache, wl.block_table[0], 130, 64), True)
    args = (rows[:, :512], rows[:, 512:], O.to_f64(wl.q_nope[0], True), O.to_f64(wl.q_pe[0], True),
            129, O.to_f64(wl.w_uk, True), O.to_f64(wl.w_uv, True), O.softmax_scale(128, 64), 1e4)
    nv, ab = O.naive_decode_seq(*args), O.absorbed_decode_seq(*args)
    for key in ("o", "o_latent", "lse", "q_abs"):
        assert rel(nv[key], ab[key]) < 1e-12, key


def test_position_shift_invariance():
    # encoding every key at j + delta and the query at p + delta leaves o unchanged
    a = check_absorbed_equals_naive_full_recipe(delta=0)
    b = check_absorbed_equals_naive_full_recipe(delta=100000)
    for key in ("o", "o_latent", "lse"):
        assert rel(b[key], a[key]) < 1e-10, key


# ---------------------------------------------------------------------------
# merging subsets
# ---------------------------------------------------------------------------
def check_lse_merge_partition():
    k = rand_case(n_h=3, L=40, seed=3)
    full = O.naive_decode_seq(**k, pos=39, scale=0.3, rope_base=1e4)
    r = np.random.default_rng(5)
    for cuts in ([40], [1, 39], [13, 13, 14], list(r.multinomial(40 - 6, [1 / 6] * 6) + 1)):
        bounds = np.cumsum([0] + list(cuts))
        parts = [O.naive_decode_seq(k["c"][a:b], k["k_rope"][a:b], k["q_nope"], k["q_pe"], 39,
                                    k["w_uk"], k["w_uv"], 0.3, 1e4)
                 for a, b in zip(bounds[:-1], bounds[1:])]
        ol, lse = O.lse_merge([p["o_latent"] for p in parts], [p["lse"] for p in parts])
        assert rel(ol, full["o_latent"]) < 1e-12
        assert np.max(np.abs(lse - full["lse"])) < 1e-12


def test_lse_merge_partition():
    check_lse_merge_partition()


# ---------------------------------------------------------------------------
# paging
# ---------------------------------------------------------------------------
def test_gather_matches_generator_order():
    cfg = small(CONFIGS["v2_varlen_b128"], "vs", 5, (1, 300))
    wl = generate(cfg)
    assert cfg.permute_pages
    for b in range(cfg.batch):
        L = int(wl.seq_lens[b])
        got = O.gather_rows(wl.cache, wl.block_table[b], L, 64)
        assert np.array_equal(got, sequence_rows(cfg, b, L))


def test_permuted_vs_contiguous_and_poison():
    base = small(CONFIGS["v2_varlen_b128"], "vs", 3, (1, 200))
    contiguous = generate(small(base, "vs", 3, (1, 200), permute_pages=False))
    permuted = generate(base, pad_value=float("nan"))
    assert np.isnan(O.to_f64(permuted.cache, True)).any()   # poison present in unused slots
    a = O.decode_workload(contiguous, heads=range(0, 128, 37))
    b = O.decode_workload(permuted, heads=range(0, 128, 37))
    for key in a:
        assert np.array_equal(a[key], b[key]), key


# ---------------------------------------------------------------------------
# planted mistakes: every pin above must catch at least the mistakes aimed at it
# ---------------------------------------------------------------------------
def _wrong_sign_rope(x, pos, base):
    x = np.asarray(x, np.float64)
    ang = np.asarray(pos, np.float64)[..., None] * O.rope_theta(x.shape[-1], base)
    y = np.empty_like(x * np.ones(ang.shape[:-1] + (1,)))
    y[..., 0::2] = x[..., 0::2] * np.cos(ang) + x[..., 1::2] * np.sin(ang)
    y[..., 1::2] = -x[..., 0::2] * np.sin(ang) + x[..., 1::2] * np.cos(ang)
    return y


def _half_split_theta(d, base):
    return base ** (-np.arange(d // 2, dtype=np.float64) / d)


def _naive_without_rope_term(c, k_rope, *a, **kw):
    return _ORIG_NAIVE(c, np.zeros_like(np.asarray(k_rope, np.float64)), *a, **kw)


def _naive_wrong_scale(c, k_rope, q_nope, q_pe, pos, w_uk, w_uv, scale, rope_base, **kw):
    return _ORIG_NAIVE(c, k_rope, q_nope, q_pe, pos, w_uk, w_uv, scale * np.sqrt(1.5), rope_base, **kw)


_ORIG_NAIVE = O.naive_decode_seq


def _head_rows_interleaved(w, i, d_head):
    n_h = w.shape[0] // d_head
    return w[i::n_h]


def _lse_merge_unweighted(o_parts, lse_parts):
    return np.mean(o_parts, axis=0), np.max(lse_parts, axis=0)


# ---------------------------------------------------------------------------
# multi-token queries (several new tokens of a sequence decoded at once)
# ---------------------------------------------------------------------------
def _multi_case(T, lens=(37, 5)):
    from synth import query_multi
    cfg = small(TINY, "multi", len(lens))
    wl = generate(cfg, lens=np.array(lens, np.int32))
    qs = [query_multi(cfg, b, T) for b in range(cfg.batch)]
    return wl, np.stack([q[0] for q in qs]), np.stack([q[1] for q in qs])


def check_multi_single_token():
    """T = 1 is the single-query path at position L - 1."""
    wl, qn, qp = _multi_case(1)
    m = O.multi_decode_workload(wl, qn, qp)
    wl.q_nope, wl.q_pe = qn[:, 0], qp[:, 0]
    wl.positions = wl.seq_lens - 1
    ref = O.decode_workload(wl)
    for k in ("o", "o_latent", "lse", "q_abs"):
        np.testing.assert_allclose(m[k][:, 0], ref[k], rtol=0, atol=0)


def check_multi_causal():
    """Token t never sees cached rows after its own position."""
    T = 3
    wl, qn, qp = _multi_case(T)
    a = O.multi_decode_workload(wl, qn, qp)
    L = int(wl.seq_lens[0])
    for j in range(L - T + 1, L):          # rows after token 0's position (positions L-2, L-1)
        page, slot = wl.block_table[0, j // 64], j % 64
        wl.cache[page, slot] = (wl.cache[page, slot] * 3.0 + 1.0).astype(wl.cache.dtype)
    b = O.multi_decode_workload(wl, qn, qp)
    np.testing.assert_allclose(b["o"][0, 0], a["o"][0, 0], rtol=0, atol=0)
    np.testing.assert_allclose(b["lse"][0, 0], a["lse"][0, 0], rtol=0, atol=0)
    assert not np.allclose(b["o"][0, T - 1], a["o"][0, T - 1])


def check_multi_last_token():
    """The newest token attends to every cached row, like a single query."""
    T = 4
    wl, qn, qp = _multi_case(T)
    m = O.multi_decode_workload(wl, qn, qp)
    wl.q_nope, wl.q_pe = qn[:, T - 1], qp[:, T - 1]
    wl.positions = wl.seq_lens - 1
    ref = O.decode_workload(wl)
    np.testing.assert_allclose(m["o"][:, T - 1], ref["o"], rtol=0, atol=0)


def test_multi_single_token():
    check_multi_single_token()


def test_multi_causal():
    check_multi_causal()


def test_multi_last_token():
    check_multi_last_token()


def _multi_not_causal(c, k_rope, q_nope, q_pe, w_uk, w_uv, scale, rope_base, heads=None):
    T = q_nope.shape[0]
    res = {k: [] for k in ("o", "o_latent", "lse", "q_abs")}
    for t in range(T):
        r = O.naive_decode_seq(c, k_rope, q_nope[t], q_pe[t], c.shape[0] - T + t, w_uk, w_uv, scale,
                               rope_base, heads=heads)
        for k in res:
            res[k].append(r[k])
    return {k: np.stack(v) for k, v in res.items()}


def _multi_wrong_position(c, k_rope, q_nope, q_pe, w_uk, w_uv, scale, rope_base, heads=None):
    T = q_nope.shape[0]
    res = {k: [] for k in ("o", "o_latent", "lse", "q_abs")}
    for t in range(T):
        p = c.shape[0] - 1
        r = O.naive_decode_seq(c[:p + 1], k_rope[:p + 1], q_nope[t], q_pe[t], p, w_uk, w_uv, scale,
                               rope_base, heads=heads)
        for k in res:
            res[k].append(r[k])
    return {k: np.stack(v) for k, v in res.items()}


@pytest.mark.parametrize("target,replacement,check", [
    ("multi_decode_seq", _multi_not_causal, check_multi_causal),
    ("multi_decode_seq", _multi_wrong_position, check_multi_causal),
])
def test_planted_multi_mistake_is_caught(monkeypatch, target, replacement, check):
    monkeypatch.setattr(O, target, replacement)
    with pytest.raises(AssertionError):
        check()


@pytest.mark.parametrize("target,replacement,check", [
    ("rope", _wrong_sign_rope, check_rope_planar),
    ("rope_theta", _half_split_theta, check_rope_pairing),
    ("naive_decode_seq", _naive_without_rope_term, check_two_token_rope_part),
    ("naive_decode_seq", _naive_wrong_scale, check_two_token_rope_part),
    ("_head_rows", _head_rows_interleaved, check_head_rows),
    ("lse_merge", _lse_merge_unweighted, check_lse_merge_partition),
])
def test_planted_mistake_is_caught(monkeypatch, target, replacement, check):
    monkeypatch.setattr(O, target, replacement)
    with pytest.raises(AssertionError):
        check()


# ---------------------------------------------------------------------------
# causal prefill with K/V materialised once: the per-token path, many tokens
# ---------------------------------------------------------------------------
def check_prefill_equals_multi():
    """causal_prefill_workload gives what the pinned per-token path gives
    (each token a single-query naive decode over its own prefix)."""
    from synth import query_multi
    for base, lens, T, heads in ((TINY, (37, 9), 9, None),
                                 (CONFIGS["v2lite_b32_l4096"], (70, 33), 33, [0, 5, 15])):
        cfg = small(base, "pfo", len(lens))
        wl = generate(cfg, lens=np.array(lens, np.int32))
        qs = [query_multi(cfg, b, T) for b in range(cfg.batch)]
        qn, qp = np.stack([q[0] for q in qs]), np.stack([q[1] for q in qs])
        a = O.causal_prefill_workload(wl, qn, qp, heads=heads)
        b = O.multi_decode_workload(wl, qn, qp, heads=heads)
        for k in ("o", "o_latent", "lse"):
            assert a[k].shape == b[k].shape, k
            assert rel(a[k], b[k]) < 1e-12, k


def check_prefill_causal():
    """Token 0 never sees the rows after its own position; the last token sees all."""
    from synth import query_multi
    T = 4
    cfg = small(TINY, "pfc", 1)
    wl = generate(cfg, lens=np.array([23], np.int32))
    qn, qp = (x[None] for x in query_multi(cfg, 0, T))
    a = O.causal_prefill_workload(wl, qn, qp)
    L = 23
    for j in range(L - T + 1, L):
        wl.cache[wl.block_table[0, j // 64], j % 64] *= np.float32(3.0)
    b = O.causal_prefill_workload(wl, qn, qp)
    assert np.array_equal(b["o"][0, 0], a["o"][0, 0]) and np.array_equal(b["lse"][0, 0], a["lse"][0, 0])
    assert not np.allclose(b["o"][0, T - 1], a["o"][0, T - 1])


def test_prefill_equals_multi():
    check_prefill_equals_multi()


def test_prefill_causal():
    check_prefill_causal()


def _prefill_excludes_self(c, k_rope, q_nope, q_pe, w_uk, w_uv, scale, rope_base, heads=None):
    # token t sees rows 0 .. p_t - 1 only (with a guard row so the first token is defined)
    L, T = c.shape[0], q_nope.shape[0]
    res = {k: [] for k in ("o", "o_latent", "lse")}
    for t in range(T):
        p = L - T + t
        r = O.naive_decode_seq(c[:max(p, 1)], k_rope[:max(p, 1)], q_nope[t], q_pe[t], p, w_uk, w_uv,
                               scale, rope_base, heads=heads)
        for k in res:
            res[k].append(r[k])
    return {k: np.stack(v) for k, v in res.items()}


def _prefill_unmasked(c, k_rope, q_nope, q_pe, w_uk, w_uv, scale, rope_base, heads=None):
    L, T = c.shape[0], q_nope.shape[0]
    res = {k: [] for k in ("o", "o_latent", "lse")}
    for t in range(T):
        r = O.naive_decode_seq(c, k_rope, q_nope[t], q_pe[t], L - T + t, w_uk, w_uv, scale, rope_base,
                               heads=heads)
        for k in res:
            res[k].append(r[k])
    return {k: np.stack(v) for k, v in res.items()}


def _prefill_position_off_by_one(c, k_rope, q_nope, q_pe, w_uk, w_uv, scale, rope_base, heads=None):
    L, T = c.shape[0], q_nope.shape[0]
    res = {k: [] for k in ("o", "o_latent", "lse")}
    for t in range(T):
        p = L - T + t
        r = O.naive_decode_seq(c[:p + 1], k_rope[:p + 1], q_nope[t], q_pe[t], p + 1, w_uk, w_uv, scale,
                               rope_base, heads=heads)
        for k in res:
            res[k].append(r[k])
    return {k: np.stack(v) for k, v in res.items()}


@pytest.mark.parametrize("replacement", [_prefill_excludes_self, _prefill_unmasked,
                                         _prefill_position_off_by_one])
def test_planted_prefill_mistake_is_caught(monkeypatch, replacement):
    monkeypatch.setattr(O, "causal_prefill_seq", replacement)
    with pytest.raises(AssertionError):
        check_prefill_equals_multi()
        check_prefill_causal()
