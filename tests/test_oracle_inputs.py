"""Pins of the oracle's input side: bf16 decoding and the query projections.

Every bf16 parity test decodes its inputs through bf16_to_f64; the end-to-end
tests derive queries through query_from_hidden (no query compression) or
query_from_latent (the 1536-wide compressed query of the V2 shapes).  The pins
use values fixed by the bf16 format, torch's own bf16 -> float64 conversion,
and selection-matrix weights whose correct output is known by construction.
Each pin is shown to fail on a planted mistake.
"""
import numpy as np
import pytest

import oracle.mla_oracle as O


# ---------------------------------------------------------------------------
# bf16 decoding: the bf16 format is the top 16 bits of an IEEE binary32
# ---------------------------------------------------------------------------
FIXED_BF16 = [
    (0x3F80, 1.0), (0xC000, -2.0), (0x3F81, 1.0 + 2.0 ** -7), (0x4049, 3.140625),
    (0x0080, 2.0 ** -126),                       # smallest normal
    (0x0001, 2.0 ** -133),                       # smallest subnormal
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),    # largest finite
    (0x7F80, np.inf), (0xFF80, -np.inf), (0x0000, 0.0),
]


def check_bf16_fixed():
    bits = np.array([b for b, _ in FIXED_BF16], np.uint16)
    got = O.bf16_to_f64(bits)
    assert got.dtype == np.float64
    for (b, v), g in zip(FIXED_BF16, got):
        assert g == v, f"0x{b:04X}: {g!r} != {v!r}"
    neg0 = O.bf16_to_f64(np.array([0x8000], np.uint16))[0]
    assert neg0 == 0.0 and np.signbit(neg0)
    nans = O.bf16_to_f64(np.array([0x7FC0, 0xFFC1, 0x7F81], np.uint16))
    assert np.all(np.isnan(nans))
    # multi-dimensional arrays keep their shape
    assert O.bf16_to_f64(np.full((2, 3, 4), 0x3F80, np.uint16)).shape == (2, 3, 4)


def check_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    bits = np.random.default_rng(11).integers(0, 1 << 16, 200000).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def check_to_f64():
    bits = np.array([[0x3F80, 0xC000], [0x4049, 0x0001]], np.uint16)
    assert np.array_equal(O.to_f64(bits, True), O.bf16_to_f64(bits))
    f = np.array([1.5, -2.25, np.float32(1e-40), np.float32(3.4e38)], np.float32)
    got = O.to_f64(f, False)
    assert got.dtype == np.float64 and np.array_equal(got, f.astype(np.float64))


def test_bf16_fixed_patterns():
    check_bf16_fixed()


def test_bf16_matches_torch():
    check_bf16_matches_torch()


def test_to_f64():
    check_to_f64()


def _bf16_shift15(bits):
    u32 = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(15)
    return u32.view(np.float32).astype(np.float64)


def _bf16_byteswapped(bits):
    b = np.asarray(bits, np.uint16).byteswap()
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _bf16_low_half(bits):
    # the bits placed in the low half of a binary32
    return np.asarray(bits, np.uint16).astype(np.uint32).view(np.float32).astype(np.float64)


def _to_f64_ignores_flag(x, is_bf16):
    return np.asarray(x, dtype=np.float64)


@pytest.mark.parametrize("target,replacement,check", [
    ("bf16_to_f64", _bf16_shift15, check_bf16_fixed),
    ("bf16_to_f64", _bf16_byteswapped, check_bf16_fixed),
    ("bf16_to_f64", _bf16_low_half, check_bf16_fixed),
    ("bf16_to_f64", _bf16_shift15, check_bf16_matches_torch),
    ("to_f64", _to_f64_ignores_flag, check_to_f64),
])
@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_planted_bf16_mistake_is_caught(monkeypatch, target, replacement, check):
    monkeypatch.setattr(O, target, replacement)
    with pytest.raises(AssertionError):
        check()


# ---------------------------------------------------------------------------
# query projections, with selection matrices: row r of a weight picks one
# entry of its input, so the right output of every head is known by index
# ---------------------------------------------------------------------------
def _selection(rows: int, cols: int, pick: np.ndarray) -> np.ndarray:
    w = np.zeros((rows, cols))
    w[np.arange(rows), pick] = 1.0
    return w


N_H, D_H, D_R = 3, 4, 2


def check_query_from_hidden():
    d_model = 17
    h = 1.0 + np.arange(d_model, dtype=np.float64)          # distinct entries
    rng = np.random.default_rng(3)
    pick_q = rng.permutation(d_model)[:N_H * D_H]
    pick_r = rng.permutation(d_model)[:N_H * D_R]
    qn, qp = O.query_from_hidden(h, _selection(N_H * D_H, d_model, pick_q),
                                 _selection(N_H * D_R, d_model, pick_r), N_H)
    assert qn.shape == (N_H, D_H) and qp.shape == (N_H, D_R)
    for i in range(N_H):               # head i owns rows i*D_H .. i*D_H + D_H - 1
        for j in range(D_H):
            assert qn[i, j] == h[pick_q[i * D_H + j]]
        for j in range(D_R):
            assert qp[i, j] == h[pick_r[i * D_R + j]]
    # linearity in h (a projection, nothing else)
    w_q = rng.standard_normal((N_H * D_H, d_model))
    w_qr = rng.standard_normal((N_H * D_R, d_model))
    a, b = rng.standard_normal(d_model), rng.standard_normal(d_model)
    qa, ra = O.query_from_hidden(a, w_q, w_qr, N_H)
    qb, rb = O.query_from_hidden(b, w_q, w_qr, N_H)
    qs, rs = O.query_from_hidden(2.0 * a - b, w_q, w_qr, N_H)
    assert np.allclose(qs, 2.0 * qa - qb, rtol=0, atol=1e-12)
    assert np.allclose(rs, 2.0 * ra - rb, rtol=0, atol=1e-12)


def check_query_from_latent():
    d_model, d_cq = 11, 9                 # the compressed latent is narrower than h
    h = 1.0 + np.arange(d_model, dtype=np.float64)
    rng = np.random.default_rng(4)
    pick_d = rng.integers(0, d_model, d_cq)             # c^Q[k] = h[pick_d[k]]
    pick_u = rng.integers(0, d_cq, N_H * D_H)           # (W^UQ c^Q)[r] = c^Q[pick_u[r]]
    pick_r = rng.integers(0, d_cq, N_H * D_R)
    qn, qp = O.query_from_latent(h, _selection(d_cq, d_model, pick_d),
                                 _selection(N_H * D_H, d_cq, pick_u),
                                 _selection(N_H * D_R, d_cq, pick_r), N_H)
    assert qn.shape == (N_H, D_H) and qp.shape == (N_H, D_R)
    for i in range(N_H):
        for j in range(D_H):
            assert qn[i, j] == h[pick_d[pick_u[i * D_H + j]]]
        for j in range(D_R):
            assert qp[i, j] == h[pick_d[pick_r[i * D_R + j]]]
    # with W^DQ the identity it is the uncompressed projection by W^UQ and W^QR
    w_uq = rng.standard_normal((N_H * D_H, d_model))
    w_qr = rng.standard_normal((N_H * D_R, d_model))
    x = rng.standard_normal(d_model)
    a = O.query_from_latent(x, np.eye(d_model), w_uq, w_qr, N_H)
    b = O.query_from_hidden(x, w_uq, w_qr, N_H)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_query_from_hidden():
    check_query_from_hidden()


def test_query_from_latent():
    check_query_from_latent()


def _qh_interleaved(h_t, w_q, w_qr, n_heads):
    h_t = np.asarray(h_t, np.float64)
    qn = (np.asarray(w_q) @ h_t).reshape(-1, n_heads).T      # head i takes every n_h-th row
    qp = (np.asarray(w_qr) @ h_t).reshape(-1, n_heads).T
    return qn, qp


def _qh_swapped(h_t, w_q, w_qr, n_heads):
    h_t = np.asarray(h_t, np.float64)
    return (np.asarray(w_qr) @ h_t).reshape(n_heads, -1), (np.asarray(w_q) @ h_t).reshape(n_heads, -1)


def _ql_rope_from_hidden(h_t, w_dq, w_uq, w_qr, n_heads):
    # q^R taken from h instead of the compressed latent (square shapes make it run)
    h_t = np.asarray(h_t, np.float64)
    c_q = np.asarray(w_dq) @ h_t
    return ((np.asarray(w_uq) @ c_q).reshape(n_heads, -1),
            (np.asarray(w_qr)[:, :h_t.shape[0]] @ h_t[:w_qr.shape[1]]).reshape(n_heads, -1))


def _ql_no_down_projection(h_t, w_dq, w_uq, w_qr, n_heads):
    h_t = np.asarray(h_t, np.float64)[:np.asarray(w_uq).shape[1]]
    return (np.asarray(w_uq) @ h_t).reshape(n_heads, -1), (np.asarray(w_qr) @ h_t).reshape(n_heads, -1)


def _ql_interleaved(h_t, w_dq, w_uq, w_qr, n_heads):
    c_q = np.asarray(w_dq) @ np.asarray(h_t, np.float64)
    return ((np.asarray(w_uq) @ c_q).reshape(-1, n_heads).T,
            (np.asarray(w_qr) @ c_q).reshape(-1, n_heads).T)


@pytest.mark.parametrize("target,replacement,check", [
    ("query_from_hidden", _qh_interleaved, check_query_from_hidden),
    ("query_from_hidden", _qh_swapped, check_query_from_hidden),
    ("query_from_latent", _ql_rope_from_hidden, check_query_from_latent),
    ("query_from_latent", _ql_no_down_projection, check_query_from_latent),
    ("query_from_latent", _ql_interleaved, check_query_from_latent),
])
def test_planted_query_mistake_is_caught(monkeypatch, target, replacement, check):
    monkeypatch.setattr(O, target, replacement)
    with pytest.raises(AssertionError):
        check()
