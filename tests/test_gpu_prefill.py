"""mla_prefill_naive: the q_len newest tokens through the materialised-K/V path.

Against the oracle (token t at position L - q_len + t attends to rows 0 .. its
position), on sampled heads at 128 heads and on every head at 16; including a
whole-sequence prefill (L = q_len, every row a query) and lengths that leave
ragged key tiles.  Against the absorbed multi-token decode on the same inputs
(a different order of the same arithmetic: equal within the bf16 tolerance).
"""
import numpy as np
import pytest

import mla_latent_kv_16_amd as mla
from synth import CONFIGS, generate, query_multi, small

from gpu_util import assert_close, assert_lse, dims_of, say, to_dev, upload

pytestmark = pytest.mark.gpu

V2 = CONFIGS["v2_b64_l8192"]
LITE = CONFIGS["v2lite_b32_l4096"]


def queries(wl, T):
    q = [query_multi(wl.cfg, b, T) for b in range(wl.cfg.batch)]
    return np.stack([a for a, _ in q]), np.stack([p for _, p in q])


def run_prefill(wl, dev, T):
    import torch
    qn, qp = queries(wl, T)
    dims = dims_of(wl.cfg)
    out, lse = mla.prefill_naive(dims, to_dev(qn, True), to_dev(qp, True), dev["w_uk"], dev["w_uv"],
                                 dev["cache"], dev["block_table"], dev["seq_lens"])
    torch.cuda.synchronize()
    return qn, qp, out.cpu().numpy(), lse.cpu().numpy()


CASES = [
    # name, config, lengths, q_len, sampled heads
    ("h128_whole_seq", small(V2, "pf128a", 3, permute_pages=True), [40, 41, 300], 40, [0, 1, 64, 127]),
    ("h128_long", small(V2, "pf128b", 3, permute_pages=True), [3, 2050, 8200], 3, [5, 77]),
    ("h16_T20", small(LITE, "pf16a", 3, permute_pages=True), [20, 64, 300], 20, None),
    ("h16_T1", small(LITE, "pf16b", 2, permute_pages=True), [1, 4097], 1, None),
]


@pytest.mark.parametrize("name,cfg,lens,T,heads", CASES, ids=[c[0] for c in CASES])
def test_prefill_against_oracle(gpu_lib, name, cfg, lens, T, heads):
    from oracle import multi_decode_workload
    wl = generate(cfg, lens=np.array(lens, np.int32))
    say(f"[prefill {name}] lens {lens} q_len {T}")
    dev = upload(wl)
    qn, qp, out, lse = run_prefill(wl, dev, T)
    h = list(range(cfg.n_heads)) if heads is None else heads
    ref = multi_decode_workload(wl, qn, qp, heads=h)
    assert_close(out[:, :, h], ref["o"], "out")
    assert_lse(lse[:, :, h], ref["lse"])


# The sizes the bench times: a workgroup takes 256 query tokens (eight waves of
# 32), so these fill every wave, several workgroups and a ragged last one.
# The oracle forms each head's keys and values once (causal_prefill_workload).
LARGE = [
    # name, config, lengths, q_len, sampled heads
    ("h128_T128_whole_and_long", small(V2, "pfL1", 2, permute_pages=True), [8200, 128], 128,
     [0, 77, 127]),
    ("h128_T129_ragged", small(V2, "pfL2", 1, permute_pages=True), [8300], 129, [3, 64]),
    ("h128_T256", small(V2, "pfL3", 1, permute_pages=True), [8192], 256, [10, 100]),
    ("h16_T512", small(LITE, "pfL4", 1, permute_pages=True), [4096], 512, None),
    ("h128_T2048", small(V2, "pfL5", 1, permute_pages=True), [8192], 2048, [0, 127]),
    ("h128_T300_two_workgroups", small(V2, "pfL6", 2, permute_pages=True), [300, 5000], 300, [1, 90]),
]


@pytest.mark.parametrize("name,cfg,lens,T,heads", LARGE, ids=[c[0] for c in LARGE])
def test_prefill_benchmarked_sizes(gpu_lib, name, cfg, lens, T, heads):
    from oracle import causal_prefill_workload
    wl = generate(cfg, lens=np.array(lens, np.int32))
    say(f"[prefill {name}] lens {lens} q_len {T}")
    dev = upload(wl)
    qn, qp, out, lse = run_prefill(wl, dev, T)
    h = list(range(cfg.n_heads)) if heads is None else heads
    ref = causal_prefill_workload(wl, qn, qp, heads=h)
    assert_close(out[:, :, h], ref["o"], "out")
    assert_lse(lse[:, :, h], ref["lse"])


def test_prefill_reference_moves(gpu_lib):
    """Key tiles after the first 1024 rows carry latents scaled by 5, so every
    query's score maximum grows by more than 2^8 after the first tiles and the
    kernel's per-block softmax reference must move (and rescale).  The scale
    is kept at 5: the bf16 rounding error of a score grows with its magnitude,
    and at 8 it alone takes the output to the edge of the bar."""
    from oracle import causal_prefill_workload, gather_rows, rope, softmax_scale, to_f64
    from synth import bf16_bits_to_f32, f32_to_bf16_bits
    cfg = small(V2, "pfjump", 1, permute_pages=True)
    L, T, k_big = 2100, 300, 1024
    wl = generate(cfg, lens=np.array([L], np.int32))
    for j in range(k_big, L):
        p, s = wl.block_table[0, j // 64], j % 64
        row = bf16_bits_to_f32(wl.cache[p, s])
        row[:512] *= 5.0
        wl.cache[p, s] = f32_to_bf16_bits(row)
    say("[prefill reference moves]")
    dev = upload(wl)
    qn, qp, out, lse = run_prefill(wl, dev, T)
    h = [0, 31, 64, 127]
    # precondition: for every query and sampled head the best later score beats
    # the best score of the first 32-row tile by more than 8 (log2 units)
    rows = to_f64(gather_rows(wl.cache, wl.block_table[0], L, 64), True)
    w_uk = to_f64(wl.w_uk, True)
    pos = L - T + np.arange(T)
    for i in h:
        K = np.concatenate([rows[:, :512] @ w_uk[128 * i:128 * i + 128].T, rows[:, 512:]], axis=1)
        q = np.concatenate([to_f64(qn[0, :, i], True), rope(to_f64(qp[0, :, i], True), pos, 1e4)], axis=1)
        sc = (q @ K.T) * softmax_scale(128, 64) / np.log(2.0)
        assert np.all(sc[:, k_big:].max(axis=1) - sc[:, :32].max(axis=1) > 8.0)
    ref = causal_prefill_workload(wl, qn, qp, heads=h)
    assert_close(out[:, :, h], ref["o"], "out")
    # scores 5x the usual carry 5x the bf16 rounding error of the query
    assert_lse(lse[:, :, h], ref["lse"], tol=2e-3 * float(np.abs(ref["lse"]).max()))


def test_prefill_matches_absorbed_multi_token(gpu_lib):
    """The two paths on one input: materialised K/V and the absorbed decode."""
    import torch
    cfg = small(V2, "pfcmp", 3, permute_pages=True)
    wl = generate(cfg, lens=np.array([16, 700, 5000], np.int32))
    T = 16
    say("[prefill vs absorbed multi-token]")
    dev = upload(wl)
    qn, qp, out, lse = run_prefill(wl, dev, T)
    dims = dims_of(cfg)
    B, H = cfg.batch, cfg.n_heads
    pos = (wl.seq_lens[:, None].astype(np.int64) - T + np.arange(T)[None, :]).astype(np.int32)
    q_abs = mla.absorb_q(dims, to_dev(qn.reshape(B * T, H, cfg.d_head), True),
                         to_dev(qp.reshape(B * T, H, cfg.d_rope), True), to_dev(pos.reshape(-1), False),
                         dev["w_uk"]).view(B, T, H, dims.row)
    items, offs = mla.plan_splits(dims, wl.seq_lens, 256)
    it_d, of_d = torch.from_numpy(items).cuda(), torch.from_numpy(offs).cuda()
    o_part, lse_part = mla.decode_splitkv_multi(dims, q_abs, dev["cache"], dev["block_table"],
                                                dev["seq_lens"], it_d)
    o_lat, lse2 = mla.combine_multi(dims, of_d, o_part, lse_part, B)
    out2 = mla.out_proj(dims, o_lat.view(B * T, H, -1), dev["w_uv"]).view(B, T, H, -1)
    torch.cuda.synchronize()
    assert_close(out, out2.cpu().numpy(), "out vs absorbed")
    assert_lse(lse, lse2.cpu().numpy(), "lse vs absorbed")


MAT_CASES = [
    # name, config, lengths: ends inside a tile, on a tile boundary, below one
    # tile; one sequence of the benchmarked length (256 tiles in two splits:
    # the ring's steady state and every head's start offset, wrapping around);
    # 16 heads, where each sequence's rows are split eight ways and the short
    # sequence leaves its last splits one tile or none
    ("short", V2, [300, 64, 20]),
    ("full_length", V2, [8192]),
    ("h16_splits", LITE, [4096, 700]),
]


@pytest.mark.parametrize("name,base,lens", MAT_CASES, ids=[c[0] for c in MAT_CASES])
def test_materialised_kv_rows(gpu_lib, name, base, lens):
    """White-box check of the materialisation inside mla_prefill_naive (the
    workspace contents are not part of the ABI; the layout read here is the
    kernel's [K^C | V^C], each [b][h][row][128] bf16 with max_pages * 64 rows).

    Every head and every row below L against the float64 products
    W^UK_i c_j and W^UV_i c_j rounded once to bf16 (the kernel sums in float32,
    so it may differ by a rounding step); the rows of the last 32-row tile past
    L are written (finite) and every row past that tile keeps the NaN sentinel
    the workspace was filled with, bit for bit.  The pages are permuted."""
    import torch
    from oracle import gather_rows, to_f64
    from synth import bf16_bits_to_f32, f32_to_bf16_bits
    cfg = small(base, "pfmat_" + name, len(lens), permute_pages=True)
    T = min(lens)
    wl = generate(cfg, lens=np.array(lens, np.int32))
    say(f"[prefill materialise rows {name}] lens {lens}")
    dev = upload(wl)
    dims = dims_of(cfg)
    B, H = cfg.batch, cfg.n_heads
    max_pages = wl.block_table.shape[1]
    max_rows = max_pages * 64
    need = gpu_lib.mla_prefill_workspace_bytes(__import__("ctypes").byref(dims.c()), B, max_pages)
    assert need == 2 * B * H * max_rows * 128 * 2
    sentinel = 0x7FC1  # a bf16 NaN
    ws = torch.full((need // 2,), sentinel, dtype=torch.int16, device="cuda")
    qn, qp = queries(wl, T)
    mla.prefill_naive(dims, to_dev(qn, True), to_dev(qp, True), dev["w_uk"], dev["w_uv"], dev["cache"],
                      dev["block_table"], dev["seq_lens"], workspace=ws)
    torch.cuda.synchronize()
    got = ws.cpu().numpy().view(np.uint16).reshape(2, B, H, max_rows, 128)
    w = {"k": to_f64(wl.w_uk, True), "v": to_f64(wl.w_uv, True)}
    hc = min(16, H)  # heads per reference block (bounds the float64 temporaries)
    for b, L in enumerate(lens):
        c = to_f64(gather_rows(wl.cache, wl.block_table[b], L, 64), True)[:, :512]
        end = 32 * ((L + 31) // 32)
        for m, name_m in enumerate(("k", "v")):
            for h0 in range(0, H, hc):
                wh = w[name_m][128 * h0:128 * (h0 + hc)]
                ref = (c @ wh.T).reshape(L, hc, 128).transpose(1, 0, 2)  # [hc, L, 128]
                mag = (np.abs(c) @ np.abs(wh).T).reshape(L, hc, 128).transpose(1, 0, 2)
                ref_bf = bf16_bits_to_f32(f32_to_bf16_bits(ref.astype(np.float32))).astype(np.float64)
                g = bf16_bits_to_f32(got[m, b, h0:h0 + hc, :L]).astype(np.float64)
                # one bf16 rounding step at that size, plus what 512 float32
                # additions can lose where the sum cancels
                step = np.abs(ref_bf) * 2.0 ** -7 + 4e-5 * mag
                bad = np.abs(g - ref_bf) > step
                assert not bad.any(), (f"{name_m} seq {b} heads {h0}..{h0 + hc - 1}: {bad.sum()} values off by "
                                       f"more than one bf16 step; max |diff| {np.abs(g - ref_bf).max():.3e}")
            tail = bf16_bits_to_f32(got[m, b, :, L:end])
            assert np.all(np.isfinite(tail)), f"{name_m} seq {b}: rows {L}..{end} of the last tile not written"
            assert np.all(got[m, b, :, end:] == sentinel), f"{name_m} seq {b}: rows past the last tile written"
