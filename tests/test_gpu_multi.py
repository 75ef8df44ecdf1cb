"""Multi-token decode (q_len query tokens per sequence, causal within them).

Against the oracle (token t of sequence b at position L_b - q_len + t attends
to rows 0 .. L_b - q_len + t), on sampled heads; and, on every head, against
the single-token kernel run once per token with the length cut to that
token's prefix on the same plan, which must give the same bits.  Items that
lie wholly after a token must come back as empty partials (lse -inf, o 0).
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


def run_multi(wl, dev, T, slots):
    """absorb (B*T rows) -> decode_splitkv_multi -> combine_multi -> out_proj."""
    import torch
    cfg = wl.cfg
    dims = dims_of(cfg)
    bf = cfg.dtype == "bf16"
    B, H = cfg.batch, cfg.n_heads
    qn, qp = queries(wl, T)
    pos = (wl.seq_lens[:, None].astype(np.int64) - T + np.arange(T)[None, :]).astype(np.int32)
    q_abs = mla.absorb_q(dims, to_dev(qn.reshape(B * T, H, cfg.d_head), bf),
                         to_dev(qp.reshape(B * T, H, cfg.d_rope), bf), to_dev(pos.reshape(-1), False),
                         dev["w_uk"]).view(B, T, H, dims.row)
    items, offs = mla.plan_splits(dims, wl.seq_lens, slots)
    it_d = torch.from_numpy(items).cuda()
    of_d = torch.from_numpy(offs).cuda()
    o_part, lse_part = mla.decode_splitkv_multi(dims, q_abs, dev["cache"], dev["block_table"],
                                                dev["seq_lens"], it_d)
    o_lat, lse = mla.combine_multi(dims, of_d, o_part, lse_part, B)
    out = mla.out_proj(dims, o_lat.view(B * T, H, dims.d_latent), dev["w_uv"]).view(B, T, H, -1)
    torch.cuda.synchronize()
    res = {"q_abs_dev": q_abs, "items_dev": it_d, "items": items, "offs": offs, "qn": qn, "qp": qp}
    for k, t in (("q_abs", q_abs), ("o_part", o_part), ("lse_part", lse_part),
                 ("o_latent", o_lat), ("lse", lse), ("out", out)):
        res[k] = t.float().cpu().numpy()
    return res


def check_empty_partials(wl, res, T):
    """(item, token) pairs whose range starts after the token: lse -inf, o 0;
    all others finite."""
    P = wl.cfg.page_size
    n_empty = 0
    for w, (b, _, p0, _) in enumerate(res["items"]):
        for t in range(T):
            last = int(wl.seq_lens[b]) - T + t          # the token's own position
            if p0 * P > last:
                n_empty += 1
                assert np.all(res["lse_part"][w, t] == -np.inf), (w, t)
                assert not res["o_part"][w, t].any(), (w, t)
            else:
                assert np.all(np.isfinite(res["lse_part"][w, t])), (w, t)
    return n_empty


def check_against_single_token(wl, dev, res, T):
    """Token t of the multi call == the single-token kernel on the same plan
    with seq_lens cut to L - T + t + 1 (bit for bit on the fast path)."""
    import torch
    dims = dims_of(wl.cfg)
    for t in range(T):
        lens_t = torch.from_numpy((wl.seq_lens - T + t + 1).astype(np.int32)).cuda()
        q_t = res["q_abs_dev"][:, t].contiguous()
        o1, l1 = mla.decode_splitkv(dims, q_t, dev["cache"], dev["block_table"], lens_t,
                                    res["items_dev"])
        torch.cuda.synchronize()
        assert np.array_equal(l1.cpu().numpy(), res["lse_part"][:, t]), f"token {t}: lse_part"
        assert np.array_equal(o1.cpu().numpy(), res["o_part"][:, t]), f"token {t}: o_part"


def against_oracle(wl, res, T, heads, f32=False):
    from oracle import multi_decode_workload
    ref = multi_decode_workload(wl, res["qn"], res["qp"], heads=heads)
    sel = lambda a: np.asarray(a)[:, :, heads]  # noqa: E731
    tol = dict(rel_tol=1e-5, max_tol=1e-4) if f32 else {}
    assert_close(sel(res["q_abs"]), ref["q_abs"], "q_abs", **tol)
    assert_close(sel(res["o_latent"]), ref["o_latent"], "o_latent", **tol)
    assert_close(sel(res["out"]), ref["o"], "out", **tol)
    assert_lse(sel(res["lse"]), ref["lse"], tol=1e-4 if f32 else 1e-2)


CASES = [
    # name, config, lengths, q_len, plan slots, sampled heads
    ("h128_T2", small(V2, "q128a", 6, permute_pages=True), [2, 64, 65, 129, 3000, 8205], 2, 2048,
     [0, 5, 63, 64, 100, 127]),
    ("h128_T4", small(V2, "q128b", 5, permute_pages=True), [4, 66, 130, 4097, 9000], 4, 2048,
     [1, 62, 65, 127]),
    ("h128_T3_few_items", small(V2, "q128c", 3, permute_pages=True), [700, 5000, 12], 3, 256,
     [0, 127]),
    ("h128_T8", small(V2, "q128d", 3, permute_pages=True), [8, 1000, 8200], 8, 2048, [2, 70, 127]),
    ("h16_T2", small(LITE, "q16a", 5, permute_pages=True), [2, 64, 65, 4097, 700], 2, 2048, None),
    ("h16_T5", small(LITE, "q16b", 4, permute_pages=True), [5, 69, 3333, 8000], 5, 2048, None),
    ("h64_T3", small(V2, "q64", 3, n_heads=64, permute_pages=True), [3, 130, 4097], 3, 2048, None),
    ("h48_T2", small(V2, "q48", 3, n_heads=48, permute_pages=True), [2, 65, 3000], 2, 2048, None),
    ("tiny_f32_T3", CONFIGS["tiny_f32"], None, 3, 64, None),
]


@pytest.mark.parametrize("name,cfg,lens,T,slots,heads", CASES, ids=[c[0] for c in CASES])
def test_multi_token(gpu_lib, name, cfg, lens, T, slots, heads):
    wl = generate(cfg, lens=None if lens is None else np.array(lens, np.int32))
    assert np.all(wl.seq_lens >= T)
    say(f"[multi {name}] lens {wl.seq_lens.tolist()} q_len {T}")
    dev = upload(wl)
    res = run_multi(wl, dev, T, slots)
    n_empty = check_empty_partials(wl, res, T)
    say(f"  items {len(res['items'])}, empty (item, token) partials {n_empty}")
    fast = mla.fast_path(dims_of(cfg)) == 1
    if fast:
        check_against_single_token(wl, dev, res, T)
    h = list(range(cfg.n_heads)) if heads is None else heads
    against_oracle(wl, res, T, h, f32=cfg.dtype != "bf16")


def test_multi_q_len_one_is_single_token(gpu_lib):
    """q_len = 1 through the multi entry points gives the bits of the plain calls."""
    import torch
    for cfg, lens in ((small(V2, "q1a", 3, permute_pages=True), [1, 777, 8205]),
                      (small(LITE, "q1b", 3, permute_pages=True), [65, 4000, 3])):
        wl = generate(cfg, lens=np.array(lens, np.int32))
        say(f"[multi q_len 1, {cfg.n_heads} heads]")
        dev = upload(wl)
        dims = dims_of(cfg)
        res = run_multi(wl, dev, 1, 2048)
        o1, l1 = mla.decode_splitkv(dims, res["q_abs_dev"][:, 0].contiguous(), dev["cache"],
                                    dev["block_table"], dev["seq_lens"], res["items_dev"])
        of_d = torch.from_numpy(res["offs"]).cuda()
        ol, ll = mla.combine(dims, of_d, o1, l1, cfg.batch)
        torch.cuda.synchronize()
        assert np.array_equal(o1.cpu().numpy(), res["o_part"][:, 0])
        assert np.array_equal(l1.cpu().numpy(), res["lse_part"][:, 0])
        assert np.array_equal(ol.cpu().numpy(), res["o_latent"][:, 0])
        assert np.array_equal(ll.cpu().numpy(), res["lse"][:, 0])


def test_multi_token_full_size_sampled(gpu_lib):
    """The headline batch (B 64, L 8192, 128 heads) at q_len 4, in the launch
    configuration the bench times (its plan for slots // q_len, the fused merge
    and W^UV), against the oracle on sampled sequences and heads."""
    import torch
    from oracle import multi_decode_workload
    cfg = V2
    T = 4
    wl = generate(cfg)
    B, H = cfg.batch, cfg.n_heads
    say(f"[multi full size] q_len {T}")
    dev = upload(wl)
    dims = dims_of(cfg)
    qn, qp = queries(wl, T)
    pos = (wl.seq_lens[:, None].astype(np.int64) - T + np.arange(T)[None, :]).astype(np.int32)
    q_abs = mla.absorb_q(dims, to_dev(qn.reshape(B * T, H, cfg.d_head), True),
                         to_dev(qp.reshape(B * T, H, cfg.d_rope), True), to_dev(pos.reshape(-1), False),
                         dev["w_uk"]).view(B, T, H, dims.row)
    slots = int(torch.cuda.get_device_properties(0).multi_processor_count)
    items, offs = mla.plan_splits(dims, wl.seq_lens, max(1, slots // T))
    o_part, lse_part = mla.decode_splitkv_multi(dims, q_abs, dev["cache"], dev["block_table"],
                                                dev["seq_lens"], torch.from_numpy(items).cuda())
    o_lat = torch.empty((B, T, H, cfg.d_latent), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, T, H), dtype=torch.float32, device="cuda")
    out = mla.combine_out_proj(dims, torch.from_numpy(offs).cuda(), o_part, lse_part, dev["w_uv"], B,
                               o_latent=o_lat, lse=lse)
    torch.cuda.synchronize()
    seqs, heads = [0, 37, 63], [0, 45, 127]
    ref = multi_decode_workload(wl, qn, qp, seqs=seqs, heads=heads)
    sel = lambda a: a.cpu().numpy()[seqs][:, :, heads]  # noqa: E731
    assert_close(sel(o_lat), ref["o_latent"], "o_latent")
    assert_close(sel(out), ref["o"], "out")
    assert_lse(sel(lse), ref["lse"])
