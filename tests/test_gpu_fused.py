"""mla_combine_out_proj: the log-sum-exp merge and the W^UV product in one launch.

Against the two separate calls on the same partials: o_latent and lse must be
the same bits (the merge repeats the combine's arithmetic in its order) and
out the same bits as mla_out_proj on that o_latent; with o_latent and lse left
NULL, out must not change.  Covers 128 and 16 heads, many-split plans, more
than 64 rows (two row groups), q_len > 1 and the fp32 generic shapes, and
each workgroup size the launch picks (32, 16 or 8 rows, with a ragged last
group).
"""
import numpy as np
import pytest

import mla_latent_kv_16_amd as mla
from synth import CONFIGS, generate, small

from gpu_util import dims_of, say, upload

pytestmark = pytest.mark.gpu

V2 = CONFIGS["v2_b64_l8192"]
LITE = CONFIGS["v2lite_b32_l4096"]


def partials(wl, dev, slots, T):
    """Plan, absorb and decode; with q_len T > 1 every token reuses the query
    of the sequence (any partials serve for this comparison; the causal
    ranges still differ per token)."""
    import torch
    dims = dims_of(wl.cfg)
    B, H = wl.cfg.batch, wl.cfg.n_heads
    items, offs = mla.plan_splits(dims, wl.seq_lens, slots)
    it_d, of_d = torch.from_numpy(items).cuda(), torch.from_numpy(offs).cuda()
    q_abs = mla.absorb_q(dims, dev["q_nope"], dev["q_pe"], dev["positions"], dev["w_uk"])
    if T == 1:
        o_part, lse_part = mla.decode_splitkv(dims, q_abs, dev["cache"], dev["block_table"],
                                              dev["seq_lens"], it_d)
    else:
        q4 = q_abs[:, None].expand(B, T, H, dims.row).contiguous()
        o_part, lse_part = mla.decode_splitkv_multi(dims, q4, dev["cache"], dev["block_table"],
                                                    dev["seq_lens"], it_d)
    return dims, of_d, o_part, lse_part


@pytest.mark.parametrize("name,cfg,lens,slots,T", [
    ("h128", small(V2, "f128", 6, permute_pages=True), [1, 64, 65, 777, 5000, 8205], 256, 1),
    ("h128_many_rows", small(V2, "f128b", 70, lens=(1, 3000), permute_pages=True), None, 2048, 1),
    ("h128_T3", small(V2, "f128c", 4, permute_pages=True), [3, 100, 4097, 9000], 2048, 3),
    ("h128_rows20", small(V2, "f128d", 20, lens=(1, 2000), permute_pages=True), None, 512, 1),
    ("h128_rows12", small(V2, "f128e", 12, lens=(1, 3000), permute_pages=True), None, 512, 1),   # 8-row groups
    ("h128_rows5", small(V2, "f128f", 5, lens=(1, 9000), permute_pages=True), None, 2048, 1),    # 4-row groups
    ("h16", small(LITE, "f16", 5, permute_pages=True), [1, 100, 4096, 4097, 700], 2048, 1),
    ("h16_T2_many_rows", small(LITE, "f16b", 40, lens=(2, 2000), permute_pages=True), None, 512, 2),
    ("h16_ragged_rows", small(LITE, "f16c", 21, lens=(1, 3000), permute_pages=True), None, 512, 1),
    # 8-row groups and up to ~140 one-page items per row: several lse chunks
    ("h16_many_items", small(LITE, "f16d", 3, permute_pages=True), [5000, 9000, 100], 2048, 1),
    ("tiny_f32", CONFIGS["tiny_f32"], None, 64, 1),
    ("tiny_f32_T4", CONFIGS["tiny_f32"], None, 64, 4),
])
def test_fused_matches_separate_calls(gpu_lib, name, cfg, lens, slots, T):
    import torch
    wl = generate(cfg, lens=None if lens is None else np.array(lens, np.int32))
    say(f"[combine_out_proj {name}] B {cfg.batch} q_len {T}")
    dev = upload(wl)
    dims, offs, o_part, lse_part = partials(wl, dev, slots, T)
    B, H = cfg.batch, cfg.n_heads
    if T == 1:
        ol_ref, lse_ref = mla.combine(dims, offs, o_part, lse_part, B)
        out_ref = mla.out_proj(dims, ol_ref, dev["w_uv"])
    else:
        ol_ref, lse_ref = mla.combine_multi(dims, offs, o_part, lse_part, B)
        out_ref = mla.out_proj(dims, ol_ref.view(B * T, H, -1), dev["w_uv"]).view(B, T, H, -1)
    ol = torch.full_like(ol_ref, float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    out = mla.combine_out_proj(dims, offs, o_part, lse_part, dev["w_uv"], B, o_latent=ol, lse=lse)
    torch.cuda.synchronize()
    assert np.array_equal(ol.cpu().numpy(), ol_ref.cpu().numpy()), "o_latent differs"
    assert np.array_equal(lse.cpu().numpy(), lse_ref.cpu().numpy()), "lse differs"
    assert np.array_equal(out.cpu().numpy(), out_ref.cpu().numpy()), "out differs"
    if mla.fast_path(dims) == 1:
        out2 = mla.combine_out_proj(dims, offs, o_part, lse_part, dev["w_uv"], B)
        torch.cuda.synchronize()
        assert np.array_equal(out2.cpu().numpy(), out_ref.cpu().numpy()), "out differs without o_latent"
