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
