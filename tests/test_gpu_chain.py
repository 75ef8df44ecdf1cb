"""The decode step from hidden states, as the V2 and V2-Lite workloads define
their inputs, against the oracle's float64 chain from the same states.

GPU side: every cached row of every sequence is written by one mla_append_kv
call (row r is token t of sequence b: block-table row of b, position t, so
c^KV = RMSNorm(W^DKV h_t) and k^R = RoPE_t(W^KR h_t) land in their paged
slots; slots no token owns hold NaN); the query of the newest token comes from
its hidden state (V2: through the 1536-wide query latent, c^Q = W^DQ h,
q^C = W^UQ c^Q, q^R = W^QR c^Q; V2-Lite: q^C = W^Q h, q^R = W^QR h), projected
here with plain float32 torch ops on the CPU and stored as bf16; then
absorb -> decode -> merge + W^UV, the step the bench times.

Oracle side: cache_rows_from_hidden and query_from_latent / query_from_hidden
in float64 from the same bf16 inputs, then the naive path.  No intermediate is
rounded on that side, so the comparison carries every bf16 storage rounding of
the GPU chain (cache rows, query, q_abs, weights P): held to the usual bar.
"""
import numpy as np
import pytest

import mla_latent_kv_16_amd as mla
from synth import CONFIGS, bf16_bits_to_f32, block_table, chain_recipe, f32_to_bf16_bits, small

from gpu_util import assert_close, assert_lse, dims_of, num_slots, say, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    ("v2_b64_l8192", [700, 129, 1, 64]),     # 128 heads, query latent 1536
    ("v2lite_b32_l4096", [700, 65, 2]),      # 16 heads, no query compression
]


def _bf(a):
    return f32_to_bf16_bits(np.asarray(a, np.float32))


def _f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("name,lens", CASES, ids=[c[0] for c in CASES])
def test_chain_from_hidden(gpu_lib, name, lens):
    import torch
    import oracle as O

    cfg = small(CONFIGS[name], "chain", len(lens), permute_pages=True)
    lens = np.asarray(lens, np.int32)
    B, H, dc = cfg.batch, cfg.n_heads, cfg.d_latent
    say(f"[chain {name}] lens {lens.tolist()}")
    raw = chain_recipe(cfg, lens)
    w = {k: _bf(v) for k, v in raw.items() if k != "h"}          # stored weights (bf16)
    hs = [_bf(h) for h in raw["h"]]                               # stored hidden states
    bt, num_pages = block_table(cfg, lens)
    dims = dims_of(cfg)

    # ---- GPU: the cache written row by row, one call ----
    seq_of = np.concatenate([np.full(n, b) for b, n in enumerate(lens)])
    tok_of = np.concatenate([np.arange(n) for n in lens]).astype(np.int32)
    cache = torch.full((num_pages, cfg.page_size, cfg.d_qk), float("nan"), dtype=torch.bfloat16,
                       device="cuda")
    mla.append_kv(dims, to_dev(np.concatenate(hs), True), to_dev(w["w_dkv"], True),
                  to_dev(w["w_kr"], True), to_dev(tok_of, False), cache,
                  to_dev(np.ascontiguousarray(bt[seq_of]), False), rms_norm=True)

    # ---- the query of the newest token, float32 torch on the CPU ----
    def proj(name_, x):
        return torch.from_numpy(bf16_bits_to_f32(w[name_])) @ x

    qn_l, qp_l = [], []
    for b, n in enumerate(lens):
        h_last = torch.from_numpy(bf16_bits_to_f32(hs[b][n - 1]))
        src = proj("w_dq", h_last) if cfg.q_latent else h_last
        q_c = proj("w_uq" if cfg.q_latent else "w_q", src).reshape(H, cfg.d_head)
        q_r = proj("w_qr", src).reshape(H, cfg.d_rope)
        qn_l.append(_bf(q_c.numpy()))
        qp_l.append(_bf(q_r.numpy()))
    q_nope, q_pe = np.stack(qn_l), np.stack(qp_l)

    # ---- GPU: the step ----
    items, offs = mla.plan_splits(dims, lens, num_slots())
    q_abs = mla.absorb_q(dims, to_dev(q_nope, True), to_dev(q_pe, True), to_dev(lens - 1, False),
                         to_dev(w["w_uk"], True))
    o_part, lse_part = mla.decode_splitkv(dims, q_abs, cache, to_dev(bt, False), to_dev(lens, False),
                                          to_dev(items, False))
    o_lat = torch.empty((B, H, dc), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    out = mla.combine_out_proj(dims, to_dev(offs, False), o_part, lse_part, to_dev(w["w_uv"], True), B,
                               o_latent=o_lat, lse=lse)
    torch.cuda.synchronize()
    got_cache = cache.view(torch.int16).cpu().numpy().view(np.uint16)

    # ---- oracle: the same chain in float64 ----
    w64 = {k: _f64(v) for k, v in w.items()}
    scale = O.softmax_scale(cfg.d_head, cfg.d_rope)
    refs = []
    for b, n in enumerate(lens):
        h64 = _f64(hs[b])
        rows = O.cache_rows_from_hidden(h64, w64["w_dkv"], w64["w_kr"], np.arange(n), cfg.rope_base,
                                        rms_norm=True)
        written = _f64(O.gather_rows(got_cache, bt[b], int(n), cfg.page_size))
        assert_close(written, rows, f"cache rows of sequence {b}")
        if cfg.q_latent:
            qn, qp = O.query_from_latent(h64[n - 1], w64["w_dq"], w64["w_uq"], w64["w_qr"], H)
        else:
            qn, qp = O.query_from_hidden(h64[n - 1], w64["w_q"], w64["w_qr"], H)
        refs.append(O.naive_decode_seq(rows[:, :dc], rows[:, dc:], qn, qp, int(n) - 1, w64["w_uk"],
                                       w64["w_uv"], scale, cfg.rope_base))
    # slots no token owns were never written
    written_mask = np.zeros(got_cache.shape[:2], bool)
    written_mask[bt[seq_of, tok_of // cfg.page_size], tok_of % cfg.page_size] = True
    assert np.all(np.isnan(bf16_bits_to_f32(got_cache[~written_mask])))
    ref = {k: np.stack([r[k] for r in refs]) for k in ("o", "o_latent", "lse")}
    assert_close(out.cpu().numpy(), ref["o"], "out")
    assert_close(o_lat.cpu().numpy(), ref["o_latent"], "o_latent")
    assert_lse(lse.cpu().numpy(), ref["lse"])
