"""Degenerate inputs whose exact result has a closed form.

* A zero query: every score is 0, so every visible token gets weight exactly 1
  and o~ is the plain mean of the sequence's cached latents, lse = ln L.  The
  weights, the sums and the merge are then exact up to float32 rounding, so
  the check is held to 2e-6 (far tighter than the bf16 bar): a masked token
  that leaked in (or a visible one dropped) moves the mean by about 1/L.
* Identical rows: every token of a sequence holds the same cached row, so
  the weights are equal whatever the query and o~ is that row's latent.
Both at 128 and 16 heads, with lengths that end inside a page, on a page
boundary, at one token, and with many split items (partials to merge).
"""
import numpy as np
import pytest

from synth import CONFIGS, generate, small

from gpu_util import run, say

pytestmark = pytest.mark.gpu

LENS = [1, 64, 65, 777, 3000]


def _latents(wl, b):
    from oracle import gather_rows, to_f64
    rows = to_f64(gather_rows(wl.cache, wl.block_table[b], int(wl.seq_lens[b]), wl.cfg.page_size), True)
    return rows[:, :wl.cfg.d_latent]


@pytest.mark.parametrize("base,heads,slots", [("v2_b64_l8192", 128, 8), ("v2_b64_l8192", 128, 4096),
                                              ("v2lite_b32_l4096", 16, 8)])
def test_zero_query_gives_the_mean(mla, base, heads, slots):
    cfg = small(CONFIGS[base], "zq", len(LENS), permute_pages=True)
    wl = generate(cfg, lens=np.array(LENS, np.int32))
    wl.q_nope[...] = 0
    wl.q_pe[...] = 0
    say(f"[zero query H={heads} slots {slots}]")
    out = run(wl, slots=slots)
    say(f"  {len(out['items'])} items")
    worst = 0.0
    for b, L in enumerate(LENS):
        mean = _latents(wl, b).mean(axis=0)                        # [d_c]
        got = out["o_latent"][b].astype(np.float64)                # [H, d_c]
        err = np.abs(got - mean[None, :]).max() / np.abs(mean).max()
        worst = max(worst, err)
        assert err <= 2e-6, f"sequence {b} (L {L}): o~ differs from the mean by {err:.2e}"
        lse_err = np.abs(out["lse"][b].astype(np.float64) - np.log(L)).max()
        assert lse_err <= 2e-6 * max(1.0, np.log(L)), f"sequence {b}: lse off by {lse_err:.2e}"
    say(f"  worst relative difference from the mean: {worst:.2e}")


@pytest.mark.parametrize("base,heads", [("v2_b64_l8192", 128), ("v2lite_b32_l4096", 16)])
def test_identical_rows_give_that_row(mla, base, heads):
    cfg = small(CONFIGS[base], "same", len(LENS), permute_pages=True)
    wl = generate(cfg, lens=np.array(LENS, np.int32))
    for b, L in enumerate(LENS):
        p0 = wl.block_table[b, 0]
        row = wl.cache[p0, 0].copy()
        for j in range(L):
            wl.cache[wl.block_table[b, j // 64], j % 64] = row
    say(f"[identical rows H={heads}]")
    out = run(wl, slots=4096)
    for b, L in enumerate(LENS):
        c = _latents(wl, b)[0]
        got = out["o_latent"][b].astype(np.float64)
        err = np.abs(got - c[None, :]).max() / np.abs(c).max()
        assert err <= 2e-6, f"sequence {b} (L {L}): o~ differs from the row by {err:.2e}"


@pytest.mark.parametrize("base,heads,T", [("v2_b64_l8192", 128, 4), ("v2lite_b32_l4096", 16, 5)])
def test_zero_query_multi_token_gives_prefix_means(mla, base, heads, T):
    """q_len tokens with zero queries: token t sees rows 0 .. L - T + t, each
    with weight 1, so its o~ is the mean of that prefix (causal mask exact)."""
    import torch

    from gpu_util import dims_of, to_dev, upload
    lens = [T, 65, 777, 3000]
    cfg = small(CONFIGS[base], "zqm", len(lens), permute_pages=True)
    wl = generate(cfg, lens=np.array(lens, np.int32))
    dims = dims_of(cfg)
    B, H = cfg.batch, cfg.n_heads
    dev = upload(wl)
    q_abs = torch.zeros((B, T, H, dims.row), dtype=torch.bfloat16, device="cuda")
    items, offs = mla.plan_splits(dims, wl.seq_lens, 4096)
    o_part, lse_part = mla.decode_splitkv_multi(dims, q_abs, dev["cache"], dev["block_table"],
                                                dev["seq_lens"], torch.from_numpy(items).cuda())
    o_lat, lse = mla.combine_multi(dims, torch.from_numpy(offs).cuda(), o_part, lse_part, B)
    torch.cuda.synchronize()
    o_lat, lse = o_lat.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    say(f"[zero query, q_len {T}, H={heads}] {len(items)} items")
    for b, L in enumerate(lens):
        c = _latents(wl, b)
        for t in range(T):
            n = L - T + t + 1
            mean = c[:n].mean(axis=0)
            err = np.abs(o_lat[b, t] - mean[None, :]).max() / np.abs(mean).max()
            assert err <= 2e-6, f"sequence {b} token {t} (prefix {n}): {err:.2e}"
            assert np.abs(lse[b, t] - np.log(n)).max() <= 2e-6 * max(1.0, np.log(n))
