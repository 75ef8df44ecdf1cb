"""mla_append_kv: the cache write of the decoded token, against the oracle.

The written rows must match cache_rows_from_hidden (the oracle's reading of
the cache-write recipe, fp64) within the bf16 tolerance, land in exactly the
slot the block table names (every other byte of the cache unchanged: integer
work, bit-exact), and repeat bit for bit.
"""
import numpy as np
import pytest

import mla_latent_kv_16_amd as mla
from synth import CONFIGS, append_recipe, bf16_bits_to_f32, block_table, f32_to_bf16_bits, small

from gpu_util import F32_REL, assert_close, dims_of, say

pytestmark = pytest.mark.gpu

V2 = CONFIGS["v2_b64_l8192"]


def _case(cfg, lens, rms_norm):
    import torch
    from oracle import cache_rows_from_hidden
    bf = cfg.dtype == "bf16"
    B = len(lens)
    lens = np.asarray(lens, np.int32)
    raw = append_recipe(cfg, B)
    if bf:
        store = lambda a: f32_to_bf16_bits(a.astype(np.float32))  # noqa: E731
        back = bf16_bits_to_f32
    else:
        store = lambda a: a.astype(np.float32)  # noqa: E731
        back = lambda a: a.astype(np.float64)   # noqa: E731
    h, w_dkv, w_kr = store(raw["h"]), store(raw["w_dkv"]), store(raw["w_kr"])
    bt, num_pages = block_table(cfg, lens)
    pos = (lens - 1).astype(np.int32)
    D = cfg.d_latent + cfg.d_rope
    # sentinel cache: random finite values everywhere
    rng = np.random.default_rng(7)
    cache0 = store(rng.standard_normal((num_pages, cfg.page_size, D)).astype(np.float32))

    def dev(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if bf and a.dtype == np.uint16:
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.cuda()

    dims = dims_of(cfg)
    outs = []
    for _ in range(2):
        cache = dev(cache0)
        mla.append_kv(dims, dev(h), dev(w_dkv), dev(w_kr), dev(pos), cache, dev(bt), rms_norm=rms_norm)
        torch.cuda.synchronize()
        c = cache.cpu()
        outs.append(c.view(torch.int16).numpy().view(np.uint16) if bf else c.numpy())
    assert np.array_equal(outs[0], outs[1]), "not deterministic"
    got = outs[0]
    ref = cache_rows_from_hidden(back(h), back(w_dkv), back(w_kr), pos, cfg.rope_base, rms_norm)
    mask = np.zeros(got.shape[:2], bool)
    rows = []
    for b in range(B):
        page, slot = bt[b, pos[b] // cfg.page_size], pos[b] % cfg.page_size
        mask[page, slot] = True
        rows.append(back(got[page, slot]))
    # paging: every other row untouched, bit for bit
    assert np.array_equal(got[~mask], cache0[~mask]), "bytes outside the written slots changed"
    return np.array(rows), ref


@pytest.mark.parametrize("lens", [[1, 64, 65, 777, 8192, 8205], list(range(1, 35))])
def test_append_v2(gpu_lib, lens):
    cfg = small(V2, "app", len(lens), permute_pages=True)
    say(f"[append V2 B={len(lens)}]")
    got, ref = _case(cfg, lens, rms_norm=True)
    assert_close(got[:, :cfg.d_latent], ref[:, :cfg.d_latent], "c^KV")
    assert_close(got[:, cfg.d_latent:], ref[:, cfg.d_latent:], "k^R")


def test_append_without_norm(gpu_lib):
    cfg = small(V2, "app_nonorm", 3, permute_pages=True)
    got, ref = _case(cfg, [5, 130, 4000], rms_norm=False)
    assert_close(got, ref, "row")


def test_append_f32_generic(gpu_lib):
    cfg = CONFIGS["tiny_f32"]
    cfg = small(cfg, "app_f32", 3)
    got, ref = _case(cfg, [1, 37, 100], rms_norm=False)
    assert_close(got, ref, "row", rel_tol=F32_REL, max_tol=10 * F32_REL)
