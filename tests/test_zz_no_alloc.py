"""mla_append_kv_noalloc: the cache write with its partial sums in the
library's static device buffer (no workspace, nothing allocated), through the
C ABI, against mla_append_kv on the same inputs.

Both run the same kernels in the same order, so the written caches must agree
bit for bit: on two calls in a row, the second with fewer tokens than the
first (the static buffer keeps the first call's partial sums, which the
second must not read), and with a token count the buffer cannot hold refused
before anything is enqueued.
"""
import ctypes

import numpy as np
import pytest

import mla_latent_kv_16_amd as mla
from synth import CONFIGS, append_recipe, block_table, f32_to_bf16_bits, small

from gpu_util import dims_of, say, to_dev

pytestmark = pytest.mark.gpu

V2 = CONFIGS["v2_b64_l8192"]


def _case(lens, seed):
    cfg = small(V2, f"na{len(lens)}", len(lens), permute_pages=True)
    lens = np.asarray(lens, np.int32)
    raw = append_recipe(cfg, len(lens))
    store = lambda a: f32_to_bf16_bits(np.asarray(a, np.float32))  # noqa: E731
    bt, num_pages = block_table(cfg, lens)
    rng = np.random.default_rng(seed)
    cache0 = store(rng.standard_normal((num_pages, cfg.page_size, cfg.d_qk)))
    return cfg, (store(raw["h"]), store(raw["w_dkv"]), store(raw["w_kr"])), (lens - 1).astype(np.int32), \
        bt, cache0


def test_noalloc_matches_append_kv(gpu_lib):
    import torch
    lib = mla.load()
    assert lib.mla_append_kv_noalloc_max_bytes() == 8 << 20
    # first call: 200 tokens; second call: 7 tokens
    for n, seed in ((200, 1), (7, 2)):
        lens = list(np.random.default_rng(seed).integers(1, 9000, n))
        cfg, (h, wdkv, wkr), pos, bt, cache0 = _case(lens, seed)
        dims = dims_of(cfg)
        say(f"[noalloc] {n} tokens")
        dev = dict(h=to_dev(h, True), wdkv=to_dev(wdkv, True), wkr=to_dev(wkr, True),
                   pos=to_dev(pos, False), bt=to_dev(bt, False))
        ref = to_dev(cache0, True)
        got = to_dev(cache0, True)
        mla.append_kv(dims, dev["h"], dev["wdkv"], dev["wkr"], dev["pos"], ref, dev["bt"])
        # the new entry point, called through the C ABI directly
        d = dims.c()
        st = lib.mla_append_kv_noalloc(
            ctypes.byref(d), cfg.d_model, n, dev["h"].data_ptr(), dev["wdkv"].data_ptr(),
            dev["wkr"].data_ptr(), dev["pos"].data_ptr(), 1, ctypes.c_float(1e-6), got.data_ptr(),
            got.shape[0], dev["bt"].data_ptr(), bt.shape[1],
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0, st
        torch.cuda.synchronize()
        a = ref.view(torch.int16).cpu().numpy()
        b = got.view(torch.int16).cpu().numpy()
        assert np.array_equal(a, b), f"{n} tokens: caches differ"
        assert not np.array_equal(b, cache0.view(np.int16)), "nothing was written"
    # more tokens than the buffer holds: refused, nothing enqueued
    too_many = (8 << 20) // (8 * 576 * 4) + 1
    d = dims_of(small(V2, "x", 1)).c()
    x = torch.empty(16, dtype=torch.int32, device="cuda")
    st = lib.mla_append_kv_noalloc(ctypes.byref(d), 5120, too_many, x.data_ptr(), x.data_ptr(),
                                   x.data_ptr(), x.data_ptr(), 1, ctypes.c_float(1e-6), x.data_ptr(),
                                   1, x.data_ptr(), 1, None)
    assert st == -3, st
