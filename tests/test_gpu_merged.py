"""mla_decode_merged: decode and log-sum-exp merge in one launch.

Against the two separate calls on the same plan (the merge repeats the
combine's arithmetic in the same order, so the results are bit-identical on
the fast path) and against the oracle; the tickets must come back zero, so a
second call on the same buffers must repeat the first.
"""
import numpy as np
import pytest

import mla_latent_kv_16_amd as mla
from synth import CONFIGS, generate, small

from gpu_util import assert_close, assert_lse, dims_of, num_slots, run, say, upload

pytestmark = pytest.mark.gpu

V2 = CONFIGS["v2_b64_l8192"]
LITE = CONFIGS["v2lite_b32_l4096"]


def merged(wl, ref, dev):
    import torch
    dims = dims_of(wl.cfg)
    B = wl.cfg.batch
    items = torch.from_numpy(ref["items"]).cuda()
    offs = torch.from_numpy(ref["offs"]).cuda()
    q_abs = torch.from_numpy(ref["q_abs"]).cuda()
    q_abs = q_abs.to(torch.bfloat16) if wl.cfg.dtype == "bf16" else q_abs
    tickets = torch.zeros(2 * B, dtype=torch.int32, device="cuda")
    outs = []
    for _ in range(2):
        o, l = mla.decode_merged(dims, q_abs, dev["cache"], dev["block_table"], dev["seq_lens"],
                                 items, offs, tickets)
        torch.cuda.synchronize()
        outs.append((o.cpu().numpy(), l.cpu().numpy(), tickets.cpu().numpy()))
    return outs


@pytest.mark.parametrize("name,cfg,lens,slots", [
    ("h128_ragged", small(V2, "m128", 6, permute_pages=True), [1, 64, 65, 777, 5000, 8205], None),
    ("h128_many", small(V2, "m128b", 2, permute_pages=True), [9000, 3000], 2048),
    ("h16_ragged", small(LITE, "m16", 5, permute_pages=True), [1, 100, 4096, 4097, 700], None),
    ("h16_many", small(LITE, "m16b", 2, permute_pages=True), [6000, 70], 2048),
    # other head counts: the fast decode and the fast merge as two launches
    ("h64_ragged", small(V2, "m64", 4, n_heads=64, permute_pages=True), [1, 65, 4097, 700], None),
    ("h32_many", small(V2, "m32", 2, n_heads=32, permute_pages=True), [6000, 70], 2048),
    ("tiny_f32", CONFIGS["tiny_f32"], None, None),
    ("h128_full_size", V2, None, None),   # the headline batch (bench.py --merged)
])
def test_merged_matches_separate_calls(gpu_lib, name, cfg, lens, slots):
    wl = generate(cfg, lens=None if lens is None else np.array(lens, np.int32))
    say(f"[merged {name}]")
    dev = upload(wl)
    ref = run(wl, dev=dev, slots=slots)
    n_split = np.diff(ref["offs"])
    say(f"  items {len(ref['items'])}, splits per sequence {n_split.tolist()}")
    outs = merged(wl, ref, dev)
    fast = mla.fast_path(dims_of(wl.cfg)) == 1
    for k, (o, l, t) in enumerate(outs):
        assert not t.any(), f"call {k}: tickets not reset"
        if fast:
            assert np.array_equal(o, ref["o_latent"]), f"call {k}: o_latent differs"
            assert np.array_equal(l, ref["lse"]), f"call {k}: lse differs"
        else:
            assert_close(o, ref["o_latent"], "o_latent", rel_tol=1e-6, max_tol=1e-5)
            assert_lse(l, ref["lse"], tol=1e-5)


def test_merged_against_oracle(gpu_lib):
    from oracle import decode_workload
    cfg = small(V2, "moracle", 3, permute_pages=True)
    wl = generate(cfg, lens=np.array([4000, 33, 9000], np.int32))
    say("[merged vs oracle]")
    dev = upload(wl)
    ref_gpu = run(wl, dev=dev, slots=3 * num_slots())
    (o, l, _), _ = merged(wl, ref_gpu, dev)
    ref = decode_workload(wl)
    assert_close(o, ref["o_latent"], "o_latent")
    assert_lse(l, ref["lse"])
