"""mla_decode_splitkv_balanced: the two items of a pair split their joint range
at run time.

Against the oracle (the merged result is the same attention, only the split
point moves), with the counters back at zero after every call; at full size on
sampled sequences; with the reference moves and the exact-maximum pass forced
(a workgroup that takes its slices from the back starts with the ragged last
slice); and on 16 heads, where the call is the ordered decode.
"""
import numpy as np
import pytest

import mla_latent_kv_16_amd as mla
from synth import CONFIGS, generate, small

from gpu_util import assert_close, assert_lse, compare_with_oracle, dims_of, run, say, upload

pytestmark = pytest.mark.gpu

V2 = CONFIGS["v2_b64_l8192"]
LITE = CONFIGS["v2lite_b32_l4096"]

# single token, one page, a pair just long enough to balance (15 pages = 29
# slices), pairs of ~8-page items, an odd item count, a pair too short to
# balance (11 pages), ragged last slices
LENS = [1, 64, 900, 3000, 8205, 2000, 641]


def _pairs(items, offs):
    """(front, back) item pairs and the number of slices of their joint range."""
    out = []
    for b in range(len(offs) - 1):
        for s in range(offs[b], offs[b + 1] - 1, 2):
            out.append((s, s + 1))
    return out


def test_balanced_against_oracle(gpu_lib):
    cfg = small(V2, "bal", len(LENS), permute_pages=True)
    wl = generate(cfg, lens=np.array(LENS, np.int32))
    say(f"[balanced] lens {LENS}")
    dev = upload(wl)
    for rep in range(2):   # the second call starts from the counters the first left
        out = run(wl, dev=dev, slots=64, balanced=True)
        n_pairs = len(_pairs(out["items"], out["offs"]))
        say(f"  call {rep}: {len(out['items'])} items, {n_pairs} pairs")
        assert n_pairs >= 8
        assert not out["counters"].any(), "counters not left at zero"
        compare_with_oracle(wl, out, range(len(LENS)))


def test_balanced_matches_fixed_split(gpu_lib):
    cfg = small(V2, "bal2", len(LENS), permute_pages=True)
    wl = generate(cfg, lens=np.array(LENS, np.int32))
    dev = upload(wl)
    fixed = run(wl, dev=dev, slots=64)
    bal = run(wl, dev=dev, slots=64, balanced=True)
    say("[balanced vs fixed split]")
    # a different split of the same tokens: the plan-invariance bound
    assert_close(bal["o_latent"], fixed["o_latent"], "o_latent", 3e-3, 1e-2)
    assert_close(bal["out"], fixed["out"], "out", 3e-3, 1e-2)
    assert_lse(bal["lse"], fixed["lse"], tol=1e-3)


@pytest.mark.parametrize("var", ["MLA_DECODE_MAX_JUMP", "MLA_DECODE_SAFE_JUMP"])
def test_balanced_forced_paths(gpu_lib, monkeypatch, var):
    # 0.25 moves the softmax reference in most items, or (safe jump) sends
    # nearly every workgroup through the exact-maximum pass over the slices it
    # claimed
    cfg = small(V2, "bal3", len(LENS), permute_pages=True)
    wl = generate(cfg, lens=np.array(LENS, np.int32))
    dev = upload(wl)
    monkeypatch.setenv(var, "0.25")
    say(f"[balanced, {var}=0.25]")
    mla.exact_pass_count(reset=True)
    out = run(wl, dev=dev, slots=64, balanced=True)
    n = mla.exact_pass_count(reset=True)
    say(f"  workgroups through the exact pass: {n}")
    if var == "MLA_DECODE_SAFE_JUMP":
        assert n > 0
    assert not out["counters"].any()
    compare_with_oracle(wl, out, range(len(LENS)))


@pytest.mark.parametrize("name,seqs", [("v2_b64_l8192", [0, 31, 63]), ("v2_varlen_b128", None)])
def test_balanced_full_size(gpu_lib, name, seqs):
    cfg = CONFIGS[name]
    wl = generate(cfg)
    if seqs is None:
        order = np.argsort(wl.seq_lens)
        seqs = [int(order[0]), int(order[-1]), int(order[len(order) // 2])]
    say(f"[balanced full {name}] checking sequences {seqs}")
    dev = upload(wl)
    out = run(wl, dev=dev, ordered=True, balanced=True)   # the plan the bench times
    assert not out["counters"].any()
    assert np.all(np.isfinite(out["out"])) and np.all(np.isfinite(out["lse"]))
    compare_with_oracle(wl, out, seqs)


def test_balanced_heads16_is_ordered_decode(gpu_lib):
    cfg = small(LITE, "bal16", 4, permute_pages=True)
    wl = generate(cfg, lens=np.array([1, 700, 3000, 4096], np.int32))
    dev = upload(wl)
    a = run(wl, dev=dev, slots=64, ordered=True)
    b = run(wl, dev=dev, slots=64, ordered=True, balanced=True)
    say("[balanced at 16 heads]")
    assert not b["counters"].any()
    for k in ("o_part", "lse_part", "out"):
        assert np.array_equal(a[k], b[k]), k
