"""libmla on the GPU against the fp64 oracle, through the C ABI.

Tolerances: bf16 inputs with float32 accumulation must match within a relative
L2 error of 5e-3 and a max-abs error of 2e-2 * max|ref| (q_abs, o_latent, out);
lse within 1e-2 absolute.  float32 storage (tiny workload): 1e-5.
"""
import numpy as np
import pytest

from synth import CONFIGS, generate, small

from gpu_util import assert_close, assert_lse, compare_with_oracle, dims_of, run, say, upload

pytestmark = pytest.mark.gpu

V2 = CONFIGS["v2_b64_l8192"]
LITE = CONFIGS["v2lite_b32_l4096"]


def test_tiny_f32(mla):
    cfg = CONFIGS["tiny_f32"]
    say(f"[tiny_f32] {cfg}")
    wl = generate(cfg)
    out = run(wl)
    compare_with_oracle(wl, out, [0], f32=True)


# ragged lengths: single token, one page, page + 1, several 32-token slices with
# a tail, many pages with a tail
RAGGED = [1, 64, 65, 777, 2 * 4096 + 13]


def test_v2_heads128_ragged(mla):
    cfg = small(V2, "v2_ragged", len(RAGGED), permute_pages=True)
    say(f"[v2 ragged] lens {RAGGED}")
    wl = generate(cfg, lens=np.array(RAGGED, np.int32))
    out = run(wl)
    compare_with_oracle(wl, out, range(len(RAGGED)))


def test_v2_heads128_many_splits(mla):
    # a plan with many small items per sequence (several work items per page run)
    cfg = small(V2, "v2_split", 3, permute_pages=True)
    lens = np.array([3000, 1, 4500], np.int32)
    wl = generate(cfg, lens=lens)
    say(f"[v2 many splits] lens {lens.tolist()}")
    out = run(wl, slots=4096)
    assert len(out["items"]) > 3
    compare_with_oracle(wl, out, range(3))


def test_lite_heads16_ragged(mla):
    cfg = small(LITE, "lite_ragged", 4, permute_pages=True)
    lens = np.array([1, 100, 2000, 4096], np.int32)
    say(f"[lite ragged] lens {lens.tolist()}")
    wl = generate(cfg, lens=lens)
    out = run(wl)
    compare_with_oracle(wl, out, range(4))


def test_generic_heads8(mla):
    # 8 heads (not a multiple of 16) is outside the fast path: the
    # straightforward kernels serve it, at the V2 row shape
    cfg = small(V2, "v2_h8", 2, n_heads=8)
    lens = np.array([70, 300], np.int32)
    say("[generic heads 8]")
    wl = generate(cfg, lens=lens)
    assert mla.fast_path(dims_of(cfg)) == 0
    out = run(wl)
    compare_with_oracle(wl, out, range(2))


# Other head counts on the fast path: ceil(H / 64) workgroups of 64 heads per
# item, the last one partly on zero queries when 64 does not divide H (32, 48:
# one group with 2 or 3 of its 4 head blocks real; 80: a second group with
# one); ragged lengths, permuted pages and many-split plans, every head
# against the oracle.
OTHER_HEADS = [
    # heads, lengths, plan slots
    (32, [1, 65, 700, 4100], 2048),
    (48, [64, 129, 3000], 256),
    (64, [1, 64, 65, 777, 5000], 2048),
    (80, [2, 300, 4097], 2048),
    (192, [33, 2050, 700], 256),
]


@pytest.mark.parametrize("heads,lens,slots", OTHER_HEADS, ids=[f"h{h}" for h, _, _ in OTHER_HEADS])
def test_fast_path_other_head_counts(mla, heads, lens, slots):
    cfg = small(V2, f"v2_h{heads}", len(lens), n_heads=heads, permute_pages=True)
    say(f"[fast path heads {heads}] lens {lens}")
    wl = generate(cfg, lens=np.array(lens, np.int32))
    assert mla.fast_path(dims_of(cfg)) == 1
    out = run(wl, slots=slots)
    compare_with_oracle(wl, out, range(len(lens)))


def _scale_latents(wl, first, factor):
    """Multiply the latent part of every cached row from token `first` on."""
    from synth import bf16_bits_to_f32, f32_to_bf16_bits
    for b in range(wl.cfg.batch):
        for j in range(first, int(wl.seq_lens[b])):
            p, s = wl.block_table[b, j // 64], j % 64
            row = bf16_bits_to_f32(wl.cache[p, s])
            row[:512] *= factor
            wl.cache[p, s] = f32_to_bf16_bits(row)


@pytest.mark.parametrize("heads", [128, 16])
def test_score_jump_moves_reference(mla, heads):
    # The first 32-token slice has small scores; later latents are scaled up so
    # a head's maximum jumps far beyond the first slice's (several moves of
    # the softmax reference, each rescaling the accumulators).  The jump of
    # any one slice stays far below 2^64, so no item is redone.  Scores are
    # ~8x larger than usual, and so is the absolute error that bf16 rounding
    # of q_abs puts on them: lse is held to 2e-3 of its magnitude instead of
    # 1e-2 absolute.
    cfg = small(V2, "v2_jump", 2, n_heads=heads, permute_pages=True)
    lens = np.array([700, 200], np.int32)
    wl = generate(cfg, lens=lens)
    _scale_latents(wl, 32, 8.0)
    say(f"[score jump H={heads}]")
    mla.exact_pass_count(reset=True)
    out = run(wl)
    assert mla.exact_pass_count() == 0
    from oracle import decode_workload
    ref = decode_workload(wl)
    assert_close(out["o_latent"], ref["o_latent"], "o_latent")
    assert_close(out["out"], ref["o"], "out")
    assert_lse(out["lse"], ref["lse"], tol=2e-3 * float(np.abs(ref["lse"]).max()))


@pytest.mark.parametrize("heads", [128, 16])
def test_reference_moves_forced(mla, monkeypatch, heads):
    # A 0.25 (log2) threshold moves the reference on ordinary inputs in most
    # work items (every time a slice's maximum passes it by that much).
    cfg = small(V2, "v2_moves", len(RAGGED), n_heads=heads, permute_pages=True)
    wl = generate(cfg, lens=np.array(RAGGED, np.int32))
    base = run(wl)
    monkeypatch.setenv("MLA_DECODE_MAX_JUMP", "0.25")
    say(f"[forced reference moves H={heads}]")
    forced = run(wl, items=base["items"], offs=base["offs"])
    compare_with_oracle(wl, forced, range(len(RAGGED)))
    assert_close(forced["o_latent"], base["o_latent"], "forced vs default", 3e-3, 1e-2)


def test_exact_pass_forced(mla, monkeypatch):
    # A 0.25 (log2) bound on the weights sends nearly every work item of the
    # 128-head kernel through the exact-maximum pass on ordinary inputs.
    cfg = small(V2, "v2_exact", len(RAGGED), permute_pages=True)
    wl = generate(cfg, lens=np.array(RAGGED, np.int32))
    base = run(wl)
    monkeypatch.setenv("MLA_DECODE_SAFE_JUMP", "0.25")
    say("[forced exact-max pass]")
    mla.exact_pass_count(reset=True)
    forced = run(wl, items=base["items"], offs=base["offs"])
    n = mla.exact_pass_count(reset=True)
    say(f"  items redone: {n} of {2 * len(base['items'])} workgroups")
    assert n > 0
    compare_with_oracle(wl, forced, range(len(RAGGED)))
    assert_close(forced["o_latent"], base["o_latent"], "forced vs default", 3e-3, 1e-2)


@pytest.mark.parametrize("name,seqs,heads", [
    ("v2lite_b32_l4096", [0, 17, 31], None),
    ("v2_b64_l8192", [0, 63], None),
    ("v2_varlen_b128", None, None),
    ("v2_b8_l131072", [5], list(range(0, 128, 16))),
])
def test_full_size_sampled(mla, name, seqs, heads):
    """Full-size workloads in the launch configuration the bench times; the
    oracle checks sampled sequences (and, at 128K, sampled heads)."""
    cfg = CONFIGS[name]
    say(f"[full {name}] generating")
    wl = generate(cfg)
    if seqs is None:  # shortest, longest and one in between
        order = np.argsort(wl.seq_lens)
        seqs = [int(order[0]), int(order[-1]), int(order[len(order) // 2])]
    say(f"[full {name}] running; checking sequences {seqs}")
    dev = upload(wl)
    out = run(wl, dev=dev, ordered=True)   # the bench's plan and dispatch
    assert np.all(np.isfinite(out["out"])) and np.all(np.isfinite(out["lse"]))
    compare_with_oracle(wl, out, seqs, heads=heads)
    # the step the bench times merges and projects in one launch: on the same
    # partials it must give the bits of mla_combine + mla_out_proj above
    import torch
    fused = mla.combine_out_proj(dims_of(cfg), torch.from_numpy(out["offs"]).cuda(),
                                 torch.from_numpy(out["o_part"]).cuda(), torch.from_numpy(out["lse_part"]).cuda(),
                                 dev["w_uv"], cfg.batch)
    torch.cuda.synchronize()
    assert np.array_equal(fused.cpu().numpy(), out["out"]), "combine_out_proj differs from combine + out_proj"
