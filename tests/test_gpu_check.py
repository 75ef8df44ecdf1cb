"""mla_check_paging on the GPU, and the MLA_DEBUG switch of the binding.

The check's two results (number of bad values, first bad sequence) are integer
work: they must equal a plain host count over the same table exactly.  Tables
the check reads are never handed to a decode kernel with a bad entry: in the
MLA_DEBUG tests the "bad" pages lie past num_pages but inside the cache's
allocation, so even a check that missed them could not make a kernel read
outside its buffers.
"""
import numpy as np
import pytest

from synth import CONFIGS, generate, small

from gpu_util import dims_of, say, to_dev, upload

pytestmark = pytest.mark.gpu

V2 = CONFIGS["v2_b64_l8192"]


def host_count(lens, bt, page, num_pages, min_len):
    """Bad values: one per length outside [min_len, max_pages * page] (its
    entries are skipped), one per entry outside [0, num_pages) among the pages
    a good length uses; and the first sequence with any, or -1."""
    cap = bt.shape[1] * page
    bad, first = 0, -1
    for b, L in enumerate(int(x) for x in lens):
        if L < max(min_len, 1) or L > cap:
            bad += 1
            first = b if first < 0 else first
            continue
        for p in range((L + page - 1) // page):
            if not 0 <= int(bt[b, p]) < num_pages:
                bad += 1
                first = b if first < 0 else first
    return bad, first


def device_count(mla, dims, lens, bt, num_pages, min_len=1):
    import torch
    r = mla.check_paging(dims, to_dev(np.ascontiguousarray(bt, np.int32), False),
                         to_dev(np.asarray(lens, np.int32), False), num_pages, min_len)
    torch.cuda.synchronize()
    return tuple(int(v) for v in r.cpu())


def test_clean_workload_has_no_bad_values(mla):
    cfg = small(V2, "chk", 6, permute_pages=True)
    wl = generate(cfg, lens=np.array([1, 63, 64, 65, 1000, 3333], np.int32))
    say("[check clean]")
    assert device_count(mla, dims_of(cfg), wl.seq_lens, wl.block_table, wl.num_pages) == (0, -1)
    # the same table one page short: every entry naming the last page is bad
    got = device_count(mla, dims_of(cfg), wl.seq_lens, wl.block_table, wl.num_pages - 1)
    assert got == host_count(wl.seq_lens, wl.block_table, 64, wl.num_pages - 1, 1)
    assert got[0] == 1


@pytest.mark.parametrize("seed", range(6))
def test_random_tables_match_host_count(mla, seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 300))
    max_pages = int(rng.integers(1, 40))
    num_pages = int(rng.integers(1, 500))
    page = int(rng.choice([1, 16, 64]))
    cap = max_pages * page
    lens = rng.integers(-3, cap + 70, B).astype(np.int32)
    bt = rng.integers(0, num_pages, (B, max_pages)).astype(np.int32)
    flip = rng.random((B, max_pages)) < 0.02
    bt[flip] = rng.choice([-7, -1, num_pages, num_pages + 5], int(flip.sum()))
    min_len = int(rng.choice([1, 4]))
    from mla_latent_kv_16_amd import Dims
    dims = Dims(16, 128, 512, 64, page_size=page)
    say(f"[check random seed={seed} B={B} max_pages={max_pages} page={page} min_len={min_len}]")
    got = device_count(mla, dims, lens, bt, num_pages, min_len)
    assert got == host_count(lens, bt, page, num_pages, min_len)


def test_large_table_and_extreme_lengths(mla):
    rng = np.random.default_rng(11)
    B, max_pages, num_pages = 4096, 64, 100000
    lens = rng.integers(1, max_pages * 64 + 1, B).astype(np.int32)
    bt = rng.integers(0, num_pages, (B, max_pages)).astype(np.int32)
    lens[[7, 4000]] = [np.iinfo(np.int32).max, np.iinfo(np.int32).min]
    bt[4095, 0] = -1
    bt[3000, max_pages - 1] = num_pages         # used only if sequence 3000 is long enough
    say("[check large]")
    got = device_count(mla, dims_of(V2), lens, bt, num_pages)
    assert got == host_count(lens, bt, 64, num_pages, 1)
    assert got[1] == 7


def _padded(cache, extra):
    """A cache view of the first num_pages pages of an allocation with `extra`
    more, so that entries num_pages .. num_pages + extra - 1 stay in bounds."""
    import torch
    pad = torch.zeros((extra,) + tuple(cache.shape[1:]), dtype=cache.dtype, device=cache.device)
    return torch.cat([cache, pad])[:cache.shape[0]]


def test_debug_switch_raises_before_the_launch(mla, monkeypatch):
    import torch
    cfg = small(V2, "dbg", 3, permute_pages=True)
    lens = np.array([700, 65, 3], np.int32)
    wl = generate(cfg, lens=lens)
    dims = dims_of(cfg)
    dev = upload(wl)
    cache = _padded(dev["cache"], 8)
    items, offs = mla.plan_splits(dims, lens, 256)
    it_d, of_d = torch.from_numpy(items).cuda(), torch.from_numpy(offs).cuda()
    q_abs = mla.absorb_q(dims, dev["q_nope"], dev["q_pe"], dev["positions"], dev["w_uk"])
    bt = wl.block_table.copy()
    bt[1, 1] = wl.num_pages + 3                 # sequence 1 uses pages 0 and 1
    bad_bt = to_dev(bt, False)

    monkeypatch.delenv("MLA_DEBUG", raising=False)
    ref = mla.decode_splitkv(dims, q_abs, cache, dev["block_table"], dev["seq_lens"], it_d)
    torch.cuda.synchronize()
    ref = [t.cpu() for t in ref]

    monkeypatch.setenv("MLA_DEBUG", "1")
    say("[debug switch]")
    # a clean table passes the check and gives the same bits
    got = mla.decode_splitkv(dims, q_abs, cache, dev["block_table"], dev["seq_lens"], it_d)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b.cpu())
    with pytest.raises(mla.MlaError, match="first in sequence 1"):
        mla.decode_splitkv(dims, q_abs, cache, bad_bt, dev["seq_lens"], it_d)
    q2 = q_abs.unsqueeze(1).expand(-1, 2, -1, -1).contiguous()
    with pytest.raises(mla.MlaError, match="first in sequence 1"):
        mla.decode_splitkv_multi(dims, q2, cache, bad_bt, dev["seq_lens"], it_d)
    tickets = torch.zeros(2 * len(lens), dtype=torch.int32, device="cuda")  # 2 per sequence, as the ABI needs
    with pytest.raises(mla.MlaError, match="first in sequence 1"):
        mla.decode_merged(dims, q_abs, cache, bad_bt, dev["seq_lens"], it_d, of_d, tickets)
    q_nope = dev["q_nope"].unsqueeze(1).contiguous()
    q_pe = dev["q_pe"].unsqueeze(1).contiguous()
    with pytest.raises(mla.MlaError, match="first in sequence 1"):
        mla.prefill_naive(dims, q_nope, q_pe, dev["w_uk"], dev["w_uv"], cache, bad_bt,
                          dev["seq_lens"])
    # a length shorter than q_len is bad for the multi-token paths only
    short = to_dev(np.array([700, 65, 1], np.int32), False)
    with pytest.raises(mla.MlaError, match="first in sequence 2"):
        mla.decode_splitkv_multi(dims, q2, cache, dev["block_table"], short, it_d)
    torch.cuda.synchronize()
