"""The split-KV planner (host, integer): every page exactly once, balanced items."""
import ctypes

import numpy as np
import pytest

import mla_latent_kv_16_amd as mla
from synth import CONFIGS, seq_lens

V2 = mla.Dims(128, 128, 512, 64)
LITE = mla.Dims(16, 128, 512, 64)


def check_plan(lens, items, offs, page=64):
    lens = np.asarray(lens)
    B = len(lens)
    pages = (lens + page - 1) // page
    assert offs[0] == 0 and offs[-1] == len(items)
    assert np.all(np.diff(offs) >= 1)
    for b in range(B):
        its = items[offs[b]:offs[b + 1]]
        assert np.all(its[:, 0] == b)
        assert np.array_equal(its[:, 1], np.arange(len(its)))      # split index
        assert its[0, 2] == 0 and its[-1, 3] == pages[b]            # first/last page
        assert np.all(its[1:, 2] == its[:-1, 3])                    # contiguous, no overlap
        assert np.all(its[:, 3] > its[:, 2])                        # non-empty
        sizes = its[:, 3] - its[:, 2]
        assert sizes.max() - sizes.min() <= 1                       # near-equal parts


@pytest.mark.parametrize("lens", [[1], [64], [65], [32768], [1, 64, 65, 32768], [4096] * 32,
                                  [8192] * 64, [131072] * 8])
def test_plan_edges(lens):
    items, offs = mla.plan_splits(V2, lens, 256)
    check_plan(lens, items, offs)


def test_plan_headline_shapes():
    # uniform lengths that divide evenly fill the machine with equal items; at
    # 128 heads each item takes two workgroups, so 256 slots make 128 items
    items, offs = mla.plan_splits(V2, [8192] * 64, 256)
    assert len(items) == 128 and np.all(items[:, 3] - items[:, 2] == 64)
    items, offs = mla.plan_splits(V2, [131072] * 8, 256)
    assert len(items) == 128 and np.all(items[:, 3] - items[:, 2] == 128)
    items, offs = mla.plan_splits(LITE, [4096] * 32, 256)
    assert len(items) == 256 and np.all(items[:, 3] - items[:, 2] == 8)
    L = seq_lens(CONFIGS["v2_varlen_b128"])
    items, offs = mla.plan_splits(V2, L, 256)
    check_plan(L, items, offs)
    sizes = items[:, 3] - items[:, 2]
    assert sizes.max() <= 133 and len(items) >= 256


def test_plan_is_deterministic():
    L = np.random.default_rng(3).integers(1, 20000, 77)
    a = mla.plan_splits(V2, L, 256)
    b = mla.plan_splits(V2, L, 256)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_plan_capacity_error_reports_need():
    lib = mla.load()
    pi32 = ctypes.POINTER(ctypes.c_int32)
    lens = np.array([8192] * 64, np.int32)
    items = np.zeros((10, 4), np.int32)
    offs = np.zeros(65, np.int32)
    n = ctypes.c_int32(0)
    st = lib.mla_plan_splits(ctypes.byref(V2.c()), 64, lens.ctypes.data_as(pi32), 256, 10,
                             items.ctypes.data_as(pi32), offs.ctypes.data_as(pi32), ctypes.byref(n))
    assert st == -3 and n.value == 128   # two workgroups per item at 128 heads
    assert not items.any() and not offs.any()


@pytest.mark.parametrize("seed", range(5))
def test_plan_random(seed):
    r = np.random.default_rng(seed)
    L = r.integers(1, 70000, r.integers(1, 300))
    for dims in (V2, LITE):
        items, offs = mla.plan_splits(dims, L, int(r.integers(1, 600)))
        check_plan(L, items, offs)


@pytest.mark.parametrize("dims", [V2, LITE], ids=["h128", "h16"])
@pytest.mark.parametrize("lens", [[1], [65], [1, 64, 65, 32768], [4096] * 32, [8192] * 64,
                                  list(np.random.default_rng(3).integers(1, 20000, 77))])
def test_plan_ordered(dims, lens):
    """Longest-first plans: a valid cover, and an order that is a permutation
    of the items with non-increasing sizes (equal sizes in item order)."""
    items, offs, order = mla.plan_splits(dims, lens, 256, ordered=True)
    check_plan(lens, items, offs)
    assert sorted(order.tolist()) == list(range(len(items)))
    sz = (items[:, 3] - items[:, 2])[order]
    assert np.all(np.diff(sz) <= 0)
    for a, b in zip(order[:-1], order[1:]):
        if sz[list(order).index(a)] == sz[list(order).index(b)]:
            assert a < b


def test_plan_ordered_uniform_is_the_plain_plan():
    # equal lengths: longest first is the item order, and the sizes are the same
    for dims, lens in ((V2, [8192] * 64), (V2, [131072] * 8), (LITE, [4096] * 32)):
        a_items, a_offs = mla.plan_splits(dims, lens, 256)
        b_items, b_offs, order = mla.plan_splits(dims, lens, 256, ordered=True)
        assert np.array_equal(a_items, b_items) and np.array_equal(a_offs, b_offs)
        assert np.array_equal(order, np.arange(len(b_items)))


def test_plan_ordered_varlen_takes_fewer_items():
    L = seq_lens(CONFIGS["v2_varlen_b128"])
    items, _ = mla.plan_splits(V2, L, 256)
    o_items, _, _ = mla.plan_splits(V2, L, 256, ordered=True)
    assert len(o_items) < len(items)
