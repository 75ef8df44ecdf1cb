"""The C ABI: exported symbols and host-side argument checks (no GPU needed).

Every call here fails validation before any HIP call, so it runs on a CPU-only
host; misaligned "device pointers" are plain integers that are never touched.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import mla_latent_kv_16_amd as mla

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "mla.h")
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3


@pytest.fixture(scope="module")
def lib():
    return mla.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"mla_absorb_q", "mla_plan_splits", "mla_decode_splitkv", "mla_combine",
            "mla_decode_merged", "mla_append_kv", "mla_out_proj", "mla_decode_splitkv_multi",
            "mla_combine_multi", "mla_combine_out_proj", "mla_prefill_naive"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.mla_version() == 100
    for s in (0, -1, -2, -3, -4):
        assert lib.mla_status_string(s)
    assert lib.mla_status_string(7) == b"unknown status"


V2 = mla.Dims(128, 128, 512, 64)


def test_fast_path_shapes(lib):
    assert mla.fast_path(V2) == 1
    assert mla.fast_path(mla.Dims(16, 128, 512, 64)) == 1
    assert mla.fast_path(mla.Dims(4, 16, 64, 8, dtype=mla.F32)) == 0
    for h in (32, 48, 64, 192, 1024):                             # any multiple of 16
        assert mla.fast_path(mla.Dims(h, 128, 512, 64)) == 1, h
    for h in (8, 24, 100):                                        # straightforward kernels
        assert mla.fast_path(mla.Dims(h, 128, 512, 64)) == 0, h
    assert mla.fast_path(mla.Dims(128, 128, 512, 64, page_size=32)) == 0
    assert mla.fast_path(mla.Dims(4, 16, 64, 7)) == INVALID     # odd RoPE width
    assert mla.fast_path(mla.Dims(4, 16, 2048, 8)) == UNSUPPORTED
    assert mla.fast_path(mla.Dims(4, 16, 64, 8, dtype=5)) == UNSUPPORTED
    assert mla.fast_path(mla.Dims(4, 16, 64, 8, softmax_scale=float("nan"))) == INVALID
    assert mla.fast_path(mla.Dims(4, 16, 64, 8, rope_base=0.0)) == INVALID


A = 0x7f0000000000          # 16-byte aligned stand-in address (never dereferenced)
MIS = A + 8                 # misaligned


def _d(dims=V2):
    return ctypes.byref(dims.c())


def test_absorb_rejects_bad_arguments(lib):
    f = lib.mla_absorb_q
    assert f(None, 1, A, A, A, A, A, None) == INVALID
    assert f(_d(), 0, A, A, A, A, A, None) == INVALID
    assert f(_d(), 1, None, A, A, A, A, None) == INVALID
    assert f(_d(), 1, A, A, A, A, None, None) == INVALID
    assert f(_d(), 1, MIS, A, A, A, A, None) == INVALID
    assert f(_d(), 1, A, A, A + 2, A, A, None) == INVALID       # positions not 4-aligned
    assert f(_d(mla.Dims(4, 16, 4096, 8)), 1, A, A, A, A, A, None) == UNSUPPORTED


def test_decode_rejects_bad_arguments(lib):
    f = lib.mla_decode_splitkv
    good = [A, A, 10, A, 4, A, A, 3, A, A, None]
    assert f(_d(), 0, *good) == INVALID
    for i in (0, 1, 3, 5, 6, 8, 9):                # each pointer argument set to NULL
        args = list(good)
        args[i] = None
        assert f(_d(), 2, *args) == INVALID, i
    for i, bad in ((2, 0), (4, 0), (7, 0)):        # num_pages, max_pages, num_items < 1
        args = list(good)
        args[i] = bad
        assert f(_d(), 2, *args) == INVALID, i
    args = list(good)
    args[1] = MIS                                  # kv_cache misaligned
    assert f(_d(), 2, *args) == INVALID
    args = list(good)
    args[8] = A + 4                                # o_part misaligned
    assert f(_d(), 2, *args) == INVALID


def test_decode_multi_rejects_bad_arguments(lib):
    f = lib.mla_decode_splitkv_multi
    # q_abs kv_cache num_pages bt max_pages seq_lens items num_items o_part lse_part stream
    good = [A, A, 10, A, 4, A, A, 3, A, A, None]
    assert f(_d(), 0, 2, *good) == INVALID         # batch < 1
    assert f(_d(), 2, 0, *good) == INVALID         # q_len < 1
    assert f(_d(), 2, -3, *good) == INVALID
    for i in (0, 1, 3, 5, 6, 8, 9):                # each pointer argument set to NULL
        args = list(good)
        args[i] = None
        assert f(_d(), 2, 4, *args) == INVALID, i
    for i, bad in ((2, 0), (4, 0), (7, 0)):        # num_pages, max_pages, num_items < 1
        args = list(good)
        args[i] = bad
        assert f(_d(), 2, 4, *args) == INVALID, i
    for i, bad in ((0, MIS), (1, MIS), (8, A + 4), (9, A + 2)):
        args = list(good)                          # misaligned q_abs, cache, o_part, lse_part
        args[i] = bad
        assert f(_d(), 2, 4, *args) == INVALID, i
    args = list(good)
    args[7] = 2 ** 30                              # num_items * q_len * 2 beyond the grid
    assert f(_d(), 2, 4, *args) == UNSUPPORTED
    c = lib.mla_combine_multi
    assert c(_d(), 0, 2, A, A, A, A, A, None) == INVALID
    assert c(_d(), 2, 0, A, A, A, A, A, None) == INVALID
    assert c(_d(), 2, 2, None, A, A, A, A, None) == INVALID
    assert c(_d(), 2, 2, A, MIS, A, A, A, None) == INVALID
    assert c(_d(), 2, 2, A, A, A, A, A + 2, None) == INVALID   # lse misaligned
    assert c(_d(), 2 ** 20, 2 ** 10, A, A, A, A, None, None) == UNSUPPORTED


def test_decode_merged_rejects_bad_arguments(lib):
    f = lib.mla_decode_merged
    # q_abs kv_cache num_pages bt max_pages seq_lens items num_items offs o_part lse_part tickets o_lat lse stream
    good = [A, A, 10, A, 4, A, A, 3, A, A, A, A, A, None, None]
    assert f(_d(), 0, *good) == INVALID
    for i in (0, 1, 3, 5, 6, 8, 9, 10, 11, 12):    # each required pointer set to NULL
        args = list(good)
        args[i] = None
        assert f(_d(), 2, *args) == INVALID, i
    for i, bad in ((2, 0), (4, 0), (7, 0)):        # num_pages, max_pages, num_items < 1
        args = list(good)
        args[i] = bad
        assert f(_d(), 2, *args) == INVALID, i
    for i, bad in ((1, MIS), (9, A + 4), (11, A + 2), (12, A + 8), (13, A + 2)):
        args = list(good)                          # misaligned cache, o_part, tickets, o_latent, lse
        args[i] = bad
        assert f(_d(), 2, *args) == INVALID, i


def test_append_kv_rejects_bad_arguments(lib):
    f = lib.mla_append_kv
    need = lib.mla_append_kv_workspace_bytes(_d(), 5120, 64)
    assert need == 8 * 64 * 576 * 4                   # ceil(5120 / 640) K-slices
    assert lib.mla_append_kv_workspace_bytes(_d(), 0, 64) == -1
    # d_model batch h w_dkv w_kr positions rms eps cache num_pages bt max_pages ws ws_bytes stream
    good = [5120, 64, A, A, A, A, 1, 1e-6, A, 10, A, 4, A, need, None]
    for i in (2, 3, 4, 5, 8, 10, 12):              # each pointer argument set to NULL
        args = list(good)
        args[i] = None
        assert f(_d(), *args) == INVALID, i
    for i, bad in ((0, 0), (1, 0), (9, 0), (11, 0)):   # sizes < 1
        args = list(good)
        args[i] = bad
        assert f(_d(), *args) == INVALID, i
    for i, bad in ((2, MIS), (8, MIS), (12, MIS), (5, A + 2)):  # misaligned
        args = list(good)
        args[i] = bad
        assert f(_d(), *args) == INVALID, i
    args = list(good)
    args[7] = 0.0                                  # rms_norm with eps <= 0
    assert f(_d(), *args) == INVALID
    args = list(good)
    args[13] = need - 4                            # short workspace
    assert f(_d(), *args) == WORKSPACE


def test_check_paging_rejects_bad_arguments(lib):
    f = lib.mla_check_paging
    # batch min_len seq_lens num_pages block_table max_pages result stream
    good = [64, 1, A, 10, A, 4, A, None]
    for i in (2, 4, 6):                            # each pointer argument set to NULL
        args = list(good)
        args[i] = None
        assert f(_d(), *args) == INVALID, i
    for i in (0, 1, 3, 5):                         # sizes < 1
        args = list(good)
        args[i] = 0
        assert f(_d(), *args) == INVALID, i
    for i in (2, 4, 6):                            # misaligned int32 arrays
        args = list(good)
        args[i] = A + 2
        assert f(_d(), *args) == INVALID, i
    assert f(None, *good) == INVALID


def test_combine_and_out_proj_reject_bad_arguments(lib):
    assert lib.mla_combine(_d(), 0, A, A, A, A, A, None) == INVALID
    assert lib.mla_combine(_d(), 2, None, A, A, A, A, None) == INVALID
    assert lib.mla_combine(_d(), 2, A, MIS, A, A, A, None) == INVALID
    assert lib.mla_combine(_d(), 2, A, A, A, A, A + 2, None) == INVALID   # lse misaligned
    assert lib.mla_out_proj(_d(), 0, A, A, A, None) == INVALID
    assert lib.mla_out_proj(_d(), 2, A, None, A, None) == INVALID
    assert lib.mla_out_proj(_d(), 2, A, A, MIS, None) == INVALID


def test_combine_out_proj_rejects_bad_arguments(lib):
    f = lib.mla_combine_out_proj
    # offs o_part lse_part w_uv out o_latent lse stream
    good = [A, A, A, A, A, None, None, None]
    assert f(_d(), 0, 1, *good) == INVALID
    assert f(_d(), 2, 0, *good) == INVALID
    for i in range(5):                             # each required pointer set to NULL
        args = list(good)
        args[i] = None
        assert f(_d(), 2, 1, *args) == INVALID, i
    for i, bad in ((0, A + 2), (1, MIS), (2, A + 2), (3, MIS), (4, MIS), (5, MIS), (6, A + 2)):
        args = list(good)                          # misaligned
        args[i] = bad
        assert f(_d(), 2, 1, *args) == INVALID, i
    assert f(_d(), 2 ** 20, 2 ** 10, *good) == UNSUPPORTED
    # off the fast path the two kernels need o_latent between them
    assert f(_d(mla.Dims(8, 128, 512, 64)), 2, 1, *good) == UNSUPPORTED


def test_prefill_rejects_bad_arguments(lib):
    f = lib.mla_prefill_naive
    need = lib.mla_prefill_workspace_bytes(_d(), 2, 4)
    assert need == 2 * 2 * 128 * 4 * 64 * 128 * 2
    assert lib.mla_prefill_workspace_bytes(_d(), 0, 4) == -1
    assert lib.mla_prefill_workspace_bytes(_d(mla.Dims(4, 16, 64, 8, dtype=mla.F32)), 2, 4) == -1
    # q_nope q_pe w_uk w_uv cache num_pages bt max_pages seq_lens ws ws_bytes out lse stream
    good = [A, A, A, A, A, 10, A, 4, A, A, need, A, None, None]
    assert f(_d(), 0, 3, *good) == INVALID
    assert f(_d(), 2, 0, *good) == INVALID
    for i in (0, 1, 2, 3, 4, 6, 8, 9, 11):         # each required pointer set to NULL
        args = list(good)
        args[i] = None
        assert f(_d(), 2, 3, *args) == INVALID, i
    for i, bad in ((5, 0), (7, 0)):                # num_pages, max_pages < 1
        args = list(good)
        args[i] = bad
        assert f(_d(), 2, 3, *args) == INVALID, i
    for i, bad in ((0, MIS), (4, MIS), (9, MIS), (11, MIS), (6, A + 2), (12, A + 2)):
        args = list(good)                          # misaligned
        args[i] = bad
        assert f(_d(), 2, 3, *args) == INVALID, i
    args = list(good)
    args[10] = need - 2                            # short workspace
    assert f(_d(), 2, 3, *args) == WORKSPACE
    assert f(_d(mla.Dims(4, 16, 64, 8, dtype=mla.F32)), 2, 3, *good) == UNSUPPORTED
    # the materialisation grid holds 65535 sequences along y: one more is
    # refused before the workspace is looked at, and 65535 gets that far
    assert f(_d(), 65536, 3, *good) == UNSUPPORTED
    assert f(_d(), 65535, 3, *good) == WORKSPACE


def test_plan_rejects_bad_arguments(lib):
    pi32 = ctypes.POINTER(ctypes.c_int32)
    lens = np.array([5, 0, 7], dtype=np.int32)
    items = np.zeros((16, 4), np.int32)
    offs = np.zeros(4, np.int32)
    n = ctypes.c_int32(-1)
    args = (lens.ctypes.data_as(pi32), 256, 16, items.ctypes.data_as(pi32),
            offs.ctypes.data_as(pi32), ctypes.byref(n))
    assert lib.mla_plan_splits(_d(), 3, *args) == INVALID               # L_b = 0
    lens[1] = 3
    assert lib.mla_plan_splits(_d(), 3, lens.ctypes.data_as(pi32), 0, 16, items.ctypes.data_as(pi32),
                               offs.ctypes.data_as(pi32), ctypes.byref(n)) == INVALID  # no slots
    assert lib.mla_plan_splits(_d(), 0, *args) == INVALID
    assert lib.mla_plan_max_items(_d(), 3, lens.ctypes.data_as(pi32)) == 3
    lens[1] = -1
    assert lib.mla_plan_max_items(_d(), 3, lens.ctypes.data_as(pi32)) == -1


def test_record_calls_does_not_nest():
    import mla_latent_kv_16_amd as mla
    with mla.record_calls() as calls:
        assert calls == []
        with pytest.raises(RuntimeError):
            with mla.record_calls():
                pass
    # the outer block ended cleanly: a new recording starts empty
    with mla.record_calls() as again:
        assert again == []


def test_append_kv_noalloc_rejects_bad_arguments(lib):
    f = lib.mla_append_kv_noalloc
    cap = lib.mla_append_kv_noalloc_max_bytes()
    assert cap == 8 << 20
    fits = cap // (8 * 576 * 4)                    # tokens at d_model 5120
    # d_model batch h w_dkv w_kr positions rms eps cache num_pages bt max_pages stream
    good = [5120, fits, A, A, A, A, 1, 1e-6, A, 10, A, 4, None]
    for i in (2, 3, 4, 5, 8, 10):                  # each pointer argument set to NULL
        args = list(good)
        args[i] = None
        assert f(_d(), *args) == INVALID, i
    for i, bad in ((0, 0), (1, 0), (9, 0), (11, 0)):   # sizes < 1
        args = list(good)
        args[i] = bad
        assert f(_d(), *args) == INVALID, i
    for i, bad in ((2, MIS), (8, MIS), (5, A + 2)):     # misaligned
        args = list(good)
        args[i] = bad
        assert f(_d(), *args) == INVALID, i
    args = list(good)
    args[1] = fits + 1                             # more than the static buffer holds
    assert f(_d(), *args) == WORKSPACE
    args = list(good)
    args[1] = 70000                                # beyond the grid limit
    assert f(_d(), *args) == UNSUPPORTED


def test_grid_limits_are_unsupported_not_hip_errors(lib):
    """Sizes whose fast-path grid would pass 65535 workgroups along y come back
    as MLA_ERR_UNSUPPORTED from the host checks, before any launch."""
    # mla_absorb_q: 64 query rows per workgroup
    assert lib.mla_absorb_q(_d(), 65535 * 64 + 1, A, A, A, A, A, None) == UNSUPPORTED
    # mla_out_proj: 32 rows per workgroup
    assert lib.mla_out_proj(_d(), 65535 * 32 + 1, A, A, A, None) == UNSUPPORTED
    # mla_combine_out_proj: at 128 heads 32 rows per workgroup once there are
    # enough rows; rows = batch * q_len
    good = [A, A, A, A, A, None, None, None]
    assert lib.mla_combine_out_proj(_d(), 65535 * 32 + 1, 1, *good) == UNSUPPORTED
    assert lib.mla_combine_out_proj(_d(), (65535 * 32 + 2) // 2, 2, *good) == UNSUPPORTED
    # at 16 heads too
    lite = mla.Dims(16, 128, 512, 64)
    assert lib.mla_combine_out_proj(_d(lite), 65535 * 32 + 1, 1, *good) == UNSUPPORTED
    # mla_decode_merged: two workgroups per item must fit a 32-bit grid
    args = [A, A, 10, A, 4, A, A, 2 ** 30, A, A, A, A, A, None, None]
    assert lib.mla_decode_merged(_d(), 2, *args) == UNSUPPORTED
