"""Streams and HIP graphs: every entry point enqueues on the stream it is given.

The step (absorb -> decode -> combine_out_proj) run on a side stream must give
the bits of the same step on the default stream; and the step captured in a
HIP graph must give, on every replay, the bits of the eager step on the
inputs the replay finds in its buffers (new queries are copied in between
replays, with eager work and a synchronisation in between).
"""
import numpy as np
import pytest

import mla_latent_kv_16_amd as mla
from synth import CONFIGS, generate, small

from gpu_util import dims_of, say, to_dev, upload

pytestmark = pytest.mark.gpu

V2 = CONFIGS["v2_b64_l8192"]


def _setup():
    import torch
    cfg = small(V2, "streams", 4, permute_pages=True)
    wl = generate(cfg, lens=np.array([70, 4000, 1, 9000], np.int32))
    dev = upload(wl)
    dims = dims_of(cfg)
    items, offs = mla.plan_splits(dims, wl.seq_lens, 512)
    B, H = cfg.batch, cfg.n_heads
    W = len(items)
    bufs = {
        "items": torch.from_numpy(items).cuda(), "offs": torch.from_numpy(offs).cuda(),
        "q_abs": torch.empty((B, H, dims.row), dtype=torch.bfloat16, device="cuda"),
        "o_part": torch.empty((W, H, cfg.d_latent), dtype=torch.float32, device="cuda"),
        "lse_part": torch.empty((W, H), dtype=torch.float32, device="cuda"),
        "out": torch.empty((B, H, cfg.d_head), dtype=torch.float32, device="cuda"),
    }
    return wl, dev, dims, bufs


def _step(dims, dev, b, stream=None):
    mla.absorb_q(dims, dev["q_nope"], dev["q_pe"], dev["positions"], dev["w_uk"], b["q_abs"], stream)
    mla.decode_splitkv(dims, b["q_abs"], dev["cache"], dev["block_table"], dev["seq_lens"], b["items"],
                       b["o_part"], b["lse_part"], stream)
    mla.combine_out_proj(dims, b["offs"], b["o_part"], b["lse_part"], dev["w_uv"], dev["seq_lens"].shape[0],
                         b["out"], stream=stream)


def test_side_stream_matches_default(gpu_lib):
    import torch
    say("[streams: side stream]")
    wl, dev, dims, bufs = _setup()
    _step(dims, dev, bufs)
    torch.cuda.synchronize()
    ref = bufs["out"].cpu().numpy().copy()
    bufs["out"].fill_(float("nan"))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        _step(dims, dev, bufs)          # the binding passes the current stream
    side.synchronize()
    assert np.array_equal(bufs["out"].cpu().numpy(), ref)
    bufs["out"].fill_(float("nan"))
    torch.cuda.synchronize()
    _step(dims, dev, bufs, stream=side)  # an explicit stream argument
    side.synchronize()
    assert np.array_equal(bufs["out"].cpu().numpy(), ref)


def test_graph_replays_match_eager(gpu_lib):
    import torch
    say("[streams: graph capture]")
    wl, dev, dims, bufs = _setup()
    cfg = wl.cfg
    rng = np.random.default_rng(11)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(dims, dev, bufs)  # warm-up on the capture stream's side
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(dims, dev, bufs)
    torch.cuda.synchronize()
    from synth import f32_to_bf16_bits
    for r in range(3):
        qn = rng.standard_normal((cfg.batch, cfg.n_heads, cfg.d_head), dtype=np.float32)
        dev["q_nope"].copy_(to_dev(f32_to_bf16_bits(qn), True))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = bufs["out"].cpu().numpy().copy()
        # eager step on the same inputs, then compare
        bufs["out"].fill_(float("nan"))
        _step(dims, dev, bufs)
        torch.cuda.synchronize()
        ref = bufs["out"].cpu().numpy()
        assert np.all(np.isfinite(got)), f"replay {r}: non-finite"
        assert np.array_equal(got, ref), f"replay {r} differs from the eager step"


def test_recorded_calls_replay(gpu_lib):
    """record_calls() keeps the step's library calls (arguments marshalled once);
    replaying them gives the bits of the step issued through the binding."""
    import torch
    say("[streams: recorded calls]")
    wl, dev, dims, bufs = _setup()
    _step(dims, dev, bufs)
    torch.cuda.synchronize()
    ref = bufs["out"].cpu().numpy().copy()
    with mla.record_calls() as calls:
        _step(dims, dev, bufs)   # nothing is enqueued here
    assert [name for _, _, name in calls] == ["mla_absorb_q", "mla_decode_splitkv", "mla_combine_out_proj"]
    bufs["out"].fill_(float("nan"))
    torch.cuda.synchronize()
    for _ in range(2):
        mla.replay_calls(calls)
    torch.cuda.synchronize()
    assert np.array_equal(bufs["out"].cpu().numpy(), ref)
