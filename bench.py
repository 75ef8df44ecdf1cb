"""Benchmark of one MLA decode step on one MI355X.

A step is one pass of the whole path over a batch for one attention layer:
mla_absorb_q -> mla_decode_splitkv -> mla_combine_out_proj (the log-sum-exp
merge and the W^UV product in one launch), on synthetic inputs already resident
in HBM; the split plan is made once per batch shape, before timing.
--unfused runs mla_combine and mla_out_proj as two launches instead; --merged
fuses the merge into the decode (mla_decode_merged) and runs mla_out_proj after
it.  With --q-len T every sequence decodes its T newest tokens at once (causal
among them): absorb on B*T rows, mla_decode_splitkv_multi, then the merge and
W^UV on B*T rows.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--heads H] [--merged | --unfused]
                    [--q-len T] [--slots N] [--back-to-back] [--prefill T [--prefill-batch B]]
                    [--settle-ms MS] [--graph] [--fenced-events] [--no-cpu-baseline]
                    [--copy-probe]

Prints ONE JSON line on stdout; progress goes to stderr.

Timing.  Before every step a 512 MiB buffer is read (a reduction, untimed), so
the 256 MB last-level cache holds other data and the step reads its cache rows
from HBM; each step is timed between two HIP events recorded at its
boundaries, and ms_per_step is their mean (the JSON line also gives p10,
median and p90).  (The flush reads rather than
writes so that the step does not also pay for writing back dirty lines.)  A
second pass with an event between every two kernels gives the per-kernel
breakdown (each event adds a few microseconds, so it sums to more than the
step); a third pass times the decode launch alone in the same way, for the
roofline of the decode kernel.

--back-to-back instead runs the steps back to back, as the layers of a model
do, cycling over the inputs of several layers (latent caches, weights and
queries of the same shapes in different memory; enough layers that together
they hold more than twice the last-level cache) with no flush, and times all K
steps (and, in the third pass, K decode launches) between two events: the
sustained rate, in which the chip runs at the clock its power limit allows
under continuous decode.  All events are recorded on the stream the kernels
run on.  They are HIP events created with hipEventDisableSystemFence (timing
only: recording one does not write back and invalidate the caches);
--fenced-events uses torch.cuda.Event instead.

Before the warm-up the flush kernel runs for --settle-ms (100 ms): straight
out of idle the first steps run up to 10% slower.  The timed passes issue the
library calls recorded once per layer after the warm-up (mla.record_calls),
so that the host's per-step cost stays below the GPU's and the kernels of a
step run back to back.  --graph replays a HIP graph of the step instead.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
TARGET_FRAC = 0.60                # decode kernel: fraction of its binding roofline aimed at
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
METRIC = "MLA decode TFLOP/s + latent-cache GB/s (% roofline), B=64 S=8192 H=128, 1 GPU"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipTimingEvent:
    """A HIP event made for timing only: created with hipEventDisableSystemFence,
    so that recording it performs no system-scope cache write-back and
    invalidate (which otherwise adds several microseconds to every bracket and
    slows the work after it).  Same interface as torch.cuda.Event for what the
    bench uses; it lives in the HIP runtime torch has loaded."""
    _lib = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if HipTimingEvent._lib is None:
            import torch  # noqa: F401  (loads the HIP runtime this must share)
            lib = ctypes.CDLL("libamdhip64.so.7")
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            HipTimingEvent._lib = lib
        self._ctypes = ctypes
        self.ev = ctypes.c_void_p()
        rc = self._lib.hipEventCreateWithFlags(ctypes.byref(self.ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream):
        rc = self._lib.hipEventRecord(self.ev, self._ctypes.c_void_p(int(stream.cuda_stream)))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end) -> float:
        ms = self._ctypes.c_float(0.0)
        rc = self._lib.hipEventElapsedTime(self._ctypes.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def __del__(self):
        if self._lib is not None and self.ev:
            self._lib.hipEventDestroy(self.ev)


def algorithmic(cfg, lens, q_len: int = 1, n_items: int = 0):
    """Algorithmic work of one step and of its kernels (q_len query tokens per
    sequence; token t of T sees L - T + t + 1 rows).

    Decode bytes: every cached row once, q_abs read, the latent output written
    once in bf16 (B T H d_c values), 4 bytes per page of block table.  The
    split partials are implementation overhead and are not counted.  A second
    figure counts the latent output at float32 with its lse (what a merged
    result written once would take at float32) for comparison.
    Step bytes: the step's own inputs and outputs (cache rows, block table,
    q^C and q^R, W^UK and W^UV, the float32 output o); the intermediates
    (q_abs, partials) are not counted.
    """
    L = lens.astype(np.int64)
    B, H, T = cfg.batch, cfg.n_heads, q_len
    D = cfg.d_latent + cfg.d_rope
    pages = int(((L + cfg.page_size - 1) // cfg.page_size).sum())
    seen = int(L.sum()) * T - B * T * (T - 1) // 2       # rows scored, over all tokens
    decode_flop = seen * H * 2 * (D + cfg.d_latent)
    dense_flop = 2 * B * T * H * cfg.d_head * cfg.d_latent * 2   # absorb + out_proj
    cache_bytes = int(L.sum()) * D * 2
    q_abs_bytes = B * T * H * D * 2
    decode_bytes = cache_bytes + q_abs_bytes + B * T * H * cfg.d_latent * 2 + 4 * pages
    decode_bytes_f32 = cache_bytes + q_abs_bytes + B * T * H * (cfg.d_latent + 1) * 4 + 4 * pages
    w_bytes = H * cfg.d_head * cfg.d_latent * 2                  # one of W^UK, W^UV
    q_in = B * T * H * (cfg.d_head + cfg.d_rope) * 2
    out_bytes = B * T * H * cfg.d_head * 4
    absorb_bytes = w_bytes + q_in + q_abs_bytes
    merge_bytes = n_items * T * H * (cfg.d_latent + 1) * 4 + w_bytes + out_bytes
    step_bytes = cache_bytes + 4 * pages + q_in + 2 * w_bytes + out_bytes
    return dict(decode_flop=decode_flop, step_flop=decode_flop + dense_flop,
                cache_bytes=cache_bytes, decode_bytes=decode_bytes, decode_bytes_f32=decode_bytes_f32,
                absorb_bytes=absorb_bytes, merge_bytes=merge_bytes, step_bytes=step_bytes, pages=pages)


def decode_source_hash() -> str:
    """sha256 (16 hex digits) of the decode kernel's sources."""
    h = hashlib.sha256()
    for f in ("decode_fast.hip", "decode_common.h"):
        h.update(open(os.path.join(ROOT, "mla_latent_kv_16_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per decode launch from the committed counter summary, if it was
    taken on the current decode kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"decode_{workload}_counters.md")
    if not os.path.exists(p):
        return None
    txt = open(p).read()
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    h = re.search(r"decode_source_sha256_16:\s*([0-9a-f]+)", txt)
    if not m or not h or h.group(1) != decode_source_hash():
        return None
    return float(m.group(1))


def cpu_baseline(wl, budget_s: float = 20.0, gpu_out=None):
    """The fp64 oracle, untuned, on a bounded sample of the same workload.
    With `gpu_out` ([B, H, d_h], the timed step's output on these inputs) the
    sampled sequences' outputs are also compared with the oracle's."""
    from oracle import decode_workload
    cfg = wl.cfg
    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = affinity
    order = list(range(cfg.batch))
    done, flop, t_total = [], 0, 0.0
    ref = []
    for b in order:
        t0 = time.perf_counter()
        r = decode_workload(wl, seqs=[b])
        t_total += time.perf_counter() - t0
        ref.append(r["o"][0])
        done.append(b)
        flop += int(wl.seq_lens[b]) * cfg.n_heads * 2 * (cfg.d_latent + cfg.d_rope + cfg.d_latent)
        if t_total >= budget_s * 0.5 or len(done) == cfg.batch:
            break
    toks = int(sum(int(wl.seq_lens[b]) for b in done))
    res = {"value": flop / t_total / 1e12, "unit": "TFLOP/s", "cores": int(threads),
           "affinity_cores": int(affinity), "blas_threads": int(threads),
           "kind": "oracle",
           "sample": f"{len(done)} of {cfg.batch} sequences ({toks} cached tokens, all "
                     f"{cfg.n_heads} heads), naive fp64 path, {t_total:.1f} s wall",
           "seq_per_s": len(done) / t_total}
    if gpu_out is not None:
        # the timed step's output against the oracle on the same sequences
        got = np.asarray(gpu_out[done], np.float64)
        want = np.stack(ref)
        res["oracle_check"] = {
            "sequences": len(done),
            "out_rel_l2": float(np.linalg.norm(got - want) / np.linalg.norm(want)),
            "out_max_abs_ratio": float(np.abs(got - want).max() / np.abs(want).max()),
            "tolerance": {"rel_l2": 5e-3, "max_abs_ratio": 2e-2}}
    return res


def time_prefill(args, cfg, wl, dims, L0, block_table, seq_lens, stream, new_events, evict, slots):
    """A T-token prefill of the first sequences (each of length >= T): the
    materialised-K/V path (mla_prefill_naive) against the absorbed path
    (absorb on B*T rows, multi-token decode, merge and W^UV on B*T rows)."""
    import torch

    import mla_latent_kv_16_amd as mla
    from synth import query_multi
    T, Bp = args.prefill, min(args.prefill_batch, cfg.batch)
    H = cfg.n_heads
    lens = wl.seq_lens[:Bp].astype(np.int64)
    assert np.all(lens >= T), "every sequence must hold the T prefill tokens"
    qs = [query_multi(cfg, b, T) for b in range(Bp)]

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).view(torch.int16).view(torch.bfloat16).cuda()
    qn, qp = dev(np.stack([a for a, _ in qs])), dev(np.stack([p for _, p in qs]))
    bt, sl = block_table[:Bp].contiguous(), seq_lens[:Bp].contiguous()
    need = mla.load().mla_prefill_workspace_bytes(__import__("ctypes").byref(dims.c()), Bp, bt.shape[1])
    ws = torch.empty(need // 2, dtype=torch.int16, device="cuda")
    out = torch.empty((Bp, T, H, cfg.d_head), dtype=torch.float32, device="cuda")
    # absorbed path buffers
    pos = (lens[:, None] - T + np.arange(T)[None, :]).reshape(-1).astype(np.int32)
    pos_d = torch.from_numpy(pos).cuda()
    items_h, offs_h = mla.plan_splits(dims, wl.seq_lens[:Bp], max(1, slots // T))
    items, offs = torch.from_numpy(items_h).cuda(), torch.from_numpy(offs_h).cuda()
    q_abs = torch.empty((Bp, T, H, dims.row), dtype=torch.bfloat16, device="cuda")
    o_part = torch.empty((len(items_h), T, H, cfg.d_latent), dtype=torch.float32, device="cuda")
    lse_part = torch.empty((len(items_h), T, H), dtype=torch.float32, device="cuda")
    out2 = torch.empty((Bp, T, H, cfg.d_head), dtype=torch.float32, device="cuda")

    def naive():
        mla.prefill_naive(dims, qn, qp, L0["w_uk"], L0["w_uv"], L0["cache"], bt, sl, out=out,
                          want_lse=False, workspace=ws, stream=stream)

    def absorbed():
        mla.absorb_q(dims, qn.view(Bp * T, H, cfg.d_head), qp.view(Bp * T, H, cfg.d_rope), pos_d,
                     L0["w_uk"], q_abs.view(Bp * T, H, dims.row), stream)
        mla.decode_splitkv_multi(dims, q_abs, L0["cache"], bt, sl, items, o_part, lse_part, stream)
        mla.combine_out_proj(dims, offs, o_part, lse_part, L0["w_uv"], Bp, out2, stream=stream)

    res = {"q_len": T, "batch": Bp, "seq_len": int(lens.max())}
    seen = int(lens.sum()) * T - Bp * T * (T - 1) // 2          # (query, key) pairs
    for name, fn in (("naive", naive), ("absorbed", absorbed)):
        for _ in range(2):
            evict()
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(max(3, min(args.steps, 10))):
            evict()
            e0, e1 = new_events(2)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = float(np.mean(ts))
        if name == "naive":
            flop = 2 * int(lens.sum()) * H * cfg.d_head * cfg.d_latent * 2 + seen * H * 2 * (dims.row - cfg.d_latent + 2 * cfg.d_head)
        else:
            flop = seen * H * 2 * (dims.row + cfg.d_latent) + 2 * Bp * T * H * cfg.d_head * cfg.d_latent * 2
        res[name] = {"ms": round(ms, 4), "TFLOPs": round(flop / (ms * 1e-3) / 1e12, 1),
                     "tokens_per_s": round(Bp * T / (ms * 1e-3), 1)}
        log(f"[bench] prefill T={T} B={Bp} {name}: {ms:.3f} ms, {flop / (ms * 1e-3) / 1e12:.1f} TFLOP/s")
    d = float(np.linalg.norm((out - out2).cpu().numpy()) / np.linalg.norm(out2.cpu().numpy()))
    res["rel_l2_naive_vs_absorbed"] = d
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="v2_b64_l8192")
    ap.add_argument("--heads", type=int, default=0, metavar="H",
                    help="run the workload with H heads instead of its own (a multiple of 16 "
                         "takes the gfx950 kernels; the workload is then named <workload>_h<H>)")
    ap.add_argument("--back-to-back", action="store_true",
                    help="no flush: steps back to back over several layers' inputs, two events")
    ap.add_argument("--merged", action="store_true",
                    help="decode and merge in one launch (mla_decode_merged)")
    ap.add_argument("--unfused", action="store_true",
                    help="merge and W^UV product as two launches (mla_combine, mla_out_proj)")
    ap.add_argument("--q-len", type=int, default=1,
                    help="query tokens per sequence (multi-token decode)")
    ap.add_argument("--slots", type=int, default=0,
                    help="workgroup slots the split plan aims at (default: the CU count)")
    ap.add_argument("--in-order", action="store_true",
                    help="plan for in-order dispatch and run the items in plan order "
                         "(default: longest-first plan and dispatch, mla_plan_splits_ordered)")
    ap.add_argument("--fenced-events", action="store_true",
                    help="time with torch.cuda.Event (each record also writes back and invalidates caches)")
    ap.add_argument("--prefill", type=int, default=0, metavar="T",
                    help="also time a T-token prefill of the first --prefill-batch sequences, "
                         "materialised-K/V path and absorbed path")
    ap.add_argument("--prefill-batch", type=int, default=4)
    ap.add_argument("--graph", action="store_true",
                    help="replay a HIP graph of each step's launches instead of launching them one by one")
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="before the warm-up steps, keep the GPU (and this process) busy this long "
                         "with the flush kernel: out of idle, the first steps run up to 10%% slower")
    ap.add_argument("--score-jump", type=float, default=0.0, metavar="F",
                    help="multiply the latent of every cached row after each sequence's first 32 "
                         "tokens by F (a jump of the score maxima after the first slice, which "
                         "moves the decode's softmax reference)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the decode path runs on one GPU; sharding is described, not built)", file=sys.stderr)
        sys.exit(2)
    T = args.q_len
    if T < 1 or (T > 1 and args.merged) or (args.merged and args.unfused):
        print("--q-len must be >= 1, and 1 with --merged; --merged and --unfused exclude "
              "each other", file=sys.stderr)
        sys.exit(2)

    import torch

    import mla_latent_kv_16_amd as mla
    from synth import CONFIGS, generate, query_multi

    cfg = CONFIGS[args.workload]
    if args.heads:
        from synth import small
        cfg = small(cfg, f"{cfg.name}_h{args.heads}", cfg.batch, n_heads=args.heads)
    t0 = time.perf_counter()
    wl = generate(cfg)
    log(f"[bench] generated {cfg.name} in {time.perf_counter() - t0:.1f} s "
        f"({wl.num_pages} pages, {wl.cache.nbytes / 1e9:.2f} GB cache)")

    def dev(a, bf):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if bf:
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.cuda()

    bf = cfg.dtype == "bf16"
    B, H = cfg.batch, cfg.n_heads
    if T == 1:
        q_nope, q_pe = dev(wl.q_nope, bf), dev(wl.q_pe, bf)
        positions = dev(wl.positions, False)
    else:
        qs = [query_multi(cfg, b, T) for b in range(B)]
        q_nope = dev(np.stack([a for a, _ in qs]).reshape(B * T, H, cfg.d_head), bf)
        q_pe = dev(np.stack([p for _, p in qs]).reshape(B * T, H, cfg.d_rope), bf)
        pos = wl.seq_lens[:, None].astype(np.int64) - T + np.arange(T)[None, :]
        positions = dev(pos.reshape(-1).astype(np.int32), False)
    layer0 = {"q_nope": q_nope, "q_pe": q_pe, "w_uk": dev(wl.w_uk, bf), "w_uv": dev(wl.w_uv, bf),
              "cache": dev(wl.cache, bf)}
    if args.score_jump:
        # every used slot except the first 32 tokens of each sequence
        scale = np.zeros(wl.cache.shape[:2], bool)
        for b in range(B):
            n = int(wl.seq_lens[b])
            toks = np.arange(32, n)
            scale[wl.block_table[b, toks // cfg.page_size], toks % cfg.page_size] = True
        m = torch.from_numpy(scale).cuda()
        lat = layer0["cache"][:, :, :cfg.d_latent]
        lat[m] = (lat[m].float() * args.score_jump).to(lat.dtype)
        log(f"[bench] latents after the first 32 tokens scaled by {args.score_jump:g}")
    # further layers: the same values in other memory (what matters for the
    # timing is that their rows, weights and queries are not where layer 0's are)
    args.flush = not args.back_to_back
    n_layers = 1 if args.flush else max(2, -(-(512 << 20) // wl.cache.nbytes) + 1)
    layers = [layer0] + [{k: v.clone() for k, v in layer0.items()} for _ in range(n_layers - 1)]
    block_table, seq_lens = dev(wl.block_table, False), dev(wl.seq_lens, False)
    dims = mla.Dims(cfg.n_heads, cfg.d_head, cfg.d_latent, cfg.d_rope, cfg.page_size,
                    rope_base=cfg.rope_base, dtype=mla.BF16 if bf else mla.F32)
    props = torch.cuda.get_device_properties(0)
    slots = args.slots or int(props.multi_processor_count)
    # each item is decoded once per query token: plan for the CUs over T.  The
    # single-token split decode runs the items longest first unless --in-order.
    ordered = T == 1 and not args.merged and not args.in_order
    order = None
    if ordered:
        items_h, offs_h, order_h = mla.plan_splits(dims, wl.seq_lens, max(1, slots // T), ordered=True)
        order = torch.from_numpy(order_h).cuda()
    else:
        items_h, offs_h = mla.plan_splits(dims, wl.seq_lens, max(1, slots // T))
    items, offs = torch.from_numpy(items_h).cuda(), torch.from_numpy(offs_h).cuda()
    log(f"[bench] {props.name} {getattr(props, 'gcnArchName', '')}, {props.multi_processor_count} CUs, "
        f"plan for {slots} slots; {len(items_h)} work items, q_len {T}, {n_layers} layer(s)")

    W = len(items_h)
    bufs = {
        "q_abs": torch.empty((B * T, H, dims.row), dtype=q_nope.dtype, device="cuda"),
        "o_part": torch.empty((W, T, H, cfg.d_latent), dtype=torch.float32, device="cuda"),
        "lse_part": torch.empty((W, T, H), dtype=torch.float32, device="cuda"),
        "o_latent": torch.empty((B * T, H, cfg.d_latent), dtype=torch.float32, device="cuda"),
        "lse": torch.empty((B * T, H), dtype=torch.float32, device="cuda"),
        "out": torch.empty((B * T, H, cfg.d_head), dtype=torch.float32, device="cuda"),
        "tickets": torch.zeros(2 * B, dtype=torch.int32, device="cuda"),
    }
    if T == 1:
        for k in ("o_part", "lse_part"):
            bufs[k] = bufs[k].view(W, *bufs[k].shape[2:])
    stream = torch.cuda.current_stream()
    q4 = bufs["q_abs"].view(B, T, H, dims.row)
    ol4 = bufs["o_latent"].view(B, T, H, cfg.d_latent)
    lse3 = bufs["lse"].view(B, T, H)
    out4 = bufs["out"].view(B, T, H, cfg.d_head)

    def launches_for(L):
        absorb = lambda: mla.absorb_q(dims, L["q_nope"], L["q_pe"], positions, L["w_uk"],  # noqa: E731
                                      bufs["q_abs"], cur())
        if T > 1 and args.unfused:
            names = ["absorb_q", "decode_splitkv_multi", "combine_multi", "out_proj"]
            fns = [absorb,
                   lambda: mla.decode_splitkv_multi(dims, q4, L["cache"], block_table, seq_lens, items,
                                                    bufs["o_part"], bufs["lse_part"], cur()),
                   lambda: mla.combine_multi(dims, offs, bufs["o_part"], bufs["lse_part"], B, ol4,
                                             lse3, cur()),
                   lambda: mla.out_proj(dims, bufs["o_latent"], L["w_uv"], bufs["out"], cur())]
        elif T > 1:
            names = ["absorb_q", "decode_splitkv_multi", "combine_out_proj"]
            fns = [absorb,
                   lambda: mla.decode_splitkv_multi(dims, q4, L["cache"], block_table, seq_lens, items,
                                                    bufs["o_part"], bufs["lse_part"], cur()),
                   lambda: mla.combine_out_proj(dims, offs, bufs["o_part"], bufs["lse_part"],
                                                L["w_uv"], B, out4, stream=cur())]
        elif args.merged:
            names = ["absorb_q", "decode_merged", "out_proj"]
            fns = [absorb,
                   lambda: mla.decode_merged(dims, bufs["q_abs"], L["cache"], block_table, seq_lens,
                                             items, offs, bufs["tickets"], bufs["o_part"],
                                             bufs["lse_part"], bufs["o_latent"], bufs["lse"], cur()),
                   lambda: mla.out_proj(dims, bufs["o_latent"], L["w_uv"], bufs["out"], cur())]
        elif args.unfused:
            names = ["absorb_q", "decode_splitkv", "combine", "out_proj"]
            fns = [absorb,
                   lambda: mla.decode_splitkv(dims, bufs["q_abs"], L["cache"], block_table, seq_lens,
                                              items, bufs["o_part"], bufs["lse_part"], cur(),
                                              order=order),
                   lambda: mla.combine(dims, offs, bufs["o_part"], bufs["lse_part"], B,
                                       bufs["o_latent"], bufs["lse"], cur()),
                   lambda: mla.out_proj(dims, bufs["o_latent"], L["w_uv"], bufs["out"], cur())]
        else:
            names = ["absorb_q", "decode_splitkv", "combine_out_proj"]
            fns = [absorb,
                   lambda: mla.decode_splitkv(dims, bufs["q_abs"], L["cache"], block_table, seq_lens,
                                              items, bufs["o_part"], bufs["lse_part"], cur(),
                                              order=order),
                   lambda: mla.combine_out_proj(dims, offs, bufs["o_part"], bufs["lse_part"],
                                                L["w_uv"], B, bufs["out"], stream=cur())]
        return names, fns

    def cur():
        # the stream torch makes current: `stream` when eager, the capture
        # stream while a graph is being recorded
        return torch.cuda.current_stream()

    per_layer = [launches_for(L) for L in layers]
    names = per_layer[0][0]
    n_k = len(names)
    flush = sink = None
    if args.flush:
        flush = torch.full((128 << 20,), 1.0, dtype=torch.float32, device="cuda")  # 512 MiB
        sink = torch.empty(1, dtype=torch.float32, device="cuda")

    def evict():
        if flush is not None:
            torch.sum(flush, dim=0, keepdim=True, out=sink)

    graphs = None
    recorded = None   # per layer, per kernel: the library calls, marshalled once

    def step(k, ev=None):
        if ev is None and graphs is not None:
            graphs[k % n_layers].replay()
            return
        launches = recorded[k % n_layers] if recorded is not None else per_layer[k % n_layers][1]
        for i, launch in enumerate(launches):
            if ev is not None:
                ev[i].record(stream)
            if recorded is not None:
                mla.replay_calls(launch)
            else:
                launch()
        if ev is not None:
            ev[n_k].record(stream)

    def new_events(n):
        if args.fenced_events:
            return [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        return [HipTimingEvent() for _ in range(n)]

    if args.settle_ms > 0:
        t_s = time.perf_counter()
        while (time.perf_counter() - t_s) * 1e3 < args.settle_ms:
            for _ in range(8):
                evict()
            torch.cuda.synchronize()
    for k in range(args.warmup):
        evict()
        step(k)
    torch.cuda.synchronize()
    # The timed passes issue the same library calls with their arguments
    # marshalled once (the binding's checks ran in the warm-up): a step's
    # host-side cost then stays well below its GPU time, so the kernels run
    # back to back instead of waiting for their launches.
    recorded = []
    for _, fns in per_layer:
        per_kernel = []
        for launch in fns:
            with mla.record_calls() as calls:
                launch()
            per_kernel.append(calls)
        recorded.append(per_kernel)
    if args.graph:
        # one graph per layer: the step's launches, recorded once and replayed
        # (the kernels and their arguments are those of the eager step)
        graphs = []
        for _, fns in per_layer:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for launch in fns:
                    launch()
            graphs.append(g)
        torch.cuda.synchronize()
        for k in range(2):
            evict()
            step(k)
        torch.cuda.synchronize()
    k0 = args.warmup   # the first timed step uses the layer the last warmup step did not

    # Timed region: K steps.
    torch.cuda.synchronize()
    step_ev = [new_events(2) for _ in range(args.steps)] if args.flush else None
    w0 = time.perf_counter()
    if args.flush:
        for k in range(args.steps):
            evict()
            step_ev[k][0].record(stream)
            step(k0 + k)
            step_ev[k][1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        step_ms = np.array([e[0].elapsed_time(e[1]) for e in step_ev])
        pct = {"step_ms_p10": round(float(np.percentile(step_ms, 10)), 5),
               "step_ms_median": round(float(np.median(step_ms)), 5),
               "step_ms_p90": round(float(np.percentile(step_ms, 90)), 5)}
        ms = float(step_ms.mean())
        spread = f"p10 {np.percentile(step_ms, 10):.4f}  p90 {np.percentile(step_ms, 90):.4f}"
    else:
        e0, e1 = new_events(2)
        e0.record(stream)
        for k in range(args.steps):
            step(k0 + k)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        ms = e0.elapsed_time(e1) / args.steps
        spread = f"{args.steps} steps back to back"
        pct = {}

    # Per-kernel breakdown: the same steps with an event between every two kernels.
    evs = [new_events(n_k + 1) for _ in range(args.steps)]
    for k in range(args.steps):
        evict()
        step(k0 + k, evs[k])
    torch.cuda.synchronize()
    t = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(n_k)] for e in evs])  # ms
    k_ms = t.mean(axis=0)

    # The decode kernel alone, K launches back to back (cycling over the layers).
    dec = [(lambda c=calls[1]: mla.replay_calls(c)) for calls in recorded]
    if H == 128 and bf:
        mla.exact_pass_count(reset=True)
    if args.flush:
        d_ev = [new_events(2) for _ in range(args.steps)]
        for k in range(args.steps):
            evict()
            d_ev[k][0].record(stream)
            dec[0]()
            d_ev[k][1].record(stream)
        torch.cuda.synchronize()
        dec_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in d_ev]))
    else:
        e0, e1 = new_events(2)
        e0.record(stream)
        for k in range(args.steps):
            dec[(k0 + k) % n_layers]()
        e1.record(stream)
        torch.cuda.synchronize()
        dec_ms = e0.elapsed_time(e1) / args.steps
    # work-item halves the decode redid against exact maxima, over the decode
    # launches of the last pass
    exact_passes = None
    if H == 128 and bf:
        exact_passes = mla.exact_pass_count(reset=True)
        torch.cuda.synchronize()
    log("[bench] per-kernel mean ms (event between kernels): " +
        ", ".join(f"{n} {v:.4f}" for n, v in zip(names, k_ms)))
    log(f"[bench] step ms: {ms:.4f} ({spread}); decode launch ms: {dec_ms:.4f}; "
        f"wall {wall * 1e3 / args.steps:.3f} ms/step")
    assert torch.isfinite(bufs["out"]).all().item(), "non-finite output"

    work = algorithmic(cfg, wl.seq_lens, T, n_items=len(items_h))
    dec_s = dec_ms * 1e-3
    achieved = work["decode_bytes"] / dec_s / 1e9
    # HBM fraction of each kernel's own bytes (event-bracketed times, so each
    # includes the few microseconds an event between kernels adds)
    kbytes = {"absorb_q": work["absorb_bytes"], names[1]: work["decode_bytes"],
              "combine_out_proj": work["merge_bytes"]}
    kernel_frac = {n: round(kbytes[n] / (v * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
                   for n, v in zip(names, k_ms) if n in kbytes}
    traffic = measured_traffic(cfg.name) if T == 1 and not args.merged else None
    result = {
        "metric": METRIC,
        "value": round(work["step_flop"] / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        **pct,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "seq_len": int(wl.seq_lens.max()),
                   "total_tokens": int(wl.seq_lens.sum()), "n_heads": H, "d_head": cfg.d_head,
                   "d_latent": cfg.d_latent, "d_rope": cfg.d_rope, "page_size": cfg.page_size,
                   "work_items": int(len(items_h)), "q_len": T, "decode_entry": names[1],
                   "dispatch": "longest-first" if ordered else "in-order",
                   "timing": ("per-step events, 512 MiB read flush before each step" if args.flush
                              else f"back to back, cycling over {n_layers} layers' inputs")
                             + (f"; {args.settle_ms:g} ms of the flush kernel before the warm-up"
                                if args.settle_ms > 0 else "")
                             + ("; step replayed as a HIP graph" if args.graph else "")},
        "latent_cache_GBps": round(work["cache_bytes"] / (ms * 1e-3) / 1e9, 1),
        "tokens_per_s": round(B * T / (ms * 1e-3), 1),
        "kernel_ms": {n: round(float(v), 5) for n, v in zip(names, k_ms)},
        "decode_ms": round(dec_ms, 5),
        "decode_TFLOPs": round(work["decode_flop"] / dec_s / 1e12, 2),
        "decode_mfma_frac": round(work["decode_flop"] / dec_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "roofline": {"kernel": names[1], "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": work["decode_bytes"],
                     "bytes_definition": "cache rows once + q_abs + latent output (bf16) + block table",
                     "frac_with_f32_latent_output": round(
                         work["decode_bytes_f32"] / dec_s / 1e9 / HBM_PEAK_GBPS, 4),
                     # the aim set for the decode kernel: 60 % of its binding roofline
                     "target_frac": TARGET_FRAC,
                     "target_met": bool(achieved / HBM_PEAK_GBPS >= TARGET_FRAC)},
        "kernel_hbm_frac": kernel_frac,
        "score_jump": args.score_jump or None,
        "exact_pass_workgroups_per_launch": (None if exact_passes is None
                                             else round(exact_passes / args.steps, 3)),
        "step_hbm_frac": round(work["step_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "step_mfma_frac": round(work["step_flop"] / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "step_algorithmic_bytes": work["step_bytes"],
    }
    # the step's output on the workload's own inputs (layer 0, before the cache
    # write below changes a slot), for the check against the oracle
    gpu_out = None
    if T == 1 and not args.score_jump and n_layers == 1 and not args.no_cpu_baseline:
        torch.cuda.synchronize()
        gpu_out = bufs["out"].view(B, H, cfg.d_head).float().cpu().numpy()
    # The cache write of the next token of every sequence (mla_append_kv), timed
    # on its own (per-launch events): it precedes the step in a model and is not
    # part of `value`.
    from synth import append_recipe, f32_to_bf16_bits
    ar = append_recipe(cfg, B)
    conv = (lambda a: f32_to_bf16_bits(a.astype(np.float32))) if bf else (lambda a: a.astype(np.float32))
    h_d, wdkv_d, wkr_d = dev(conv(ar["h"]), bf), dev(conv(ar["w_dkv"]), bf), dev(conv(ar["w_kr"]), bf)
    app_pos = torch.from_numpy(np.minimum(wl.seq_lens, wl.block_table.shape[1] * cfg.page_size - 1)
                               .astype(np.int32)).cuda()
    cache0 = layers[0]["cache"]  # the rows written (one slot per sequence) are rewritten identically
    import ctypes
    a_need = mla.load().mla_append_kv_workspace_bytes(ctypes.byref(dims.c()), cfg.d_model, B)
    a_ws = torch.empty(max(a_need, 4) // 4, dtype=torch.float32, device="cuda")
    a_ms = []
    for k in range(args.warmup + args.steps):
        ea, eb = new_events(2)
        # as before each step: the flush evicts the caches, and the host
        # enqueues the call while the GPU reads it, so the events bracket the
        # call's two kernels and not the host's marshalling
        evict()
        ea.record(stream)
        mla.append_kv(dims, h_d, wdkv_d, wkr_d, app_pos, cache0, block_table,
                      rms_norm=cfg.rms_norm_latent, workspace=a_ws, stream=stream)
        eb.record(stream)
        torch.cuda.synchronize()
        if k >= args.warmup:
            a_ms.append(ea.elapsed_time(eb))
    a_ms = float(np.mean(a_ms))
    esz = 2 if bf else 4
    D = cfg.d_latent + cfg.d_rope
    a_bytes = (D * cfg.d_model + B * cfg.d_model + B * D) * esz
    result["append_kv"] = {"ms": round(a_ms, 5), "algorithmic_bytes": a_bytes,
                           "GBps": round(a_bytes / (a_ms * 1e-3) / 1e9, 1), "d_model": cfg.d_model}
    log(f"[bench] append_kv {a_ms * 1e3:.1f} us for {B} tokens ({a_bytes / 1e6:.2f} MB algorithmic)")
    if args.prefill > 0:
        result["prefill"] = time_prefill(args, cfg, wl, dims, layers[0], block_table, seq_lens, stream,
                                         new_events, evict, slots)
    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(3)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy probe: 1 GiB device-to-device copy done")
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(wl, gpu_out=gpu_out)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
