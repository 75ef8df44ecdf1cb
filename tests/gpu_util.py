"""Helpers for the GPU tests: upload a synthetic workload, run libmla, compare."""
from __future__ import annotations

import sys

import numpy as np

import mla_latent_kv_16_amd as mla

REL_L2 = 5e-3          # bf16 inputs, float32 accumulation
MAX_ABS = 2e-2         # times max |reference|
LSE_ABS = 1e-2
F32_REL = 1e-5         # float32 storage


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dims_of(cfg) -> mla.Dims:
    return mla.Dims(cfg.n_heads, cfg.d_head, cfg.d_latent, cfg.d_rope, cfg.page_size,
                    rope_base=cfg.rope_base, dtype=mla.BF16 if cfg.dtype == "bf16" else mla.F32)


def to_dev(a: np.ndarray, bf16: bool):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if bf16 and a.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.cuda()


def upload(wl) -> dict:
    bf = wl.cfg.dtype == "bf16"
    return {
        "q_nope": to_dev(wl.q_nope, bf), "q_pe": to_dev(wl.q_pe, bf),
        "positions": to_dev(wl.positions.astype(np.int32), False),
        "w_uk": to_dev(wl.w_uk, bf), "w_uv": to_dev(wl.w_uv, bf),
        "cache": to_dev(wl.cache, bf), "block_table": to_dev(wl.block_table, False),
        "seq_lens": to_dev(wl.seq_lens, False),
    }


def num_slots() -> int:
    import torch
    return int(torch.cuda.get_device_properties(0).multi_processor_count)


def run(wl, dev=None, slots=None, items=None, offs=None, ordered=False) -> dict:
    """Run the four device steps; return numpy copies of every output.
    `ordered`: the longest-first plan and dispatch (as the bench runs them)."""
    import torch
    dims = dims_of(wl.cfg)
    dev = upload(wl) if dev is None else dev
    order = None
    if items is None:
        if ordered:
            items, offs, order = mla.plan_splits(dims, wl.seq_lens, slots or num_slots(), ordered=True)
        else:
            items, offs = mla.plan_splits(dims, wl.seq_lens, slots or num_slots())
    it_d = torch.from_numpy(items).cuda()
    of_d = torch.from_numpy(offs).cuda()
    or_d = None if order is None else torch.from_numpy(order).cuda()
    b = mla.decode_step(dims, dev["q_nope"], dev["q_pe"], dev["positions"], dev["w_uk"],
                        dev["w_uv"], dev["cache"], dev["block_table"], dev["seq_lens"], it_d, of_d,
                        order=or_d)
    torch.cuda.synchronize()
    out = {}
    for k in ("q_abs", "o_latent", "lse", "out", "o_part", "lse_part"):
        t = b[k]
        out[k] = t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()
    out["items"], out["offs"] = items, offs
    return out


def errors(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    mx = np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300)
    return rel, mx


def assert_close(got, ref, name, rel_tol=REL_L2, max_tol=MAX_ABS):
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    rel, mx = errors(got, ref)
    say(f"  {name}: rel L2 {rel:.3e}  max-abs/max|ref| {mx:.3e}")
    assert rel <= rel_tol, f"{name}: rel L2 {rel:.3e} > {rel_tol}"
    assert mx <= max_tol, f"{name}: max-abs ratio {mx:.3e} > {max_tol}"


def assert_lse(got, ref, name="lse", tol=LSE_ABS):
    d = float(np.max(np.abs(np.asarray(got, np.float64) - ref)))
    say(f"  {name}: max abs diff {d:.3e}")
    assert d <= tol, f"{name}: max abs diff {d:.3e} > {tol}"


def compare_with_oracle(wl, out, seqs, heads=None, f32=False):
    """Check q_abs, o_latent, lse and out of the chosen sequences against the oracle."""
    from oracle import decode_workload
    ref = decode_workload(wl, seqs=seqs, heads=heads)
    seqs = list(seqs)
    h = slice(None) if heads is None else list(heads)
    sel = lambda a: np.asarray(a)[seqs][:, h]  # noqa: E731
    tol = dict(rel_tol=F32_REL, max_tol=10 * F32_REL) if f32 else {}
    assert_close(sel(out["q_abs"]), ref["q_abs"], "q_abs", **tol)
    assert_close(sel(out["o_latent"]), ref["o_latent"], "o_latent", **tol)
    assert_close(sel(out["out"]), ref["o"], "out", **tol)
    assert_lse(sel(out["lse"]), ref["lse"], tol=1e-4 if f32 else LSE_ABS)
    return ref
