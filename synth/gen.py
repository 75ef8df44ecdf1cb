"""Seeded synthetic inputs for one MLA decode step.

This module only draws random numbers and lays them out; it computes nothing
of the method (no projection, no normalisation layer, no rotation, no
attention).  Both the fp64 oracle and the HIP path consume what it returns.

What one decode step receives, per sequence b of length L_b:
  * the paged latent cache: for every token j < L_b one row
    [c^KV_j (d_c) | k^R_j (d_h^R)], k^R_j being the position-encoded key as the
    cache keeps it (page "DeepSeek V2 技术解析" 2.2.2: the key's RoPE part is
    cached after encoding);
  * the per-head query parts q^C_{b,i} (d_h) and q^R_{b,i} (d_h^R, not yet
    position-encoded), and the query position p_b = L_b - 1;
  * the up-projections W^UK, W^UV, each [n_h * d_h, d_c], head i owning rows
    i*d_h .. i*d_h + d_h - 1;
  * a block table and the sequence lengths.

Value distributions (drawn directly, in place of projecting hidden states):
  * c^KV_j: for RMS-normalised workloads, uniform on the sphere of radius
    sqrt(d_c) -- the law of an RMS-normalised isotropic Gaussian; otherwise
    N(0, 1) per component.
  * k^R_j: N(0, 1) per component.  A rotation maps an isotropic Gaussian to
    itself, so this is also the law of a position-encoded N(0, I) key.
  * q^C, q^R: N(0, 1) per component (the variance of W h with
    W ~ N(0, 1/fan_in), h ~ N(0, 1)).
  * W^UK, W^UV: N(0, 1/d_c) (standard deviation 1/sqrt(d_c)).

Random streams are numpy PCG64 generators seeded from
SeedSequence(value_seed, spawn_key=key) with key = (0,) for the weights,
(1, b) for the query of sequence b and (2, b, chunk) for 2048-token chunks of
sequence b, so any sequence can be regenerated alone.

bf16 storage rounds float32 to the nearest bf16, ties to even.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import MLAConfig

CHUNK_TOKENS = 2048


# ----------------------------------------------------------------------------
# storage formats
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits.

    NaN stays a quiet NaN; infinities are preserved.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(cfg: MLAConfig, x32: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(x32) if cfg.dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


def _rng(cfg: MLAConfig, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(cfg.value_seed, spawn_key=tuple(key)))


# ----------------------------------------------------------------------------
# lengths and pages
# ----------------------------------------------------------------------------
def seq_lens(cfg: MLAConfig) -> np.ndarray:
    if cfg.seq_len is not None:
        return np.full(cfg.batch, cfg.seq_len, dtype=np.int32)
    lo, hi = cfg.len_range
    return np.random.default_rng(cfg.len_seed).integers(lo, hi + 1, cfg.batch).astype(np.int32)


def pages_per_seq(lens: np.ndarray, page_size: int) -> np.ndarray:
    return ((lens.astype(np.int64) + page_size - 1) // page_size).astype(np.int32)


def block_table(cfg: MLAConfig, lens: np.ndarray) -> tuple[np.ndarray, int]:
    """Block table [batch][max_pages] (unused entries 0) and the page count.

    Logical page p of sequence b is the (offset_b + p)-th entry of the page
    order, where offset_b counts the pages of earlier sequences; the order is
    the identity, or a seeded permutation of all pages.
    """
    npg = pages_per_seq(lens, cfg.page_size)
    total = int(npg.sum())
    order = (np.random.default_rng(cfg.page_seed).permutation(total) if cfg.permute_pages
             else np.arange(total))
    bt = np.zeros((cfg.batch, max(int(npg.max()), 1)), dtype=np.int32)
    off = 0
    for b in range(cfg.batch):
        bt[b, :npg[b]] = order[off:off + npg[b]]
        off += int(npg[b])
    return bt, total


# ----------------------------------------------------------------------------
# values
# ----------------------------------------------------------------------------
def weights(cfg: MLAConfig) -> tuple[np.ndarray, np.ndarray]:
    """W^UK, W^UV as stored: [n_h * d_h, d_c] each (drawn in that order)."""
    r = _rng(cfg, 0)
    shape = (cfg.n_heads * cfg.d_head, cfg.d_latent)
    s = np.float32(1.0 / np.sqrt(cfg.d_latent))
    w_uk = r.standard_normal(shape, dtype=np.float32) * s
    w_uv = r.standard_normal(shape, dtype=np.float32) * s
    return _store(cfg, w_uk), _store(cfg, w_uv)


def query(cfg: MLAConfig, b: int) -> tuple[np.ndarray, np.ndarray]:
    """q^C [n_h, d_h] and q^R [n_h, d_h^R] of sequence b, as stored."""
    r = _rng(cfg, 1, b)
    qn = r.standard_normal((cfg.n_heads, cfg.d_head), dtype=np.float32)
    qp = r.standard_normal((cfg.n_heads, cfg.d_rope), dtype=np.float32)
    return _store(cfg, qn), _store(cfg, qp)


def query_multi(cfg: MLAConfig, b: int, q_len: int) -> tuple[np.ndarray, np.ndarray]:
    """q^C [q_len, n_h, d_h] and q^R [q_len, n_h, d_h^R] (not yet encoded) of the
    q_len newest tokens of sequence b, in the storage type; N(0, 1)."""
    r = _rng(cfg, 5, b)
    qn = r.standard_normal((q_len, cfg.n_heads, cfg.d_head), dtype=np.float32)
    qp = r.standard_normal((q_len, cfg.n_heads, cfg.d_rope), dtype=np.float32)
    return _store(cfg, qn), _store(cfg, qp)


def token_chunk(cfg: MLAConfig, b: int, chunk: int, n: int) -> np.ndarray:
    """Rows [n, d_c + d_h^R] for tokens chunk*2048 .. chunk*2048 + n - 1 of sequence b."""
    r = _rng(cfg, 2, b, chunk)
    c = r.standard_normal((n, cfg.d_latent), dtype=np.float32)
    if cfg.rms_norm_latent:
        # uniform direction, radius sqrt(d_c): the law of an RMS-normalised
        # isotropic Gaussian vector
        nrm = np.sqrt(np.einsum("ij,ij->i", c.astype(np.float64), c.astype(np.float64)))
        c = (c * (np.sqrt(cfg.d_latent) / nrm)[:, None]).astype(np.float32)
    kr = r.standard_normal((n, cfg.d_rope), dtype=np.float32)
    return _store(cfg, np.concatenate([c, kr], axis=1))


def sequence_rows(cfg: MLAConfig, b: int, length: int) -> np.ndarray:
    """All cached rows of sequence b in token order (regenerated from its seeds)."""
    parts = []
    for ch in range((length + CHUNK_TOKENS - 1) // CHUNK_TOKENS):
        n = min(CHUNK_TOKENS, length - ch * CHUNK_TOKENS)
        parts.append(token_chunk(cfg, b, ch, n))
    dt = np.uint16 if cfg.dtype == "bf16" else np.float32
    return np.concatenate(parts, axis=0) if parts else np.zeros((0, cfg.d_qk), dt)


@dataclass
class Workload:
    cfg: MLAConfig
    seq_lens: np.ndarray      # [B] int32
    positions: np.ndarray     # [B] int32, query position L_b - 1
    block_table: np.ndarray   # [B, max_pages] int32
    num_pages: int
    cache: np.ndarray         # [num_pages, page_size, d_c + d_h^R] (uint16 bf16 bits or float32)
    q_nope: np.ndarray        # [B, n_h, d_h]
    q_pe: np.ndarray          # [B, n_h, d_h^R]
    w_uk: np.ndarray          # [n_h * d_h, d_c]
    w_uv: np.ndarray          # [n_h * d_h, d_c]

    @property
    def is_bf16(self) -> bool:
        return self.cfg.dtype == "bf16"


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def generate(cfg: MLAConfig, pad_value: Optional[float] = None,
             lens: Optional[np.ndarray] = None) -> Workload:
    """Build the full workload of `cfg`.

    pad_value: value written into the cache slots that hold no token (the tail
    of each sequence's last page); zero when None.  A NaN here poisons them.
    lens: override the sequence lengths (same seeds for everything else).
    """
    L = seq_lens(cfg) if lens is None else np.asarray(lens, dtype=np.int32)
    if L.shape != (cfg.batch,):
        raise ValueError("lens must have one entry per sequence")
    bt, total = block_table(cfg, L)
    P, D = cfg.page_size, cfg.d_qk
    dt = np.uint16 if cfg.dtype == "bf16" else np.float32
    fill = 0 if pad_value is None else pad_value
    if cfg.dtype == "bf16":
        fillv = f32_to_bf16_bits(np.array([fill], np.float32))[0]
    else:
        fillv = np.float32(fill)
    cache = np.empty((total, P, D), dtype=dt)
    # only the last page of a sequence can have empty slots
    for b in range(cfg.batch):
        n = int(L[b])
        if n % P:
            cache[bt[b, (n - 1) // P], n % P:, :] = fillv

    jobs = [(b, ch) for b in range(cfg.batch)
            for ch in range((int(L[b]) + CHUNK_TOKENS - 1) // CHUNK_TOKENS)]

    def work(job):
        b, ch = job
        n = min(CHUNK_TOKENS, int(L[b]) - ch * CHUNK_TOKENS)
        rows = token_chunk(cfg, b, ch, n)
        t0 = ch * CHUNK_TOKENS
        for i0 in range(0, n, P):          # chunks start on page boundaries
            t = t0 + i0
            k = min(P, n - i0)
            cache[bt[b, t // P], :k, :] = rows[i0:i0 + k]

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, jobs))

    qs = [query(cfg, b) for b in range(cfg.batch)]
    q_nope = np.stack([q[0] for q in qs])
    q_pe = np.stack([q[1] for q in qs])
    w_uk, w_uv = weights(cfg)
    return Workload(cfg=cfg, seq_lens=L, positions=(L - 1).astype(np.int32), block_table=bt,
                    num_pages=total, cache=cache, q_nope=q_nope, q_pe=q_pe,
                    w_uk=w_uk, w_uv=w_uv)


# ----------------------------------------------------------------------------
# raw draws for the full cache-write recipe (hidden states and all weights);
# used where the oracle itself derives the cache from hidden states
# ----------------------------------------------------------------------------
def hidden_recipe(cfg: MLAConfig, length: int) -> dict:
    """h_t ~ N(0, 1) for t < length and every projection ~ N(0, 1/fan_in), float64.

    Matrices map column vectors: W^DKV [d_c, d_model], W^KR [d_h^R, d_model],
    W^Q [n_h d_h, d_model], W^QR [n_h d_h^R, d_model], W^UK/W^UV [n_h d_h, d_c].
    """
    r = _rng(cfg, 3)
    dm, H = cfg.d_model, cfg.n_heads

    def w(rows, fan_in):
        return r.standard_normal((rows, fan_in)) / np.sqrt(fan_in)

    out = {
        "w_dkv": w(cfg.d_latent, dm),
        "w_kr": w(cfg.d_rope, dm),
        "w_uk": w(H * cfg.d_head, cfg.d_latent),
        "w_uv": w(H * cfg.d_head, cfg.d_latent),
        "w_q": w(H * cfg.d_head, dm),
        "w_qr": w(H * cfg.d_rope, dm),
    }
    out["h"] = r.standard_normal((length, dm))
    return out


def chain_recipe(cfg: MLAConfig, lens) -> dict:
    """Everything one decode step derives from hidden states, float32 draws.

    h_b [L_b, d_model] ~ N(0, 1) for every sequence b (its tokens 0 .. L_b - 1;
    the query is token L_b - 1), and every projection ~ N(0, 1/fan_in), each
    mapping column vectors: W^DKV [d_c, d_model], W^KR [d_h^R, d_model],
    W^UK and W^UV [n_h d_h, d_c]; with a query latent of width d_cq
    (cfg.q_latent): W^DQ [d_cq, d_model], W^UQ [n_h d_h, d_cq],
    W^QR [n_h d_h^R, d_cq]; without one: W^Q [n_h d_h, d_model],
    W^QR [n_h d_h^R, d_model].  Streams: key (6,) for the weights, (7, b) for
    the hidden states of sequence b.
    """
    r = _rng(cfg, 6)
    dm, H = cfg.d_model, cfg.n_heads

    def w(rows, fan_in):
        return (r.standard_normal((rows, fan_in), dtype=np.float32) /
                np.float32(np.sqrt(fan_in)))

    out = {"w_dkv": w(cfg.d_latent, dm), "w_kr": w(cfg.d_rope, dm),
           "w_uk": w(H * cfg.d_head, cfg.d_latent), "w_uv": w(H * cfg.d_head, cfg.d_latent)}
    if cfg.q_latent:
        out["w_dq"] = w(cfg.q_latent, dm)
        out["w_uq"] = w(H * cfg.d_head, cfg.q_latent)
        out["w_qr"] = w(H * cfg.d_rope, cfg.q_latent)
    else:
        out["w_q"] = w(H * cfg.d_head, dm)
        out["w_qr"] = w(H * cfg.d_rope, dm)
    out["h"] = [_rng(cfg, 7, b).standard_normal((int(n), dm), dtype=np.float32)
                for b, n in enumerate(lens)]
    return out


def append_recipe(cfg: MLAConfig, batch: int) -> dict:
    """Inputs of the cache write of one new token per sequence, float64:
    h [batch, d_model] ~ N(0, 1), W^DKV [d_c, d_model] and W^KR [d_h^R, d_model]
    ~ N(0, 1/d_model) (matrices map column vectors)."""
    r = _rng(cfg, 4)
    dm = cfg.d_model
    return {
        "w_dkv": r.standard_normal((cfg.d_latent, dm)) / np.sqrt(dm),
        "w_kr": r.standard_normal((cfg.d_rope, dm)) / np.sqrt(dm),
        "h": r.standard_normal((batch, dm)),
    }
