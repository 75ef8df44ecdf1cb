"""fp64 CPU oracle for one MLA decode step (the pages' naive path).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call this module.  It shares no code with the
HIP path and imports nothing from the product package.

Pages cited (titles as published):
  [V2-解析]  "DeepSeek V2 技术解析：多头潜在注意力（MLA）与混合专家模型（MoE）的创新实践"
  [两张账]   "DeepSeek-V2/V3：大模型的两张账，为什么 MLA 与 MoE 要一起看"
  [笔记]     "DeepSeek-V2: A Strong, Economical, and Efficient Mixture-of-Experts
              Language Model" (reading notes)

What is computed, for one sequence of L cached tokens and every head i:
  k^C_{j,i} = W^UK_i c_j,  v^C_{j,i} = W^UV_i c_j           [V2-解析] 2.2.1.1
  k_{j,i}   = [k^C_{j,i} ; k^R_j]   (k^R_j shared by heads,
              cached already position-encoded)             [V2-解析] 2.2.2; [两张账] RoPE section
  q_i       = [q^C_i ; RoPE_p(q^R_i)]                        [V2-解析] 2.2.2
  s_ij      = q_i . k_{j,i} / sqrt(d_h + d_h^R)
  a_ij      = softmax_j(s_ij),  o_i = sum_j a_ij v^C_{j,i}
The naive form recovers k^C and v^C from the cached latent before attending
([V2-解析] 2.2.2, last paragraphs; [两张账] "第一张账", the "naive" path).
Also reported, for per-kernel checks, by their definitions:
  q~_i   = (W^UK_i)^T q^C_i     (W^UK moved to the query side)
  o~_i   = sum_j a_ij c_j       (aggregation in latent space)
  lse_i  = log sum_j exp(s_ij)
([两张账] "第一张账": scores from the transformed query and the cached latent,
aggregation in latent space and then mapped out.)

Readings where the pages are silent (all formulas there were images):
  * scale 1/sqrt(d_h + d_h^R), the width of the concatenated dot product;
  * RoPE on adjacent pairs (2k, 2k+1) with theta_k = base^(-2k/d) and the
    rotation [[cos, -sin], [sin, cos]]; angles in float64;
  * W^UK, W^UV are [n_h d_h, d_c] with head i owning rows i*d_h .. i*d_h+d_h-1;
  * the query sits at position L-1 and attends to tokens 0..L-1.

Every function is pinned in tests/test_oracle.py against closed forms,
identities the pages state, fixed bit patterns, library routines, or inputs
built so that the right answer is known by construction (selection
matrices), and each pin is shown to fail on a planted mistake; none is
"parity unpinned".  The two whole-workload drivers (decode_workload,
multi_decode_workload) only gather rows and loop over sequences around the
pinned per-sequence functions; they are checked against each other and
against the generator's token order.
"""
from __future__ import annotations

from typing import Dict, Iterable, Optional

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------
# storage decoding
# ----------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 (exact: bf16 is the top half of float32)."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(F64)


def to_f64(x: np.ndarray, is_bf16: bool) -> np.ndarray:
    return bf16_to_f64(x) if is_bf16 else np.asarray(x, dtype=F64)


# ----------------------------------------------------------------------------
# RoPE  ([V2-解析] 2.2.2: S = Q^T R_m^T R_n K with R_m the rotation at position m)
# ----------------------------------------------------------------------------
def rope_theta(d_rope: int, base: float) -> np.ndarray:
    """theta_k = base^(-2k/d_rope), k = 0 .. d_rope/2 - 1."""
    k = np.arange(d_rope // 2, dtype=F64)
    return base ** (-2.0 * k / d_rope)


def rope(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate each adjacent pair (x_2k, x_2k+1) of the last axis by angle pos*theta_k.

    x: [..., d_rope]; pos: scalar or array broadcastable to x.shape[:-1].
    """
    x = np.asarray(x, dtype=F64)
    d = x.shape[-1]
    ang = np.asarray(pos, dtype=F64)[..., None] * rope_theta(d, base)  # [..., d/2]
    cos, sin = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y = np.empty(np.broadcast_shapes(x.shape, cos.shape[:-1] + (d,)), dtype=F64)
    y[..., 0::2] = x0 * cos - x1 * sin
    y[..., 1::2] = x0 * sin + x1 * cos
    return y


def rope_matrix(pos: float, d_rope: int, base: float) -> np.ndarray:
    """The block-diagonal matrix R_pos with rope(x, pos) == R_pos @ x."""
    R = np.zeros((d_rope, d_rope), dtype=F64)
    for k, th in enumerate(rope_theta(d_rope, base)):
        c, s = np.cos(pos * th), np.sin(pos * th)
        R[2 * k, 2 * k], R[2 * k, 2 * k + 1] = c, -s
        R[2 * k + 1, 2 * k], R[2 * k + 1, 2 * k + 1] = s, c
    return R


# ----------------------------------------------------------------------------
# paged cache addressing ([V2-解析] 2.1.1: paged KV memory; tokens are rows of
# fixed-size pages reached through a per-sequence block table)
# ----------------------------------------------------------------------------
def gather_rows(cache: np.ndarray, block_table_row: np.ndarray, length: int,
                page_size: int) -> np.ndarray:
    """Rows of tokens 0..length-1: token j is slot j % page_size of page block_table_row[j // page_size]."""
    j = np.arange(length)
    pages = np.asarray(block_table_row)[j // page_size]
    return cache[pages, j % page_size]


# ----------------------------------------------------------------------------
# the naive decode step for one sequence
# ----------------------------------------------------------------------------
def _head_rows(w: np.ndarray, i: int, d_head: int) -> np.ndarray:
    """W_i: rows i*d_head .. i*d_head + d_head - 1 of a [n_h d_h, d_c] matrix."""
    return w[i * d_head:(i + 1) * d_head]


def naive_decode_seq(c: np.ndarray, k_rope: np.ndarray, q_nope: np.ndarray, q_pe: np.ndarray,
                     pos: int, w_uk: np.ndarray, w_uv: np.ndarray, scale: float,
                     rope_base: float, heads: Optional[Iterable[int]] = None,
                     head_block: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Attention of one query over L cached tokens, all in float64.

    c [L, d_c] latents; k_rope [L, d_h^R] cached (already encoded) keys;
    q_nope [n_h, d_h], q_pe [n_h, d_h^R] (q_pe not yet encoded); pos: query position;
    w_uk, w_uv [n_h d_h, d_c].
    Returns o [n, d_h], o_latent [n, d_c], lse [n], q_abs [n, d_c + d_h^R] for the
    selected heads (all by default), in head order.
    """
    c = np.asarray(c, F64)
    k_rope = np.asarray(k_rope, F64)
    L, d_c = c.shape
    n_h, d_h = q_nope.shape
    heads = list(range(n_h)) if heads is None else list(heads)
    if head_block is None:
        # bound the materialised per-head K/V to ~256 MB
        head_block = max(1, min(len(heads), (256 << 20) // max(1, L * (2 * d_h + k_rope.shape[1]) * 8)))
    q_rot = rope(q_pe, pos, rope_base)  # RoPE_p(q^R_i), [n_h, d_h^R]

    out = {k: [] for k in ("o", "o_latent", "lse", "q_abs")}
    for h0 in range(0, len(heads), head_block):
        hs = heads[h0:h0 + head_block]
        wk = np.stack([_head_rows(w_uk, i, d_h) for i in hs]).astype(F64)  # [n, d_h, d_c]
        wv = np.stack([_head_rows(w_uv, i, d_h) for i in hs]).astype(F64)
        n = len(hs)
        # naive recovery of per-head keys and values from the latent
        kC = (c @ wk.reshape(n * d_h, d_c).T).reshape(L, n, d_h)     # k^C_{j,i} = W^UK_i c_j
        vC = (c @ wv.reshape(n * d_h, d_c).T).reshape(L, n, d_h)     # v^C_{j,i} = W^UV_i c_j
        K = np.concatenate([kC, np.broadcast_to(k_rope[:, None, :], (L, n, k_rope.shape[1]))], axis=2)
        q = np.concatenate([np.asarray(q_nope, F64)[hs], q_rot[hs]], axis=1)  # [n, d_h + d_h^R]
        s = np.einsum("lnd,nd->nl", K, q) * scale                           # [n, L]
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        a = e / z
        out["o"].append(np.einsum("nl,lnd->nd", a, vC))
        out["o_latent"].append(a @ c)
        out["lse"].append((m + np.log(z))[:, 0])
        q_abs = np.einsum("ndc,nd->nc", wk, np.asarray(q_nope, F64)[hs])   # (W^UK_i)^T q^C_i
        out["q_abs"].append(np.concatenate([q_abs, q_rot[hs]], axis=1))
    return {k: np.concatenate(v, axis=0) for k, v in out.items()}


def absorbed_decode_seq(c: np.ndarray, k_rope: np.ndarray, q_nope: np.ndarray, q_pe: np.ndarray,
                        pos: int, w_uk: np.ndarray, w_uv: np.ndarray, scale: float,
                        rope_base: float) -> Dict[str, np.ndarray]:
    """The weight-absorbed form, float64; for checking the naive form only.

    Scores read the latent directly through q~_i = (W^UK_i)^T q^C_i; the weighted
    sum stays in latent space and is mapped out by W^UV_i afterwards
    ([两张账] "第一张账"; [V2-解析] 2.2.1.1 absorption remark).
    """
    c = np.asarray(c, F64)
    k_rope = np.asarray(k_rope, F64)
    n_h, d_h = q_nope.shape
    q_rot = rope(q_pe, pos, rope_base)
    o, o_lat, lse, q_abs = [], [], [], []
    for i in range(n_h):
        qt = _head_rows(w_uk, i, d_h).astype(F64).T @ np.asarray(q_nope[i], F64)   # [d_c]
        s = (c @ qt + k_rope @ q_rot[i]) * scale
        m = s.max()
        e = np.exp(s - m)
        z = e.sum()
        ol = (e / z) @ c
        o_lat.append(ol)
        o.append(_head_rows(w_uv, i, d_h).astype(F64) @ ol)
        lse.append(m + np.log(z))
        q_abs.append(np.concatenate([qt, q_rot[i]]))
    return {"o": np.array(o), "o_latent": np.array(o_lat), "lse": np.array(lse),
            "q_abs": np.array(q_abs)}


# ----------------------------------------------------------------------------
# merging attention over disjoint token subsets
# ----------------------------------------------------------------------------
def lse_merge(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Merge per-subset results (o_s normalised within subset s, lse_s) into the whole.

    o_parts [S, ..., d], lse_parts [S, ...].  Softmax over a union of disjoint
    subsets: weight of subset s is exp(lse_s) / sum_t exp(lse_t).
    """
    o_parts = np.asarray(o_parts, F64)
    lse_parts = np.asarray(lse_parts, F64)
    M = lse_parts.max(axis=0)
    w = np.exp(lse_parts - M)
    z = w.sum(axis=0)
    return (w[..., None] * o_parts).sum(axis=0) / z[..., None], M + np.log(z)


# ----------------------------------------------------------------------------
# whole-batch driver over a synthetic workload
# ----------------------------------------------------------------------------
def softmax_scale(d_head: int, d_rope: int) -> float:
    return 1.0 / np.sqrt(d_head + d_rope)


def decode_workload(wl, seqs: Optional[Iterable[int]] = None, heads=None) -> Dict[str, np.ndarray]:
    """Naive fp64 decode of the selected sequences of a synthetic workload.

    `wl` carries: cfg (n_heads, d_head, d_latent, d_rope, page_size, rope_base, dtype),
    cache, block_table, seq_lens, positions, q_nope, q_pe, w_uk, w_uv.
    Returns arrays stacked over the selected sequences.
    """
    cfg = wl.cfg
    bf = cfg.dtype == "bf16"
    seqs = range(cfg.batch) if seqs is None else list(seqs)
    w_uk = to_f64(wl.w_uk, bf)
    w_uv = to_f64(wl.w_uv, bf)
    scale = softmax_scale(cfg.d_head, cfg.d_rope)
    res = {k: [] for k in ("o", "o_latent", "lse", "q_abs")}
    for b in seqs:
        rows = to_f64(gather_rows(wl.cache, wl.block_table[b], int(wl.seq_lens[b]), cfg.page_size), bf)
        r = naive_decode_seq(rows[:, :cfg.d_latent], rows[:, cfg.d_latent:],
                             to_f64(wl.q_nope[b], bf), to_f64(wl.q_pe[b], bf),
                             int(wl.positions[b]), w_uk, w_uv, scale, cfg.rope_base, heads=heads)
        for k in res:
            res[k].append(r[k])
    return {k: np.stack(v) for k, v in res.items()}


def multi_decode_seq(c: np.ndarray, k_rope: np.ndarray, q_nope: np.ndarray, q_pe: np.ndarray,
                     w_uk: np.ndarray, w_uv: np.ndarray, scale: float, rope_base: float,
                     heads: Optional[Iterable[int]] = None) -> Dict[str, np.ndarray]:
    """T query tokens of one sequence whose L cached rows already hold them.

    Query t sits at position p_t = L - T + t and attends causally to tokens
    0 .. p_t (the current token is cached before attention, [两张账] "第一张账";
    a token never attends to later ones).  q_nope [T, n_h, d_h], q_pe
    [T, n_h, d_h^R].  Each token is the single-query naive path over its prefix.
    Returns arrays with a leading T axis.
    """
    L = c.shape[0]
    T = q_nope.shape[0]
    res = {k: [] for k in ("o", "o_latent", "lse", "q_abs")}
    for t in range(T):
        p = L - T + t
        r = naive_decode_seq(c[:p + 1], k_rope[:p + 1], q_nope[t], q_pe[t], p, w_uk, w_uv, scale,
                             rope_base, heads=heads)
        for k in res:
            res[k].append(r[k])
    return {k: np.stack(v) for k, v in res.items()}


def causal_prefill_seq(c: np.ndarray, k_rope: np.ndarray, q_nope: np.ndarray, q_pe: np.ndarray,
                       w_uk: np.ndarray, w_uv: np.ndarray, scale: float, rope_base: float,
                       heads: Optional[Iterable[int]] = None) -> Dict[str, np.ndarray]:
    """multi_decode_seq for many query tokens: the naive path with each head's
    keys and values materialised once for the whole sequence.

    The T newest tokens of a sequence of L cached rows attend causally: token t
    at position p_t = L - T + t sees rows 0 .. p_t ([V2-解析] 2.2.1.2: a query
    sees only the tokens up to its own).  k^C_{j,i} = W^UK_i c_j and
    v^C_{j,i} = W^UV_i c_j ([V2-解析] 2.2.1.1) do not depend on the query, so
    they are formed once; rows after p_t get score -inf.  q_nope [T, n_h, d_h],
    q_pe [T, n_h, d_h^R] (not yet encoded).  Returns o [T, n, d_h],
    o_latent [T, n, d_c], lse [T, n] for the selected heads.
    """
    c = np.asarray(c, F64)
    k_rope = np.asarray(k_rope, F64)
    L, d_c = c.shape
    T, n_h, d_h = q_nope.shape
    heads = list(range(n_h)) if heads is None else list(heads)
    pos = L - T + np.arange(T)                                   # p_t
    visible = np.arange(L)[None, :] <= pos[:, None]             # [T, L]
    out = {k: [] for k in ("o", "o_latent", "lse")}
    for i in heads:
        kC = c @ _head_rows(w_uk, i, d_h).astype(F64).T          # [L, d_h]
        vC = c @ _head_rows(w_uv, i, d_h).astype(F64).T
        K = np.concatenate([kC, k_rope], axis=1)                 # [L, d_h + d_h^R]
        q = np.concatenate([np.asarray(q_nope[:, i], F64),
                            rope(np.asarray(q_pe[:, i], F64), pos, rope_base)], axis=1)   # [T, .]
        s = np.where(visible, (q @ K.T) * scale, -np.inf)         # [T, L]
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        a = e / z
        out["o"].append(a @ vC)
        out["o_latent"].append(a @ c)
        out["lse"].append((m + np.log(z))[:, 0])
    return {"o": np.stack(out["o"], axis=1), "o_latent": np.stack(out["o_latent"], axis=1),
            "lse": np.stack(out["lse"], axis=1)}


def causal_prefill_workload(wl, q_nope: np.ndarray, q_pe: np.ndarray,
                            seqs: Optional[Iterable[int]] = None, heads=None) -> Dict[str, np.ndarray]:
    """causal_prefill_seq over the selected sequences of a workload (inputs as
    for multi_decode_workload)."""
    cfg = wl.cfg
    bf = cfg.dtype == "bf16"
    seqs = range(cfg.batch) if seqs is None else list(seqs)
    w_uk = to_f64(wl.w_uk, bf)
    w_uv = to_f64(wl.w_uv, bf)
    scale = softmax_scale(cfg.d_head, cfg.d_rope)
    res = {k: [] for k in ("o", "o_latent", "lse")}
    for b in seqs:
        rows = to_f64(gather_rows(wl.cache, wl.block_table[b], int(wl.seq_lens[b]), cfg.page_size), bf)
        r = causal_prefill_seq(rows[:, :cfg.d_latent], rows[:, cfg.d_latent:], to_f64(q_nope[b], bf),
                               to_f64(q_pe[b], bf), w_uk, w_uv, scale, cfg.rope_base, heads=heads)
        for k in res:
            res[k].append(r[k])
    return {k: np.stack(v) for k, v in res.items()}


def multi_decode_workload(wl, q_nope: np.ndarray, q_pe: np.ndarray,
                          seqs: Optional[Iterable[int]] = None, heads=None) -> Dict[str, np.ndarray]:
    """multi_decode_seq over the selected sequences of a workload; q_nope
    [B, T, n_h, d_h] and q_pe [B, T, n_h, d_h^R] in the workload's storage type."""
    cfg = wl.cfg
    bf = cfg.dtype == "bf16"
    seqs = range(cfg.batch) if seqs is None else list(seqs)
    w_uk = to_f64(wl.w_uk, bf)
    w_uv = to_f64(wl.w_uv, bf)
    scale = softmax_scale(cfg.d_head, cfg.d_rope)
    res = {k: [] for k in ("o", "o_latent", "lse", "q_abs")}
    for b in seqs:
        rows = to_f64(gather_rows(wl.cache, wl.block_table[b], int(wl.seq_lens[b]), cfg.page_size), bf)
        r = multi_decode_seq(rows[:, :cfg.d_latent], rows[:, cfg.d_latent:], to_f64(q_nope[b], bf),
                             to_f64(q_pe[b], bf), w_uk, w_uv, scale, cfg.rope_base, heads=heads)
        for k in res:
            res[k].append(r[k])
    return {k: np.stack(v) for k, v in res.items()}


# ----------------------------------------------------------------------------
# deriving the cache and the query from hidden states (the full recipe)
# ----------------------------------------------------------------------------
def cache_rows_from_hidden(h: np.ndarray, w_dkv: np.ndarray, w_kr: np.ndarray,
                           positions: np.ndarray, rope_base: float,
                           rms_norm: bool, eps: float = 1e-6) -> np.ndarray:
    """Cached rows [c^KV_t | RoPE_t(W^KR h_t)] for hidden states h [T, d_model].

    c^KV_t = W^DKV h_t ([V2-解析] 2.2.1.1), optionally RMS-normalised (no gain);
    the key's RoPE part is encoded at its own position before caching
    ([V2-解析] 2.2.2).
    """
    h = np.asarray(h, F64)
    c = h @ np.asarray(w_dkv, F64).T
    if rms_norm:
        c = c / np.sqrt((c * c).mean(axis=1, keepdims=True) + eps)
    kr = rope(h @ np.asarray(w_kr, F64).T, np.asarray(positions), rope_base)
    return np.concatenate([c, kr], axis=1)


def query_from_hidden(h_t: np.ndarray, w_q: np.ndarray, w_qr: np.ndarray, n_heads: int):
    """q^C_i and the (not yet encoded) q^R_i of one token without query compression.

    W^Q [n_h d_h, d_model] and W^QR [n_h d_h^R, d_model] map column vectors;
    head i owns rows i*d_h .. i*d_h + d_h - 1 (and i*d_h^R .. of W^QR), the
    same convention as W^UK ([V2-解析] 2.2.1.1, per-head up-projection).
    """
    h_t = np.asarray(h_t, F64)
    qn = (np.asarray(w_q, F64) @ h_t).reshape(n_heads, -1)
    qp = (np.asarray(w_qr, F64) @ h_t).reshape(n_heads, -1)
    return qn, qp


def query_from_latent(h_t: np.ndarray, w_dq: np.ndarray, w_uq: np.ndarray, w_qr: np.ndarray,
                      n_heads: int):
    """q^C_i and the (not yet encoded) q^R_i of one token with query compression.

    The query is compressed like the keys and values, down and then up
    ([V2-解析] 2.2.1.2): c^Q = W^DQ h_t, q^C = W^UQ c^Q ([V2-解析] 2.2.2, the
    absorbed score written with W^UQ c^Q).  The decoupled per-head q^R is read
    from the same compressed latent, q^R = W^QR c^Q (the pages' formula for
    it is lost; this is the reading that keeps the whole query on the
    compressed path).  W^DQ [d_cq, d_model], W^UQ [n_h d_h, d_cq],
    W^QR [n_h d_h^R, d_cq]; no normalisation of c^Q (the pages name none).
    """
    c_q = np.asarray(w_dq, F64) @ np.asarray(h_t, F64)
    qn = (np.asarray(w_uq, F64) @ c_q).reshape(n_heads, -1)
    qp = (np.asarray(w_qr, F64) @ c_q).reshape(n_heads, -1)
    return qn, qp
