"""Decode workloads of the MLA latent-cache path, as plain data.

Shapes follow the DeepSeek-V2 pages:
  * V2-Lite (page "DeepSeek V2 技术解析", part 2 intro): 16 heads of 128,
    KV compression dimension 512, decoupled query/key head dimension 64,
    hidden size 2048, no query compression.
  * V2: d_c = 4 d_h and d_h^R = d_h / 2 (page "DeepSeek-V2/V3：大模型的两张账",
    section "RoPE 是压缩链路里那块不能随便移动的石头"); 128K context
    (page "DeepSeek V2 技术解析", part 2 intro).
The V2 head count (128), model width (5120) and query latent (1536) are not
on the pages; they are fixed by the workload definitions used here.

Nothing in this module computes anything of the method.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

PAGE_SIZE = 64


@dataclass(frozen=True)
class MLAConfig:
    name: str
    n_heads: int
    d_head: int
    d_latent: int
    d_rope: int
    d_model: int
    batch: int
    dtype: str                      # "f32" or "bf16": storage of every input
    seq_len: Optional[int] = None   # all sequences this long, or
    len_range: Optional[Tuple[int, int]] = None  # uniform draw, both ends inclusive
    len_seed: int = 2
    q_latent: Optional[int] = None  # query compression width (shape note only)
    rms_norm_latent: bool = True    # the cached latent is RMS-normalised
    permute_pages: bool = False
    page_seed: int = 1
    page_size: int = PAGE_SIZE
    rope_base: float = 10000.0
    value_seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def d_qk(self) -> int:
        """Width of one cached token row and of an absorbed query: d_c + d_h^R."""
        return self.d_latent + self.d_rope


TINY = MLAConfig(
    name="tiny_f32", n_heads=4, d_head=16, d_latent=64, d_rope=8, d_model=128,
    batch=1, dtype="f32", seq_len=37, rms_norm_latent=False,
    note="tiny fp32 step: 37 cached tokens at positions 0..36")

V2_LITE = MLAConfig(
    name="v2lite_b32_l4096", n_heads=16, d_head=128, d_latent=512, d_rope=64,
    d_model=2048, batch=32, dtype="bf16", seq_len=4096,
    note="V2-Lite-shaped decode, contiguous block table")

V2 = MLAConfig(
    name="v2_b64_l8192", n_heads=128, d_head=128, d_latent=512, d_rope=64,
    d_model=5120, q_latent=1536, batch=64, dtype="bf16", seq_len=8192,
    permute_pages=True,
    note="V2-shaped decode, permuted block table (headline workload)")

V2_VARLEN = MLAConfig(
    name="v2_varlen_b128", n_heads=128, d_head=128, d_latent=512, d_rope=64,
    d_model=5120, q_latent=1536, batch=128, dtype="bf16", len_range=(1, 32768),
    permute_pages=True,
    note="V2-shaped variable-length batch, lengths uniform in [1, 32768]")

V2_128K = MLAConfig(
    name="v2_b8_l131072", n_heads=128, d_head=128, d_latent=512, d_rope=64,
    d_model=5120, q_latent=1536, batch=8, dtype="bf16", seq_len=131072,
    permute_pages=True,
    note="V2-shaped 128K-context decode")

CONFIGS = {c.name: c for c in (TINY, V2_LITE, V2, V2_VARLEN, V2_128K)}
ORDERED = [TINY, V2_LITE, V2, V2_VARLEN, V2_128K]


def small(base: MLAConfig, name: str, batch: int, lens=None, **kw) -> MLAConfig:
    """A reduced-size variant of `base` for quick parity cases.

    `lens` may be an int (all equal) or a (lo, hi) range drawn like the
    variable-length workload.
    """
    d = dict(base.__dict__)
    d.update(name=name, batch=batch, note=f"reduced {base.name}")
    if isinstance(lens, int):
        d.update(seq_len=lens, len_range=None)
    elif lens is not None:
        d.update(seq_len=None, len_range=tuple(lens))
    d.update(kw)
    return MLAConfig(**d)
