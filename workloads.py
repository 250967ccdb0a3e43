"""Seeded synthetic workloads for varlen attention: shapes, packing and random inputs.

This module is shared by the tests, the bench and the smoke check. It holds only
workload shapes and the seeded random draw; it contains none of the attention
arithmetic, so the CPU oracle and the GPU path can both take inputs from it
without sharing any of the computation.

Sources for the shapes (page titles and sections):
  * "FA2 vs NATTEN on A100: 3.5-4.8x perf gap" (cosmos-framework issue), benchmark
    script: one packed sequence per call, cumulative seqlens ``[0, n]`` as int32,
    32 query heads / 8 KV heads, head_dim 128, bf16 ``randn`` inputs drawn q, k, v
    in that order from a generator seeded 0, and a ``randn`` output gradient.
  * "[FA4/B200] return_lse=True makes D64 forward about 19% faster", repro script:
    shape (2, 16384, 16, 64) bf16, seed 0, timed with and without the LSE output.
  * "FA4 head_dim=256 B200 Regression Check", Environment: head_dim = head_dim_v =
    256, 8 query heads with 1 KV head (ratio 8) or MHA, batch derived from a total
    of 32K tokens (8x4K, 2x16K, 1x32K, plus longer single sequences).

Reading used here (the pages draw on the GPU with a device generator; this module
draws on the CPU so that the oracle and the GPU consume identical bits):
  ``g = torch.Generator().manual_seed(seed)``; q, k, v, dout are drawn in that
  order with ``torch.randn(shape, dtype=float32, generator=g)`` and rounded to
  bf16. Shapes: q, dout ``(total_q, n_q_heads, head_dim)``; k, v
  ``(total_k, n_kv_heads, head_dim)``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np
import torch

# Document lengths of the 16384-token packed training batch: lengths drawn with
# numpy.random.default_rng(0).integers(256, 4097) until their sum reaches 16384,
# the last one truncated to fill. Written out because numpy does not promise that
# its streams stay stable across releases.
PACKED_16K_DOC_LENGTHS = [3523, 2702, 2219, 1292, 1438, 413, 544, 319, 929, 3005]


def packed_doc_lengths(total: int = 16384, lo: int = 256, hi: int = 4096, seed: int = 0) -> List[int]:
    """Draw document lengths uniformly from [lo, hi] until they fill ``total``; truncate the last."""
    rng = np.random.default_rng(seed)
    lengths: List[int] = []
    acc = 0
    while acc < total:
        x = int(rng.integers(lo, hi + 1))
        lengths.append(x)
        acc += x
    lengths[-1] -= acc - total
    return lengths


def cu_from_lengths(lengths) -> List[int]:
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return cu


@dataclass
class Workload:
    """One attention problem: packing, heads, head_dim and masking."""

    name: str
    seqlens_q: List[int]
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    causal: bool
    seqlens_k: Optional[List[int]] = None
    backward: bool = True
    seed: int = 0
    notes: str = ""
    softmax_scale: Optional[float] = None
    # local attention band (left, right) around the bottom-right diagonal; None or
    # a negative side: unbounded on that side
    window: Optional[Tuple[int, int]] = None

    def __post_init__(self):
        if self.seqlens_k is None:
            self.seqlens_k = list(self.seqlens_q)
        if self.softmax_scale is None:
            self.softmax_scale = float(self.head_dim) ** -0.5

    @property
    def cu_seqlens_q(self) -> List[int]:
        return cu_from_lengths(self.seqlens_q)

    @property
    def cu_seqlens_k(self) -> List[int]:
        return cu_from_lengths(self.seqlens_k)

    @property
    def total_q(self) -> int:
        return sum(self.seqlens_q)

    @property
    def total_k(self) -> int:
        return sum(self.seqlens_k)

    @property
    def max_seqlen_q(self) -> int:
        return max(self.seqlens_q) if self.seqlens_q else 0

    @property
    def max_seqlen_k(self) -> int:
        return max(self.seqlens_k) if self.seqlens_k else 0

    def accounted_fwd_flop(self) -> float:
        """Forward work as the pages count it: 4 * sum_b Lq_b * Lk_b * Hq * D, halved when causal."""
        f = 4.0 * sum(a * b for a, b in zip(self.seqlens_q, self.seqlens_k)) * self.n_q_heads * self.head_dim
        return f * (0.5 if self.causal else 1.0)

    def accounted_fwdbwd_flop(self) -> float:
        """Forward+backward work as the pages count it: 3.5 x the forward."""
        return 3.5 * self.accounted_fwd_flop()

    def describe(self) -> dict:
        return {
            "workload": self.name,
            "seqlens": _compact(self.seqlens_q),
            "n_q_heads": self.n_q_heads,
            "n_kv_heads": self.n_kv_heads,
            "head_dim": self.head_dim,
            "causal": self.causal,
            "total_tokens": self.total_q,
            **({"window": list(self.window)} if self.window is not None else {}),
        }


def _compact(lengths):
    if len(set(lengths)) == 1 and len(lengths) > 1:
        return f"{len(lengths)}x{lengths[0]}"
    return list(lengths)


def make_inputs(wl: Workload, with_dout: bool = True, seed: Optional[int] = None):
    """Seeded bf16 CPU tensors q, k, v (and dout) for a workload, plus int32 cu_seqlens.

    Returns a dict of CPU tensors. The caller moves them to the GPU (same bits) or
    converts them to float64 for the oracle (bf16 -> float64 is exact).
    """
    g = torch.Generator().manual_seed(wl.seed if seed is None else seed)
    D = wl.head_dim
    q = torch.randn((wl.total_q, wl.n_q_heads, D), dtype=torch.float32, generator=g).to(torch.bfloat16)
    k = torch.randn((wl.total_k, wl.n_kv_heads, D), dtype=torch.float32, generator=g).to(torch.bfloat16)
    v = torch.randn((wl.total_k, wl.n_kv_heads, D), dtype=torch.float32, generator=g).to(torch.bfloat16)
    out = {
        "q": q,
        "k": k,
        "v": v,
        "cu_seqlens_q": torch.tensor(wl.cu_seqlens_q, dtype=torch.int32),
        "cu_seqlens_k": torch.tensor(wl.cu_seqlens_k, dtype=torch.int32),
    }
    if with_dout:
        out["dout"] = torch.randn((wl.total_q, wl.n_q_heads, D), dtype=torch.float32, generator=g).to(torch.bfloat16)
    return out


def inputs_sha256(inp) -> str:
    """Checksum of a workload's drawn inputs (q, k, v, dout and the packing), so
    that values stored for them can be checked against the inputs in use."""
    import hashlib

    h = hashlib.sha256()
    for name in ("cu_seqlens_q", "cu_seqlens_k", "q", "k", "v", "dout"):
        if name in inp:
            t = inp[name].contiguous()
            h.update(name.encode())
            h.update(str(tuple(t.shape)).encode())
            h.update(t.view(torch.int16).numpy().tobytes() if t.dtype == torch.bfloat16 else t.numpy().tobytes())
    return h.hexdigest()


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact bf16 -> float64 numpy conversion."""
    return t.to(torch.float64).numpy()


# ---------------------------------------------------------------------------
# The five workload families
# ---------------------------------------------------------------------------

def tiny(causal: bool) -> Workload:
    """Two packed sequences (200, 312), 4 Q / 2 KV heads, head_dim 64, seed 0."""
    return Workload(f"tiny-varlen-gqa-d64-{'causal' if causal else 'full'}", [200, 312], 4, 2, 64, causal)


def a100_shape(n: int = 4096) -> Workload:
    """One packed sequence of n tokens, 32 Q / 8 KV heads, head_dim 128, non-causal."""
    return Workload(f"single-{n}-gqa32/8-d128-full", [n], 32, 8, 128, False)


def packed_16k() -> Workload:
    """16384 tokens of documents with lengths in [256, 4096], causal per document, 32/8 heads, hd128."""
    return Workload("packed16k-docs-gqa32/8-d128-causal", list(PACKED_16K_DOC_LENGTHS), 32, 8, 128, True)


def long_65k() -> Workload:
    """One causal sequence of 65536 tokens, 32/8 heads, hd128."""
    return Workload("single-65536-gqa32/8-d128-causal", [65536], 32, 8, 128, True)


def single_16k_full() -> Workload:
    """One non-causal sequence of 16384 tokens, 32/8 heads, hd128 (the A100 table's 16K row)."""
    return Workload("single-16384-gqa32/8-d128-full", [16384], 32, 8, 128, False)


def hd64_mha() -> Workload:
    """Two sequences of 16384 tokens, 16 = 16 heads, head_dim 64, non-causal, forward only."""
    return Workload("2x16384-mha16-d64-full", [16384, 16384], 16, 16, 64, False, backward=False)


def hd256_gqa(batch: int, seqlen: int, causal: bool) -> Workload:
    """head_dim 256, 8 Q heads / 1 KV head, batch x seqlen tokens."""
    return Workload(f"{batch}x{seqlen}-gqa8/1-d256-{'causal' if causal else 'full'}",
                    [seqlen] * batch, 8, 1, 256, causal)


def all_configs() -> List[Workload]:
    """Every workload of the five families, including the long single sequences."""
    out = [tiny(False), tiny(True), a100_shape(4096), packed_16k(), long_65k(), hd64_mha()]
    for b, s in ((8, 4096), (2, 16384), (1, 32768), (1, 131072)):
        for c in (False, True):
            out.append(hd256_gqa(b, s, c))
    return out
