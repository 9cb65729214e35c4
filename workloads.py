"""Seeded synthetic inputs for the attention workloads.

This module only draws random tensors; it holds none of the attention
arithmetic.  Both the GPU tests/bench and the oracle read the same host bf16
tensors produced here.

Recipe (all draws from one ``torch.Generator`` on the CPU seeded with
``seed``, fp32 ``randn`` then a round-to-nearest-even cast to bf16):

* prefill workloads draw Q, then K, then V, each [B, heads, N, d] ~ N(0, 1);
* ``k_bias_std``: a per-channel bias vector b in R^d ~ N(0, k_bias_std^2),
  shared by every token, batch and head, is drawn after K and added to K in
  fp32 before the cast (exercises Smooth-K); V is drawn after the bias;
* ``outlier_frac``: round(outlier_frac * B*Hkv*N) rows of K (flattened row
  index, drawn without replacement after K) are multiplied by
  ``outlier_mult`` in fp32 before the cast; V is drawn afterwards;
* decode draws the per-sequence lengths (uniform integers in [len_lo, len_hi]),
  then q [B, H, d], then the valid K rows batch by batch ([Hkv, L_b, d] each),
  then the valid V rows the same way; cache positions at or beyond L_b hold
  bf16 NaN so that any over-read shows up in the output;
* a packed variable-length batch draws its lengths (uniform integers in
  [len_lo, len_hi], generator seeded with ``seed``), then Q, K and V over all
  packed tokens, token-major ([total, heads, d]), from a generator seeded with
  ``seed + 1``;
* paged decode takes those caches and spreads their pages over a pool in a
  random order (its own generator, seeded separately); unused pool pages and
  the rows of a last page past L_b hold NaN.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "prefill" | "decode"
    B: int
    H: int
    Hkv: int
    N: int
    d: int
    causal: bool = False
    mode: str = "exact"  # "exact" | "sage"
    out_dtype: str = "bf16"  # "bf16" | "fp32"
    k_bias_std: float = 0.0
    outlier_frac: float = 0.0
    outlier_mult: float = 20.0
    len_lo: int = 0
    len_hi: int = 0
    split_tokens: int = 512
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def flops(self, seqlens=None) -> float:
        """Algorithmic FLOPs: 4*B*H*Nq*Nk*d, half of it under a causal mask.

        For decode the count is 4*H*d*sum(L_b).  Masked-tile waste and
        quantisation prologues are not counted.
        """
        if self.kind == "decode":
            total = int(np.sum(seqlens)) if seqlens is not None else self.B * self.N
            return 4.0 * self.H * self.d * total
        if self.kind == "varlen":
            sq = float(np.sum(np.asarray(seqlens, dtype=np.float64) ** 2))
            f = 4.0 * self.H * sq * self.d
            return f / 2 if self.causal else f
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f


WORKLOADS = {
    "tiny_exact": Workload("tiny_exact", "prefill", 1, 2, 2, 256, 64, causal=False,
                           out_dtype="fp32"),
    "llm_prefill": Workload("llm_prefill", "prefill", 4, 32, 32, 4096, 128, causal=True),
    "sage_prefill": Workload("sage_prefill", "prefill", 2, 24, 24, 16384, 128, causal=False,
                             mode="sage", k_bias_std=3.0),
    "gqa_decode": Workload("gqa_decode", "decode", 64, 32, 8, 32768, 128, len_lo=1024,
                           len_hi=32768, split_tokens=512),
    "long_prefill": Workload("long_prefill", "prefill", 1, 16, 16, 65536, 128, causal=True,
                             outlier_frac=0.001, outlier_mult=20.0),
    # packed batch of 8 sequences, lengths uniform on [256, 4096] (N = the bound)
    "varlen_prefill": Workload("varlen_prefill", "varlen", 8, 32, 32, 4096, 128, causal=True,
                               len_lo=256, len_hi=4096),
}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def make_prefill(B, H, Hkv, N, d, *, seed=0, k_bias_std=0.0, outlier_frac=0.0,
                 outlier_mult=20.0):
    """Q [B,H,N,d], K/V [B,Hkv,N,d] bf16 on the CPU, drawn as the module doc says."""
    g = _gen(seed)
    q = torch.randn((B, H, N, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn((B, Hkv, N, d), generator=g, dtype=torch.float32)
    info = {}
    if k_bias_std:
        bias = torch.randn((d,), generator=g, dtype=torch.float32) * k_bias_std
        k += bias
        info["k_bias"] = bias
    if outlier_frac:
        n_out = int(round(outlier_frac * B * Hkv * N))
        idx = torch.randperm(B * Hkv * N, generator=g)[:n_out]
        k.view(B * Hkv * N, d)[idx] *= outlier_mult
        info["outlier_rows"] = torch.sort(idx).values
    k = k.to(torch.bfloat16)
    v = torch.randn((B, Hkv, N, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    return q, k, v, info


def make_decode(B, H, Hkv, N_max, d, *, len_lo, len_hi, seed=0):
    """q [B,H,d], K/V caches [B,Hkv,N_max,d] bf16 with NaN beyond each length,
    seqlens int32 [B]."""
    g = _gen(seed)
    seqlens = torch.randint(len_lo, len_hi + 1, (B,), generator=g, dtype=torch.int64)
    q = torch.randn((B, H, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    nan = torch.tensor(float("nan"), dtype=torch.bfloat16)
    caches = []
    for _ in range(2):
        c = torch.empty((B, Hkv, N_max, d), dtype=torch.bfloat16)
        for b in range(B):
            L = int(seqlens[b])
            c[b, :, :L] = torch.randn((Hkv, L, d), generator=g,
                                      dtype=torch.float32).to(torch.bfloat16)
            c[b, :, L:] = nan
        caches.append(c)
    return q, caches[0], caches[1], seqlens.to(torch.int32)


def make_page_table(seqlens, page_size: int, *, seed=0, spare_pages=0, max_pages=None):
    """A paged-cache page table: every page of every sequence gets a distinct
    pool page, in a random order (``torch.randperm`` on a generator seeded with
    ``seed``), and ``spare_pages`` pool pages stay unused.  Returns
    (table int32 [B, max_pages] with -1 past each sequence's pages, num_pages).
    """
    seqlens = [int(x) for x in seqlens]
    need = [(L + page_size - 1) // page_size for L in seqlens]
    if max_pages is None:
        max_pages = max(need)
    total = sum(need)
    num_pages = total + spare_pages
    perm = torch.randperm(num_pages, generator=_gen(seed))[:total].to(torch.int32)
    table = torch.full((len(seqlens), max_pages), -1, dtype=torch.int32)
    i = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[i:i + n]
        i += n
    return table, num_pages


def paginate(cache, table, num_pages: int, page_size: int):
    """Copy contiguous caches [B, Hkv, N_max, d] into a page pool
    [num_pages, Hkv, page_size, d] laid out by ``table`` (unused pool pages
    hold NaN).  Works on CPU or GPU tensors; N_max must be a multiple of
    page_size and table must have N_max / page_size columns."""
    B, Hkv, N_max, d = cache.shape
    if N_max % page_size or table.shape != (B, N_max // page_size):
        raise ValueError("cache length, page size and table do not agree")
    pool = torch.full((num_pages, Hkv, page_size, d), float("nan"), dtype=cache.dtype,
                      device=cache.device)
    pages = cache.view(B, Hkv, N_max // page_size, page_size, d).transpose(1, 2)
    t = table.to(cache.device, torch.int64)
    used = t >= 0
    pool[t[used]] = pages[used]
    return pool


def make_varlen(lengths, H, Hkv, d, *, seed=0):
    """A packed batch: q [total,H,d], k/v [total,Hkv,d] bf16 (token-major) and
    cu_seqlens int32 [B+1], for the given sequence lengths; Q, then K, then V
    ~ N(0, 1) over all packed tokens."""
    lengths = [int(x) for x in lengths]
    cu = torch.tensor([0] + list(np.cumsum(lengths)), dtype=torch.int32)
    T = int(cu[-1])
    g = _gen(seed)
    q = torch.randn((T, H, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn((T, Hkv, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((T, Hkv, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    return q, k, v, cu


def make(w: Workload):
    """Inputs of a named workload (CPU tensors)."""
    if w.kind == "varlen":
        lengths = torch.randint(w.len_lo, w.len_hi + 1, (w.B,), generator=_gen(w.seed))
        q, k, v, cu = make_varlen(lengths.tolist(), w.H, w.Hkv, w.d, seed=w.seed + 1)
        return dict(q=q, k=k, v=v, cu_seqlens=cu, seqlens=lengths.to(torch.int32))
    if w.kind == "decode":
        q, k, v, seqlens = make_decode(w.B, w.H, w.Hkv, w.N, w.d, len_lo=w.len_lo,
                                       len_hi=w.len_hi, seed=w.seed)
        return dict(q=q, k=k, v=v, seqlens=seqlens)
    q, k, v, info = make_prefill(w.B, w.H, w.Hkv, w.N, w.d, seed=w.seed,
                                 k_bias_std=w.k_bias_std, outlier_frac=w.outlier_frac,
                                 outlier_mult=w.outlier_mult)
    return dict(q=q, k=k, v=v, **info)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """View a CPU bf16 tensor as its uint16 bit patterns (no copy of values)."""
    if t.dtype != torch.bfloat16:
        raise TypeError("expected a bf16 tensor")
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def sample_rows(B, H, N, *, n_random=4096, seed=1234, whole_slices=((0, 0),),
                special=(0, 1, 63, 64, 127, 128), extra_rows=()):
    """Flattened (b*H + h)*N + i row indices of a declared comparison sample:
    whole (b, h) slices, a set of special rows of every slice (tile edges and
    the last row), seeded random rows, and any extra rows given."""
    rows = set()
    for (b, h) in whole_slices:
        base = (b * H + h) * N
        rows.update(range(base, base + N))
    spec = sorted({i for i in special if 0 <= i < N} | {N - 1})
    for bh in range(B * H):
        rows.update(bh * N + i for i in spec)
    rng = np.random.default_rng(seed)
    if n_random:
        rows.update(int(x) for x in rng.integers(0, B * H * N, size=n_random))
    rows.update(int(r) for r in extra_rows)
    return np.array(sorted(rows), dtype=np.int64)
