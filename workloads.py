"""Seeded synthetic attention inputs, shared by the tests, the smoke check and the benchmark.

This module draws random numbers and rounds them to the storage dtype; it holds
none of the attention arithmetic, so both the GPU path's callers and the CPU
oracle's callers can use it without sharing any of the computation.

Each workload is a forward-attention problem [B, H, N, d]:
  q, k, v ~ iid N(0, 1) drawn in fp32 from a CPU torch.Generator seeded with
  the workload's seed, in the order q, k, v; q and k are multiplied by
  ``sigma_qk`` (4 for the wide-logit case); then each is rounded to fp16 or
  bf16 (round to nearest even). The sizing follows the pages' own example
  ("Decoding flash attention", bibekananda.in: N = 8192 tokens, head dim 128,
  fp16) and the head counts / lengths listed below.
  ``scale`` is the fp32 value of 1/sqrt(d).
  For the large problems parity is checked on a sampled subset of query rows:
  per (b, h), in order, a generator seeded with ``seed + 1000`` draws
  randperm(N)[:rows_per_head]; rows 0 and N-1 are forced in (replacing the last
  draws if absent) and the set is sorted.

The backward pass of a workload also needs the upstream gradient dout = dL/do:
iid N(0, 1) in fp32 from a generator seeded with ``seed + 2000``, rounded to the
workload's dtype. Its parity checks on the large problems cover a seeded subset
of heads (``sample_heads``, generator ``seed + 3000``) and, within them, the
sampled query rows (for dq) and the same number of sampled keys (for dk, dv;
``sample_rows`` with generator ``seed + 4000``).
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "f16" or "bf16"
    causal: bool
    sigma_qk: float
    seed: int
    rows_per_head: Optional[int]   # None: every row is checked

    @property
    def torch_dtype(self):
        return torch.float16 if self.dtype == "f16" else torch.bfloat16

    @property
    def scale(self) -> float:
        """fp32 value of 1/sqrt(d), returned as a Python float (exact)."""
        return float(np.float32(1.0 / np.sqrt(self.d)))

    def flops(self) -> float:
        """Conventional forward flop count 4*B*H*N^2*d, halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f


WORKLOADS = [
    Workload("B1-H1-N256-d64-f16", 1, 1, 256, 64, "f16", False, 1.0, 1, None),
    Workload("B4-H16-N2047-d64-bf16", 4, 16, 2047, 64, "bf16", False, 1.0, 2, None),
    Workload("B1-H32-N8192-d128-f16", 1, 32, 8192, 128, "f16", False, 1.0, 3, 1024),
    Workload("B2-H16-N8192-d128-bf16-causal", 2, 16, 8192, 128, "bf16", True, 1.0, 4, 1024),
    Workload("B1-H8-N32768-d128-bf16-causal-qk4", 1, 8, 32768, 128, "bf16", True, 4.0, 5, 1024),
]

# A thin grid for split-KV: 2 heads x 64 query tiles of 256 rows leave half of the 256 compute
# units idle under the plain grid (same recipe; not one of the five parity configurations).
THIN = Workload("B1-H2-N16384-d128-f16", 1, 2, 16384, 128, "f16", False, 1.0, 6, 1024)

BY_NAME = {w.name: w for w in WORKLOADS + [THIN]}

# The configuration the headline throughput is quoted on.
HEADLINE = BY_NAME["B1-H32-N8192-d128-f16"]


def make_inputs(w: Workload):
    """(q, k, v) as CPU tensors [B, H, N, d] of the workload's dtype."""
    g = torch.Generator(device="cpu").manual_seed(w.seed)
    shape = (w.B, w.H, w.N, w.d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    if w.sigma_qk != 1.0:
        q = q * w.sigma_qk
        k = k * w.sigma_qk
    return q.to(w.torch_dtype), k.to(w.torch_dtype), v.to(w.torch_dtype)


def custom_inputs(B, H, N, d, dtype, seed, sigma_qk=1.0):
    """Same recipe as ``make_inputs`` for an arbitrary shape (tests of edge sizes)."""
    w = Workload("custom", B, H, N, d, dtype, False, sigma_qk, seed, None)
    return make_inputs(w)


def sample_rows(w: Workload, rows_per_head: int = None):
    """int64 array [B*H, R] of query rows to check (R = the workload's rows_per_head, or the given
    count), or None for every row."""
    r = w.rows_per_head if rows_per_head is None else rows_per_head
    if r is None or r >= w.N:
        return None
    g = torch.Generator(device="cpu").manual_seed(w.seed + 1000)
    out = np.empty((w.B * w.H, r), dtype=np.int64)
    for bh in range(w.B * w.H):
        rows = torch.randperm(w.N, generator=g)[:r].numpy().copy()
        if not (rows == 0).any():
            rows[r - 1] = 0
        if not (rows == w.N - 1).any():
            rows[r - 2 if rows[r - 1] == 0 else r - 1] = w.N - 1
        out[bh] = np.sort(rows)
    return out


def make_dout(w: Workload):
    """The upstream gradient dout [B, H, N, d] (CPU tensor of the workload's dtype)."""
    g = torch.Generator(device="cpu").manual_seed(w.seed + 2000)
    return torch.randn((w.B, w.H, w.N, w.d), generator=g, dtype=torch.float32).to(w.torch_dtype)


def sample_heads(w: Workload, count: int):
    """Sorted flat (b * H + h) indices of `count` heads drawn without replacement."""
    n = w.B * w.H
    if count >= n:
        return np.arange(n, dtype=np.int64)
    g = torch.Generator(device="cpu").manual_seed(w.seed + 3000)
    return np.sort(torch.randperm(n, generator=g)[:count].numpy().astype(np.int64))


def sample_keys(w: Workload):
    """int64 array [B*H, R] of keys to check (same recipe as sample_rows, its own generator)."""
    if w.rows_per_head is None or w.rows_per_head >= w.N:
        return None
    shifted = Workload(w.name, w.B, w.H, w.N, w.d, w.dtype, w.causal, w.sigma_qk, w.seed + 3000,
                       w.rows_per_head)
    return sample_rows(shifted)


def make_block_mask(w: Workload, block: int, density: float):
    """A seeded random block mask [ceil(N/block), ceil(N/block)] (uint8 numpy array) for
    block-sparse attention over the workload: each (query block, key block) byte is 1 with
    probability ``density`` (generator seeded with ``seed + 5000``), and the diagonal blocks are
    always 1 so that every row keeps its own key."""
    n = -(-w.N // block)
    g = torch.Generator(device="cpu").manual_seed(w.seed + 5000)
    m = (torch.rand((n, n), generator=g, dtype=torch.float64) < density).numpy().astype(np.uint8)
    np.fill_diagonal(m, 1)
    return m


def block_mask_pairs(mask, N: int, block_q: int, block_k: int) -> int:
    """Number of (query row, key) pairs a [n_qb, n_kb] block mask allows over N rows and keys."""
    rows = np.minimum(N, (np.arange(mask.shape[0]) + 1) * block_q) - np.arange(mask.shape[0]) * block_q
    keys = np.minimum(N, (np.arange(mask.shape[1]) + 1) * block_k) - np.arange(mask.shape[1]) * block_k
    return int((rows[:, None] * keys[None, :] * (np.asarray(mask) != 0)).sum())
