"""Seeded synthetic workloads for packed variable-length attention.

This module is the only code shared by the oracle side (``oracle/``) and the
HIP side (the ``variable_length_packed_pack_amd`` package): it draws sequence
lengths and Q/K/V values and nothing else.  It holds none of the method's
arithmetic (no prefix sums, no tiling, no attention).

Recipes (numpy PCG64 ``default_rng``; lengths use seed ``1000 + k`` and Q/K/V
use seed ``2000 + k`` for workload ``k``):

1. tiny      -- 8 sequences, lengths uniform in [1, 64] with one forced to 1;
                fp32, 2 heads x 16, non-causal.  Stands in for the worked
                example of "gigl.nn.packed_attention" (section "Example").
2. graph     -- 512 sequences, lengths clip(rint(lognormal(ln 80, 0.6)), 1,
                256) (about 90 real tokens out of 256); fp32, 8 heads x 64,
                non-causal; also run with one query per sequence.  Stands in
                for the graph-transformer batches of "gigl.nn.packed_attention"
                (the section explaining why the packed path exists, and
                "Results").  The graph data itself is not available.
3. encoder   -- 128 sequences, lengths clip(rint(gamma(2, 75)), 8, 384);
                bf16, 12 heads x 64 (BERT-Base heads), non-causal.  Stands in
                for an IMDB-like random batch ("DanLing NestedTensor",
                section 4 and Appendix C).  IMDB is not available.
4. zipf      -- 65,536 tokens over 64 sequences with Zipf (s = 1) lengths in a
                random rank permutation, each >= 1, summing exactly to 65,536;
                bf16, 16 heads x 128, causal.  The Zipf token split of "So you
                wanna CUDA Graph" (section "Hello World"), with exponent 1.
5. skewed    -- 255 sequences uniform in [64, 256] followed by one sequence
                of 32,768 tokens (placed last); bf16, 32 heads x 128, causal,
                Q/K/V with standard deviation 0.5.
6. cross     -- cross-attention at scale: the key lengths of workload 4 (the
                Zipf split of 65,536 keys over 64 sequences) with ceil(len/4)
                queries per sequence (16,408 queries); bf16, 16 heads x 128,
                non-causal ("DanLing NestedTensor" 3.3: query and key lengths
                may differ).

Q, K and V are drawn together as float32 standard normals of shape
``[T, H, D]`` in the order q, k, v, scaled (workload 5 only), then rounded to
the workload dtype with round-to-nearest-even (``torch.Tensor.to``).  Both the
oracle and the GPU consume the rounded values.

For gradient checks, the output gradient dO ``[T, H, D]`` is a separate
float32 standard-normal draw with seed ``3000 + k``, rounded the same way.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

LENGTH_SEED_BASE = 1000
VALUE_SEED_BASE = 2000
GRAD_SEED_BASE = 3000

DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass
class Workload:
    """One seeded packed batch, held on the host."""

    name: str
    index: int
    dtype: str               # "fp32" | "fp16" | "bf16"
    heads: int
    head_dim: int
    causal: bool
    lengths: np.ndarray      # int32 [B] (key lengths; also the query lengths unless lengths_q is set)
    q: torch.Tensor | None   # [T_q, H, D] in ``dtype`` (CPU)
    k: torch.Tensor | None   # [T, H, D]
    v: torch.Tensor | None
    lengths_q: np.ndarray | None = None  # int32 [B] query lengths when they differ

    @property
    def num_seqs(self) -> int:
        return int(self.lengths.shape[0])

    @property
    def total_tokens(self) -> int:
        return int(self.lengths.astype(np.int64).sum())

    @property
    def max_len(self) -> int:
        return int(self.lengths.max()) if self.lengths.size else 0

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(D), rounded to float32 (the value both sides use)."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    def cu_seqlens_host(self) -> np.ndarray:
        """Boundaries as plain Python running totals (input bookkeeping only).

        Generators and tests need the boundaries to slice inputs; the method's
        own prefix sums live in the oracle and in the C library.
        """
        out = [0]
        for n in self.lengths.tolist():
            out.append(out[-1] + int(n))
        return np.asarray(out, dtype=np.int32)

    def query_lengths(self) -> np.ndarray:
        return self.lengths if self.lengths_q is None else self.lengths_q

    def cu_seqlens_q_host(self) -> np.ndarray:
        """Query boundaries (the key boundaries unless the lengths differ)."""
        out = [0]
        for n in self.query_lengths().tolist():
            out.append(out[-1] + int(n))
        return np.asarray(out, dtype=np.int32)

    @property
    def total_queries(self) -> int:
        return int(self.query_lengths().astype(np.int64).sum())


def _largest_remainder(quotas: np.ndarray, seats: int) -> np.ndarray:
    """Integer seats summing to ``seats`` that follow real ``quotas`` (which
    sum to ``seats``): each entry gets the floor of its quota, and the seats
    the floors leave over go one each to the entries with the largest
    fractional parts (Hamilton's apportionment).  Equal fractional parts are
    served in index order."""
    seats_of = np.floor(quotas).astype(np.int64)
    left_over = seats - int(seats_of.sum())
    # primary key: fractional part, largest first; secondary key: index
    queue = np.lexsort((np.arange(quotas.size), seats_of - quotas))
    seats_of[queue[:left_over]] += 1
    return seats_of


def zipf_lengths(total_tokens: int, num_seqs: int, rng: np.random.Generator,
                 exponent: float = 1.0) -> np.ndarray:
    """Sequence lengths proportional to rank^-exponent (Zipf), each at least
    one token, summing exactly to ``total_tokens``; sequence i has rank
    ``1 + rng.permutation(num_seqs)[i]``.

    Every sequence keeps one token; the remaining ``total_tokens - num_seqs``
    are apportioned in proportion to the Zipf weights by the largest-remainder
    rule.  This is the token split of "So you wanna CUDA Graph" (section
    "Hello World"), with the exponent 1 of the Zipf batch and equal remainders
    resolved in index order.
    """
    spare = total_tokens - num_seqs
    if spare < 0:
        raise ValueError(f"{total_tokens} tokens cannot give each of {num_seqs} sequences a token")
    rank = rng.permutation(num_seqs) + 1
    weight = rank.astype(np.float64) ** (-exponent)
    quotas = weight * (spare / weight.sum())
    return (_largest_remainder(quotas, spare) + 1).astype(np.int32)


def draw_lengths(index: int) -> np.ndarray:
    rng = np.random.default_rng(LENGTH_SEED_BASE + index)
    if index == 1:
        lengths = rng.integers(1, 65, size=8)
        lengths[rng.integers(0, 8)] = 1
    elif index == 2:
        raw = rng.lognormal(mean=math.log(80.0), sigma=0.6, size=512)
        lengths = np.clip(np.rint(raw), 1, 256)
    elif index == 3:
        raw = rng.gamma(shape=2.0, scale=75.0, size=128)
        lengths = np.clip(np.rint(raw), 8, 384)
    elif index == 4:
        lengths = zipf_lengths(65536, 64, rng, exponent=1.0)
    elif index == 5:
        short = rng.integers(64, 257, size=255)
        lengths = np.concatenate([short, np.asarray([32768])])
    elif index == 6:
        return draw_lengths(4)
    else:
        raise ValueError(f"unknown workload {index}")
    return np.asarray(lengths, dtype=np.int32)


_SPECS = {
    # index: (name, dtype, heads, head_dim, causal, value std)
    1: ("tiny", "fp32", 2, 16, False, 1.0),
    2: ("graph", "fp32", 8, 64, False, 1.0),
    3: ("encoder", "bf16", 12, 64, False, 1.0),
    4: ("zipf", "bf16", 16, 128, True, 1.0),
    5: ("skewed", "bf16", 32, 128, True, 0.5),
    6: ("cross", "bf16", 16, 128, False, 1.0),
}


def random_qkv(total_tokens: int, heads: int, head_dim: int, dtype: str,
               seed: int, std: float = 1.0, k_tokens: int | None = None):
    """Draw q [T,H,D], k/v [Tk,H,D] as float32 N(0, std^2), rounded to ``dtype``."""
    rng = np.random.default_rng(seed)
    tk = total_tokens if k_tokens is None else k_tokens
    tensors = []
    for rows in (total_tokens, tk, tk):
        a = rng.standard_normal((rows, heads, head_dim), dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        tensors.append(torch.from_numpy(a).to(DTYPES[dtype]))
    return tuple(tensors)


def random_dout(total_tokens: int, heads: int, head_dim: int, dtype: str, seed: int):
    """Draw an output gradient dO [T,H,D] as float32 N(0, 1), rounded to ``dtype``."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((total_tokens, heads, head_dim), dtype=np.float32)
    return torch.from_numpy(a).to(DTYPES[dtype])


def random_rows_device(rows: int, heads: int, head_dim: int, dtype: str, seed: int,
                       device, std: float = 1.0, chunk_rows: int = 1 << 22) -> torch.Tensor:
    """A [rows, heads, head_dim] tensor of N(0, std^2) values rounded to
    ``dtype``, drawn on ``device`` by a seeded torch generator in chunks of
    ``chunk_rows`` rows (for batches too large to draw on the host; the
    values depend on the seed, the chunking and the device type only)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = torch.empty(rows, heads, head_dim, dtype=DTYPES[dtype], device=device)
    for r0 in range(0, rows, chunk_rows):
        n = min(chunk_rows, rows - r0)
        a = torch.randn(n, heads, head_dim, generator=gen, device=device, dtype=torch.float32)
        if std != 1.0:
            a *= std
        out[r0:r0 + n].copy_(a)
    return out


def make_workload(index: int, with_values: bool = True,
                  dtype_override: str | None = None) -> Workload:
    """Build workload ``index`` (1..5) on the host."""
    name, dtype, heads, head_dim, causal, std = _SPECS[index]
    if dtype_override is not None:
        dtype = dtype_override
    lengths = draw_lengths(index)
    wl = Workload(name, index, dtype, heads, head_dim, causal, lengths, None, None, None)
    if index == 6:
        wl.lengths_q = ((lengths.astype(np.int64) + 3) // 4).astype(np.int32)
    if with_values:
        if wl.lengths_q is None:
            wl.q, wl.k, wl.v = random_qkv(wl.total_tokens, heads, head_dim, dtype,
                                          VALUE_SEED_BASE + index, std)
        else:
            wl.q, wl.k, wl.v = random_qkv(wl.total_queries, heads, head_dim, dtype,
                                          VALUE_SEED_BASE + index, std, k_tokens=wl.total_tokens)
    return wl


def custom_workload(lengths, heads: int, head_dim: int, dtype: str, causal: bool,
                    seed: int, std: float = 1.0, name: str = "custom") -> Workload:
    """A workload with caller-chosen lengths (edge cases in the tests)."""
    lengths = np.asarray(lengths, dtype=np.int32)
    wl = Workload(name, 0, dtype, heads, head_dim, causal, lengths, None, None, None)
    wl.q, wl.k, wl.v = random_qkv(wl.total_tokens, heads, head_dim, dtype, seed, std)
    return wl


WORKLOAD_NAMES = {v[0]: k for k, v in _SPECS.items()}
