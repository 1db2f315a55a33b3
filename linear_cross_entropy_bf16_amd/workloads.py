"""Seeded synthetic inputs for fused linear cross-entropy.

This module only *draws* inputs.  It holds none of the loss arithmetic, so both
the fp64 CPU oracle (``oracle/``) and the HIP path can take their inputs from it
without sharing any of the method's code.

Shapes follow the pages' LLM output-layer setting (page "Cutting LLM Memory by
84%: A Deep Dive into Fused Kernels", section "The Logit Bottleneck": tokens
N = batch x sequence, hidden size D, vocabulary V, Llama-3-8B sizes D = 4096,
V = 128 256, N = 8 x 8192).  No public dataset is named for this workload, so
every tensor is synthetic:

* X ~ N(0, 1) and W ~ N(0, 1/D) drawn in fp32, then rounded to bf16
  (round-to-nearest-even) for bf16 workloads, so logits have unit variance.
* bias ~ N(0, 0.02^2) when present.
* targets uniform on [0, V) or a truncated Zipf(s) law over a seeded
  permutation of the vocabulary (natural-language token frequencies).
* exactly round(f * N) rows, chosen without replacement, carry ignore_index.

The random streams are spawned from ``SeedSequence(1000 + seed)`` in the
fixed order X, W, bias, targets, ignore, samples, so each tensor is reproducible
on its own; Gaussian tensors are drawn in fixed 4M-element chunks, each from
its own spawned PCG64 stream, so generation can run on several threads and
still give the same values.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np

IGNORE_INDEX = -100

STREAMS = ("x", "w", "bias", "targets", "ignore", "samples")


@dataclasses.dataclass(frozen=True)
class Workload:
    """One named problem: sizes, input recipe and loss options."""

    name: str
    n: int
    d: int
    v: int
    dtype: str = "bf16"            # "bf16" or "f32": dtype of X, W and bias
    bias: bool = False
    targets: str = "uniform"       # "uniform" or "zipf"
    zipf_s: float = 1.1
    ignore_frac: float = 0.0
    ignore_index: int = IGNORE_INDEX
    label_smoothing: float = 0.0
    lse_square_scale: float = 0.0
    softcap: float = 0.0
    reduction: str = "mean"        # "mean", "sum" or "none"
    seed: int = 0
    kind: str = "flce"             # "flce": X, W (+ bias); "ce_logits": logits [N, V] given directly

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def flops_fwd_bwd(self) -> float:
        """Algorithmic FLOPs of one forward + backward with recompute:
        four N x D x V contractions (forward logits, recomputed logits,
        dX and dW), 2 FLOPs per multiply-add."""
        return 8.0 * self.n * self.d * self.v


# The five workloads: a tiny fp32 case, a small LM head, one Llama-3-8B
# sequence, the pages' 8 x 8192-token headline shape and a feature-heavy wide
# vocabulary.
WORKLOADS: Dict[str, Workload] = {
    "tiny_f32": Workload("tiny_f32", 256, 128, 1024, dtype="f32",
                         ignore_frac=0.05, seed=0),
    "small_lm_head": Workload("small_lm_head", 4096, 2048, 32000,
                              ignore_frac=0.02, seed=1),
    "llama3_8b_seq": Workload("llama3_8b_seq", 8192, 4096, 128256,
                              targets="zipf", seed=2),
    "llama3_8b_batch8": Workload("llama3_8b_batch8", 65536, 4096, 128256,
                                 targets="zipf", ignore_frac=0.10, seed=3),
    "wide_vocab_features": Workload("wide_vocab_features", 16384, 8192, 256000,
                                    bias=True, targets="zipf", ignore_frac=0.25,
                                    label_smoothing=0.1, lse_square_scale=1e-4,
                                    softcap=30.0, reduction="sum", seed=4),
}
WORKLOAD_ORDER = list(WORKLOADS)

# Cross-entropy on logits given directly (the workload of the cross-entropy
# kernels on materialised logits, TransformerEngine PR #995): logits ~ N(0, 1),
# the distribution the fused workloads' X W^T has.  d is unused.  A small case,
# one Llama-3-8B sequence of 128 256-way logits, and an fp32 feature case whose
# odd V leaves most rows unaligned to 16 bytes.
CE_WORKLOADS: Dict[str, Workload] = {
    "ce_logits_small": Workload("ce_logits_small", 4096, 0, 32000, ignore_frac=0.02, seed=11,
                                kind="ce_logits"),
    "ce_logits_llama3_8b_seq": Workload("ce_logits_llama3_8b_seq", 8192, 0, 128256,
                                        targets="zipf", ignore_frac=0.05, seed=12,
                                        kind="ce_logits"),
    "ce_logits_features_f32": Workload("ce_logits_features_f32", 2048, 0, 50257, dtype="f32",
                                       targets="zipf", ignore_frac=0.25, label_smoothing=0.1,
                                       lse_square_scale=1e-4, softcap=30.0, reduction="sum",
                                       seed=13, kind="ce_logits"),
}


def _seed_seqs(seed: int) -> Dict[str, np.random.SeedSequence]:
    ss = np.random.SeedSequence(1000 + seed)
    return dict(zip(STREAMS, ss.spawn(len(STREAMS))))


def streams(seed: int) -> Dict[str, np.random.Generator]:
    return {name: np.random.Generator(np.random.PCG64(sq))
            for name, sq in _seed_seqs(seed).items()}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 with round-to-nearest-even; returns uint16 bit
    patterns.  Inputs here are finite (Gaussian draws)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).reshape(-1)
    out = np.empty(a.size, dtype=np.uint16)
    step = 1 << 22
    for i in range(0, u.size, step):
        s = u[i:i + step]
        r = (s >> np.uint32(16)) & np.uint32(1)
        r += np.uint32(0x7FFF)
        r += s
        out[i:i + step] = r >> np.uint32(16)
    return out.reshape(a.shape)


_CHUNK = 1 << 22


def _normal(sq: np.random.SeedSequence, shape, std: float, dtype: str) -> np.ndarray:
    """Gaussian tensor drawn in fixed 4M-element chunks, one spawned PCG64
    stream per chunk, so the values do not depend on the thread count."""
    total = int(np.prod(shape))
    nchunks = (total + _CHUNK - 1) // _CHUNK
    children = sq.spawn(nchunks)
    out = np.empty(total, dtype=np.uint16 if dtype == "bf16" else np.float32)

    def work(i):
        lo, hi = i * _CHUNK, min(total, (i + 1) * _CHUNK)
        a = np.random.Generator(np.random.PCG64(children[i])).standard_normal(
            hi - lo, dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        out[lo:hi] = f32_to_bf16_bits(a) if dtype == "bf16" else a

    workers = max(1, min(16, os.cpu_count() or 1, nchunks))
    if workers == 1:
        for i in range(nchunks):
            work(i)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape(shape)


def draw_targets(rng: np.random.Generator, n: int, v: int, law: str,
                 zipf_s: float) -> np.ndarray:
    if law == "uniform":
        return rng.integers(0, v, size=n, dtype=np.int64).astype(np.int32)
    if law == "zipf":
        # truncated Zipf over ranks 1..V by inverse CDF, mapped through a
        # seeded permutation so frequent tokens are spread over the vocabulary
        perm = rng.permutation(v)
        ranks = np.arange(1, v + 1, dtype=np.float64)
        cdf = np.cumsum(ranks ** (-zipf_s))
        cdf /= cdf[-1]
        u = rng.random(n)
        k = np.minimum(np.searchsorted(cdf, u, side="right"), v - 1)
        return perm[k].astype(np.int32)
    raise ValueError(f"unknown target law {law!r}")


def generate(wl: Workload, n: Optional[int] = None,
             with_x: bool = True, with_w: bool = True) -> Dict[str, np.ndarray]:
    """Draw the inputs of ``wl``.

    Returns a dict with ``x`` ([n, d]), ``w`` ([v, d], the nn.Linear LM-head
    layout), ``bias`` ([v] or None) and ``targets`` (int32 [n]).  bf16 tensors
    are uint16 bit patterns, fp32 tensors are float32.  ``n`` overrides the
    row count (rows are the leading rows of the full draw only when equal).
    """
    n = wl.n if n is None else n
    sq = _seed_seqs(wl.seed)
    st = streams(wl.seed)
    out: Dict[str, Optional[np.ndarray]] = {}
    out["x"] = _normal(sq["x"], (n, wl.d), 1.0, wl.dtype) if with_x else None
    out["w"] = (_normal(sq["w"], (wl.v, wl.d), 1.0 / np.sqrt(wl.d), wl.dtype)
                if with_w else None)
    out["bias"] = _normal(sq["bias"], (wl.v,), 0.02, wl.dtype) if wl.bias else None
    t = draw_targets(st["targets"], n, wl.v, wl.targets, wl.zipf_s)
    n_ign = int(round(wl.ignore_frac * n))
    if n_ign:
        rows = st["ignore"].choice(n, size=n_ign, replace=False)
        t[rows] = wl.ignore_index
    out["targets"] = t
    return out


def sample_rows(wl: Workload, count: int, salt: int = 0) -> np.ndarray:
    """Seeded, sorted, distinct row indices of the full workload (for checks
    on sampled rows and for sub-batches)."""
    st = streams(wl.seed)
    rng = st["samples"]
    if salt:
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000 + wl.seed, salt])))
    count = min(count, wl.n)
    return np.sort(rng.choice(wl.n, size=count, replace=False)).astype(np.int64)


def generate_logits(wl: Workload, n: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Inputs of a cross-entropy-on-logits workload: ``logits`` [n, v] ~ N(0, 1)
    (bf16 bit patterns or fp32, drawn from the X stream) and ``targets`` as for
    ``generate``."""
    n = wl.n if n is None else n
    sq = _seed_seqs(wl.seed)
    st = streams(wl.seed)
    logits = _normal(sq["x"], (n, wl.v), 1.0, wl.dtype)
    t = draw_targets(st["targets"], n, wl.v, wl.targets, wl.zipf_s)
    n_ign = int(round(wl.ignore_frac * n))
    if n_ign:
        t[st["ignore"].choice(n, size=n_ign, replace=False)] = wl.ignore_index
    return {"logits": logits, "targets": t}
