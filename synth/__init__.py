"""Seeded synthetic inputs for the W8A8 verify path.

This module only draws random numbers and shapes them; it holds none of the
method's arithmetic (no quantization, no products, no rounding rules of its
own).  Both the CPU oracle side (tests, the CPU baseline) and the GPU side
(tests, the benchmark) take their inputs from here, so the two are fed the
same bytes.

Every stream is ``numpy.random.default_rng([workload, tensor, index])``
(PCG64 seeded through SeedSequence), so a tensor, a row block of a tensor
or a trial can be regenerated on its own, on any machine.

The shapes and distributions are the synthetic stand-ins for the pages'
workloads (Qwen3-8B / Qwen3-32B linears and LM head; the pages evaluate on
real checkpoints and on MT-bench, HumanEval, GSM8k, Alpaca and CNN/DM, none
of which is used here):

* activations: bf16 of N(0, 1), optionally with a fixed set of outlier
  channels (0.1 % of K, at least one) multiplied by 20 before the bf16
  rounding, the same channels in every row;
* weights: fp32 N(0, 0.02) in nn.Linear order ``[N][K]``;
* draft ids: uniform integers in ``[0, V)``.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os as _os
from dataclasses import dataclass

import numpy as np
import torch

# Tensor ids inside one workload's seed space.
T_WEIGHT = 1
T_ACT = 2
T_DRAFT = 3
T_OUTLIER = 4
T_SMOOTH = 5

# Weight row blocks are drawn from their own streams so that any subset of
# rows can be regenerated without drawing the whole matrix.
ROW_BLOCK = 1024


def rng(workload: int, tensor: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(workload), int(tensor), int(index)])


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 with torch's CPU cast and return the bit
    patterns as uint16.  (A library conversion, used only to produce inputs.)"""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def outlier_channels(workload: int, K: int, frac: float = 0.001,
                     layer: int = 0) -> np.ndarray:
    """The outlier channel indices for a K-wide activation: max(1, round(frac*K))
    distinct channels drawn without replacement (sorted)."""
    n = max(1, int(round(frac * K)))
    r = rng(workload, T_OUTLIER, layer * 1_000_003 + K)
    return np.sort(r.choice(K, size=n, replace=False))


def activations_bf16(workload: int, M: int, K: int, index: int = 0,
                     outliers: bool = False, outlier_scale: float = 20.0,
                     layer: int = 0) -> np.ndarray:
    """bf16 bit patterns ``uint16[M][K]`` of N(0,1) draws; with ``outliers``
    the channels from :func:`outlier_channels` are scaled by ``outlier_scale``
    before the bf16 rounding."""
    z = rng(workload, T_ACT, index).standard_normal((M, K), dtype=np.float32)
    if outliers:
        z[:, outlier_channels(workload, K, layer=layer)] *= np.float32(outlier_scale)
    return to_bf16_bits(z)


def _weight_block(workload: int, tensor_index: int, b: int, K: int,
                  rows: int, std: float) -> np.ndarray:
    r = rng(workload, T_WEIGHT, tensor_index * 1_000_000 + b)
    w = r.standard_normal((rows, K), dtype=np.float32)
    w *= np.float32(std)
    return w


def weights_f32(workload: int, N: int, K: int, tensor_index: int = 0,
                std: float = 0.02, threads: int | None = None) -> np.ndarray:
    """fp32 ``[N][K]`` ~ N(0, std), drawn in row blocks of ROW_BLOCK rows,
    each block from its own stream (blocks are drawn in parallel)."""
    nblk = (N + ROW_BLOCK - 1) // ROW_BLOCK
    out = np.empty((N, K), dtype=np.float32)

    def fill(b):
        r0 = b * ROW_BLOCK
        rows = min(ROW_BLOCK, N - r0)
        out[r0:r0 + rows] = _weight_block(workload, tensor_index, b, K, rows, std)

    threads = threads or min(16, _os.cpu_count() or 1)
    if nblk == 1 or threads == 1:
        for b in range(nblk):
            fill(b)
    else:
        with _cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def weight_rows_f32(workload: int, N: int, K: int, rows: np.ndarray,
                    tensor_index: int = 0, std: float = 0.02) -> np.ndarray:
    """The given rows of :func:`weights_f32` (same values), drawing only the
    row blocks that hold them."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), K), dtype=np.float32)
    for b in np.unique(rows // ROW_BLOCK):
        r0 = int(b) * ROW_BLOCK
        nb = min(ROW_BLOCK, N - r0)
        blk = _weight_block(workload, tensor_index, int(b), K, nb, std)
        sel = np.nonzero(rows // ROW_BLOCK == b)[0]
        out[sel] = blk[rows[sel] - r0]
    return out


def weights_device(workload: int, tensor_index: int, N: int, K: int, device,
                   std: float = 0.02) -> torch.Tensor:
    """fp32 ``[N][K]`` ~ N(0, std) drawn on a GPU with torch's device
    generator seeded from (workload, tensor_index).  Used where the host
    generator is too slow (tens of GB of weights); the values differ from
    :func:`weights_f32`.  A consumer on the host takes a copy of this tensor."""
    g = torch.Generator(device=device)
    g.manual_seed(int(workload) * 1_000_003 + int(tensor_index))
    w = torch.randn(N, K, generator=g, device=device, dtype=torch.float32)
    w.mul_(std)
    return w


def draft_ids(workload: int, B: int, G: int, V: int, index: int = 0) -> np.ndarray:
    """Uniform draft ids ``int32[B][G]`` in [0, V)."""
    return rng(workload, T_DRAFT, index).integers(0, V, size=(B, G)).astype(np.int32)


def prefix_drafts(reference_argmax: np.ndarray, p: int, V: int,
                  r: np.random.Generator) -> np.ndarray:
    """Drafts for one sequence whose first ``p`` ids equal the given reference
    argmax ids (positions 0..G), the id at position p (if p < G) differs from
    the reference argmax there, and the rest are uniform.  Pure index
    bookkeeping: the reference argmax is an input."""
    a = np.asarray(reference_argmax, dtype=np.int64)
    G = len(a) - 1
    d = r.integers(0, V, size=G).astype(np.int64)
    d[:p] = a[:p]
    if p < G:
        # uniform over [0, V) without the reference id at position p
        u = int(r.integers(0, V - 1))
        d[p] = u if u < a[p] else u + 1
    return d.astype(np.int32)


def smoothing_vector(workload: int, K: int, lo: float = 0.25, hi: float = 4.0) -> np.ndarray:
    """A positive per-channel vector ``float32[K]`` (log-uniform in [lo, hi])."""
    r = rng(workload, T_SMOOTH, K)
    return np.exp(r.uniform(np.log(lo), np.log(hi), size=K)).astype(np.float32)


# --------------------------------------------------------------------------
# Workload shapes (the five synthetic workloads)
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Linear:
    name: str
    K: int
    N: int


QWEN3_8B_LAYER = (
    Linear("q", 4096, 4096), Linear("k", 4096, 1024), Linear("v", 4096, 1024),
    Linear("o", 4096, 4096), Linear("gate", 4096, 12288), Linear("up", 4096, 12288),
    Linear("down", 12288, 4096),
)
QWEN3_VOCAB = 151936
QWEN3_8B_LM_HEAD = Linear("lm_head", 4096, QWEN3_VOCAB)

QWEN3_32B_LAYER = (
    Linear("q", 5120, 8192), Linear("k", 5120, 1024), Linear("v", 5120, 1024),
    Linear("o", 8192, 5120), Linear("gate", 5120, 25600), Linear("up", 5120, 25600),
    Linear("down", 25600, 5120),
)
QWEN3_32B_LM_HEAD = Linear("lm_head", 5120, QWEN3_VOCAB)
QWEN3_32B_LAYERS = 64


def stack_tensor_index(layer: int, linear: int) -> int:
    """Weight tensor id of linear ``linear`` (0..6, in QWEN3_32B_LAYER order)
    of ``layer`` in the 32B stack; the LM head is ``layer = QWEN3_32B_LAYERS``,
    ``linear = 0``."""
    return layer * 8 + linear

# workload ids (the first element of every seed)
W_TINY = 1        # M=5, K=256, N=512, B=1, G=4
W_LAYER_M5 = 2    # Qwen3-8B layer linears at M=5
W_LM_HEAD = 3     # LM head 4096 -> 151936 at M=5, 1000 trials
W_BATCHED = 4     # Qwen3-8B layer linears at M=288 (32 x (8+1))
W_STACK32B = 5    # Qwen3-32B stack at M=8


def lm_head_trial(trial: int, reference_argmax_rows: np.ndarray | None = None,
                  V: int = QWEN3_VOCAB, K: int = 4096, G: int = 4):
    """Inputs of one LM-head verification trial: x (bf16 bits, [G+1][K]) and,
    when the reference argmax of its G+1 rows is given, drafts whose first
    ``p = trial mod (G+1)`` ids equal it (see :func:`prefix_drafts`)."""
    x = activations_bf16(W_LM_HEAD, G + 1, K, index=trial)
    if reference_argmax_rows is None:
        return x, None, trial % (G + 1)
    p = trial % (G + 1)
    d = prefix_drafts(reference_argmax_rows, p, V, rng(W_LM_HEAD, T_DRAFT, trial))
    return x, d, p
