"""Seeded generators for the synthetic multi-adapter LoRA workloads.

Every array that carries bf16 data is returned as its raw 16-bit pattern
(numpy uint16), produced from float32 normal draws by round-to-nearest-even.
Nothing here computes the LoRA product: this module only decides shapes,
adapter ids, segment lengths, ranks, scales and random values.

Workload shapes follow the multi-adapter serving and packed-training settings
described in the "Trajectory presenta C-LoRA" (vivodigitale.it) ("Come funziona l'architettura": decode
batches that mix tokens of many resident adapters) and the "Technische Samenvatting: PLoRA" (gist.science)
("LoRA Execution Engine": many heterogeneous adapters fine-tuned in one packed
job, up to 32 adapters per job, ranks and scaling factors varied across a
hyper-parameter search).

Value distributions: activations and upstream gradients ~ N(0, 1); shrink
weights A_i ~ N(0, 1/h_in); expand weights B_i ~ N(0, 1/r_i) (second
parameter = variance). Generator: numpy PCG64 via ``default_rng(seed)``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

_CHUNK_ROWS = 4096  # fixed draw granularity for large matrices (part of the recipe)


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16. Inputs are finite normal draws, so
    the NaN/overflow branches of a general converter are not needed.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def _normal_bf16(rng: np.random.Generator, rows: int, cols: int, std: float) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.uint16)
    for r0 in range(0, rows, _CHUNK_ROWS):
        r1 = min(rows, r0 + _CHUNK_ROWS)
        f = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        if std != 1.0:
            f *= np.float32(std)
        out[r0:r1] = bf16_bits_from_f32(f)
    return out


@dataclasses.dataclass
class Problem:
    """One LoRA-wrapped projection call over one token batch.

    token_ids   int32[T]  adapter id per token (-1 = no adapter) in the order
                          the batch is handed over. For id-based workloads
                          this is request order and the caller still has to
                          group tokens into segments; for segment-based
                          workloads tokens are already grouped.
    seg_lens    int32[S] or None: segment lengths when the batch is already
                          grouped (segment-based workloads)
    seg_adapter int32[S] or None: adapter of each given segment
    x           uint16[T, h_in]  bf16 bits, rows in token_ids order
    A           list of uint16[r_i, h_in]   bf16 bits (shrink weights)
    B           list of uint16[h_out, r_i]  bf16 bits (expand weights)
    dy          uint16[T, h_out] or None    upstream gradient (training)
    y0          uint16[T, h_out] or None    initial output (None = zeros)
    """

    name: str
    seed: int
    T: int
    h_in: int
    h_out: int
    ranks: np.ndarray
    scales: np.ndarray
    token_ids: np.ndarray
    seg_lens: Optional[np.ndarray]
    seg_adapter: Optional[np.ndarray]
    x: np.ndarray
    A: List[np.ndarray]
    B: List[np.ndarray]
    dy: Optional[np.ndarray] = None
    y0: Optional[np.ndarray] = None

    @property
    def N(self) -> int:
        return int(len(self.ranks))

    @property
    def segmented(self) -> bool:
        return self.seg_lens is not None


def _draw_weights(rng, N, h_in, h_out, ranks):
    A, B = [], []
    for i in range(N):
        r = int(ranks[i])
        A.append(_normal_bf16(rng, r, h_in, 1.0 / math.sqrt(h_in)))
        B.append(_normal_bf16(rng, h_out, r, (1.0 / math.sqrt(r)) if r > 0 else 1.0))
    return A, B


def _ids_problem(name, seed, rng, ids, h_in, h_out, ranks, scales, with_dy=False, y0=False):
    ids = np.asarray(ids, dtype=np.int32)
    T = int(ids.shape[0])
    x = _normal_bf16(rng, T, h_in, 1.0)
    A, B = _draw_weights(rng, len(ranks), h_in, h_out, ranks)
    dy = _normal_bf16(rng, T, h_out, 1.0) if with_dy else None
    y0a = _normal_bf16(rng, T, h_out, 1.0) if y0 else None
    return Problem(name, seed, T, h_in, h_out, np.asarray(ranks, np.int32),
                   np.asarray(scales, np.float32), ids, None, None, x, A, B, dy, y0a)


def _seg_problem(name, seed, rng, seg_lens, seg_adapter, h_in, h_out, ranks, scales,
                 with_dy=False, y0=False):
    seg_lens = np.asarray(seg_lens, dtype=np.int32)
    seg_adapter = np.asarray(seg_adapter, dtype=np.int32)
    ids = np.repeat(seg_adapter, seg_lens).astype(np.int32)
    T = int(seg_lens.sum())
    x = _normal_bf16(rng, T, h_in, 1.0)
    A, B = _draw_weights(rng, len(ranks), h_in, h_out, ranks)
    dy = _normal_bf16(rng, T, h_out, 1.0) if with_dy else None
    y0a = _normal_bf16(rng, T, h_out, 1.0) if y0 else None
    return Problem(name, seed, T, h_in, h_out, np.asarray(ranks, np.int32),
                   np.asarray(scales, np.float32), ids, seg_lens, seg_adapter, x, A, B, dy, y0a)


# ---------------------------------------------------------------------------
# The five workloads (seed = position in this list).
# ---------------------------------------------------------------------------
CONFIG_NAMES = ["tiny", "decode", "prefill", "hetero", "train"]


@dataclasses.dataclass
class Meta:
    """The batch structure of a workload without its tensors: widths, ranks,
    scales and either request-order ids or an explicit segmentation. Drawn
    with the same generator calls, in the same order, as the full workload,
    so it matches the Problem of the same name and seed."""

    name: str
    T: int
    h_in: int
    h_out: int
    ranks: np.ndarray
    scales: np.ndarray
    token_ids: np.ndarray
    seg_lens: Optional[np.ndarray] = None
    seg_adapter: Optional[np.ndarray] = None

    @property
    def N(self) -> int:
        return int(len(self.ranks))

    @property
    def segmented(self) -> bool:
        return self.seg_lens is not None


def _tiny_meta(rng):
    return rng.integers(0, 4, size=16).astype(np.int32)


def make_tiny(seed: int = 0) -> Problem:
    """16 decode tokens, 256->256, 4 adapters of rank 8, scale 2.0, ids
    uniform in [0, 4) in request order."""
    rng = np.random.default_rng(seed)
    ids = _tiny_meta(rng)
    return _ids_problem("tiny", seed, rng, ids, 256, 256, [8] * 4, [2.0] * 4)


def _decode_meta(rng):
    return rng.integers(0, 8, size=256).astype(np.int32)


DECODE_PROJECTIONS = (("q", 2560), ("o", 2560), ("gate_up", 19456))


def make_c2_projections(seed: int = 1) -> Dict[str, Problem]:
    """Mixed-adapter decode on Qwen3-4B-like projections: 256 tokens with
    adapter ids uniform in [0, 8) (request order); 8 adapters of rank 32,
    scale 2.0, separate weights per projection. Three calls share the batch:
    q (2560->2560), o (2560->2560) and gate_up (2560->19456)."""
    rng = np.random.default_rng(seed)
    ids = _decode_meta(rng)
    out = {}
    for proj, h_out in DECODE_PROJECTIONS:
        out[proj] = _ids_problem(f"decode_{proj}", seed, rng, ids, 2560, h_out,
                                 [32] * 8, [2.0] * 8)
    return out


def prefill_segment_lengths(rng: np.random.Generator, total: int = 8192,
                            median: float = 512.0, sigma: float = 1.0) -> np.ndarray:
    """Lognormal segment lengths (median 512, sigma 1.0), each at least 1,
    drawn until the running total reaches `total`; the last one is cut so the
    lengths sum to exactly `total`."""
    lens = []
    acc = 0
    mu = math.log(median)
    while acc < total:
        v = max(1, int(round(float(rng.lognormal(mu, sigma)))))
        v = min(v, total - acc)
        lens.append(v)
        acc += v
    return np.asarray(lens, dtype=np.int32)


def _prefill_meta(rng):
    lens = prefill_segment_lengths(rng)
    seg_adapter = rng.integers(0, 8, size=len(lens)).astype(np.int32)
    return lens, seg_adapter


def make_prefill(seed: int = 2) -> Problem:
    """Chunked prefill, LLaMA-3-8B-like 4096->4096: 8 adapters of rank 16,
    8192 tokens in lognormal-length segments, adapter per segment uniform."""
    rng = np.random.default_rng(seed)
    lens, seg_adapter = _prefill_meta(rng)
    return _seg_problem("prefill", seed, rng, lens, seg_adapter, 4096, 4096,
                        [16] * 8, [2.0] * 8)


def zipf_popularity(n: int = 32, exponent: float = 1.1, n_empty: int = 4) -> np.ndarray:
    """Finite Zipf probabilities over popularity ranks 1..n, p_k ~ k^-exponent,
    with the `n_empty` least popular ranks given probability 0."""
    k = np.arange(1, n + 1, dtype=np.float64)
    p = k ** (-exponent)
    if n_empty:
        p[n - n_empty:] = 0.0
    return p / p.sum()


def make_hetero(seed: int = 3) -> Problem:
    """MLP-up 4096->14336 with 32 adapters, ranks uniform from
    {8,16,32,64,128}, scale 2.0, 4096 tokens, Zipf(1.1) popularity with the
    4 least popular adapters unused (empty segments)."""
    rng = np.random.default_rng(seed)
    ranks, ids = _hetero_meta(rng)
    return _ids_problem("hetero", seed, rng, ids, 4096, 14336, ranks, [2.0] * 32)


def _hetero_meta(rng):
    ranks = rng.choice(np.array([8, 16, 32, 64, 128]), size=32).astype(np.int32)
    perm = rng.permutation(32).astype(np.int32)
    pop = rng.choice(32, size=4096, p=zipf_popularity())
    return ranks, perm[pop].astype(np.int32)


def make_train(seed: int = 4) -> Problem:
    """Packed training on Qwen-2.5-7B-like 3584->3584: 32 adapters with ranks
    uniform from {8,16,32,64}, scale 2.0, each 4 sequences x 512 tokens,
    adapter-major; random upstream gradient dy."""
    rng = np.random.default_rng(seed)
    ranks, lens, seg_adapter = _train_meta(rng)
    return _seg_problem("train", seed, rng, lens, seg_adapter, 3584, 3584, ranks,
                        [2.0] * 32, with_dy=True)


def _train_meta(rng):
    ranks = rng.choice(np.array([8, 16, 32, 64]), size=32).astype(np.int32)
    seg_adapter = np.repeat(np.arange(32, dtype=np.int32), 4)
    lens = np.full(128, 512, dtype=np.int32)
    return ranks, lens, seg_adapter


def make_meta(name: str, seed: Optional[int] = None, proj: str = "gate_up") -> Meta:
    """Batch structure of the named workload (no tensors drawn). For
    'decode', `proj` picks the projection width (q, o or gate_up)."""
    idx = CONFIG_NAMES.index(name)
    rng = np.random.default_rng(idx if seed is None else seed)
    if name == "tiny":
        ids = _tiny_meta(rng)
        return Meta(name, 16, 256, 256, np.full(4, 8, np.int32), np.full(4, 2.0, np.float32), ids)
    if name == "decode":
        ids = _decode_meta(rng)
        h_out = dict(DECODE_PROJECTIONS)[proj]
        return Meta(f"decode_{proj}", 256, 2560, h_out, np.full(8, 32, np.int32), np.full(8, 2.0, np.float32), ids)
    if name == "prefill":
        lens, sa = _prefill_meta(rng)
        return Meta(name, int(lens.sum()), 4096, 4096, np.full(8, 16, np.int32), np.full(8, 2.0, np.float32),
                    np.repeat(sa, lens).astype(np.int32), lens, sa)
    if name == "hetero":
        ranks, ids = _hetero_meta(rng)
        return Meta(name, 4096, 4096, 14336, ranks, np.full(32, 2.0, np.float32), ids)
    ranks, lens, sa = _train_meta(rng)
    return Meta(name, int(lens.sum()), 3584, 3584, ranks, np.full(32, 2.0, np.float32),
                np.repeat(sa, lens).astype(np.int32), lens, sa)


def make_config(name: str, seed: Optional[int] = None):
    """Return the named workload. 'decode' returns a dict of three Problems."""
    idx = CONFIG_NAMES.index(name)
    s = idx if seed is None else seed
    if name == "tiny":
        return make_tiny(s)
    if name == "decode":
        return make_c2_projections(s)
    if name == "prefill":
        return make_prefill(s)
    if name == "hetero":
        return make_hetero(s)
    return make_train(s)


def make_custom(seed: int, h_in: int, h_out: int, ranks, scales=None, ids=None,
                seg_lens=None, seg_adapter=None, with_dy=False, y0=False,
                name: str = "custom") -> Problem:
    """Small workloads for parity and edge-case tests: either per-token ids in
    request order (`ids`) or an explicit segmentation (`seg_lens`,
    `seg_adapter`). `scales` defaults to 2.0 for every adapter; the string
    'random' draws them uniformly from [0.25, 4)."""
    rng = np.random.default_rng(seed)
    N = len(ranks)
    if scales is None:
        scales = [2.0] * N
    elif isinstance(scales, str) and scales == "random":
        scales = rng.uniform(0.25, 4.0, size=N).astype(np.float32)
    if ids is not None:
        return _ids_problem(name, seed, rng, ids, h_in, h_out, ranks, scales, with_dy, y0)
    return _seg_problem(name, seed, rng, seg_lens, seg_adapter, h_in, h_out, ranks, scales,
                        with_dy, y0)
