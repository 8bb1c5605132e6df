"""Seeded synthetic workloads shared by the tests, the smoke check and bench.py.

This module only draws inputs and names shapes.  It holds none of the
attention arithmetic: neither the oracle nor the HIP path is imported here,
and both receive exactly the arrays made here.

Inputs follow the measured workloads of the pages: "Nax Refactor"
(ml-explore/mlx pull request 3271) times fused fp16 attention over
(B, qsl, ksl, hdim, n_qh, n_kvh, causal) grids, and the TileMix abstract
targets long-context, grouped-query, variable-length prefill with score-tile
routing.  Real model activations are not available, so Q, K and V are i.i.d.
N(0, 1) draws cast to fp16, standing in for the pages' LLaMA/Qwen/Vicuna
prefill activations and the LongEval / LV-Eval prompts.

Recipe: numpy.random.default_rng(seed).standard_normal in float64, drawn in
the order Q, K, V, each cast to float16 with round-to-nearest-even.  The
TileMix routing bitmask is a separate draw, default_rng(mask_seed).random(
(n_qtiles, n_groups)) < p_int8, where a True bit selects the INT8 path, packed
least-significant-bit first into rows of uint32 words.  Workloads marked kv8
hand K and V over as an INT8 key/value cache: the same fp16 draws, encoded by
the per-token quantiser of the side that consumes them (this module does no
encoding).
"""
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

TILE = 64  # rows per query tile and keys per key tile of the routing grid


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    qsl: int
    ksl: int
    hdim: int
    n_qh: int
    n_kvh: int
    causal: bool
    seed: int
    seqlens: Optional[List[int]] = None      # packed variable-length batch
    tiles_per_bit: int = 0                    # 0: no routing bitmask
    mask_seed: int = 0
    p_int8: float = 0.5
    kv8: bool = False                         # K and V as an INT8 key/value cache
    lowp: str = "int8"                        # what a set routing bit selects: "int8" or "fp8"
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.hdim)))

    @property
    def varlen(self) -> bool:
        return self.seqlens is not None


# The workloads: one small case the oracle finishes in seconds, then the
# measured shapes.
WORKLOADS = {
    "dense_256_d64": Workload("dense_256_d64", 1, 256, 256, 64, 4, 4, False, seed=1),
    "dense_1024_d64": Workload("dense_1024_d64", 1, 1024, 1024, 64, 32, 32, False, seed=2),
    "dense_1024_d64_causal": Workload("dense_1024_d64_causal", 1, 1024, 1024, 64, 32, 32, True, seed=2),
    "gqa_4096_d128_causal": Workload("gqa_4096_d128_causal", 1, 4096, 4096, 128, 32, 8, True, seed=3),
    "varlen_4seq_d128_causal": Workload("varlen_4seq_d128_causal", 4, 9108, 9108, 128, 32, 8, True,
                                        seed=4, seqlens=[512, 1500, 3000, 4096]),
    "bottomright_512x4096_d128": Workload("bottomright_512x4096_d128", 1, 512, 4096, 128, 32, 8, True,
                                          seed=41),
    "tilemix_16384_d128_causal": Workload("tilemix_16384_d128_causal", 1, 16384, 16384, 128, 32, 8, True,
                                          seed=5, tiles_per_bit=4, mask_seed=5005, p_int8=0.5),
    # the TileMix shape with FP8 e4m3 (rowwise scales) as the low-precision route
    "tilemix_16384_d128_causal_fp8": Workload("tilemix_16384_d128_causal_fp8", 1, 16384, 16384, 128, 32, 8, True,
                                              seed=5, tiles_per_bit=4, mask_seed=5005, p_int8=0.5, lowp="fp8"),
    # INT8 key/value cache inputs (TileMix abstract): the GQA and TileMix shapes
    "gqa_4096_d128_causal_kv8": Workload("gqa_4096_d128_causal_kv8", 1, 4096, 4096, 128, 32, 8, True,
                                         seed=3, kv8=True),
    "tilemix_16384_d128_causal_kv8": Workload("tilemix_16384_d128_causal_kv8", 1, 16384, 16384, 128, 32, 8,
                                              True, seed=5, tiles_per_bit=4, mask_seed=5005, p_int8=0.5,
                                              kv8=True),
}


def cu_seqlens_of(seqlens) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)


def draw_qkv(w: Workload, seed: Optional[int] = None):
    """fp16 numpy Q, K, V.  Dense: [B,H,S,d]; packed: [H,T,d]."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    if w.varlen:
        T = int(sum(w.seqlens))
        shapes = [(w.n_qh, T, w.hdim), (w.n_kvh, T, w.hdim), (w.n_kvh, T, w.hdim)]
    else:
        shapes = [(w.B, w.n_qh, w.qsl, w.hdim), (w.B, w.n_kvh, w.ksl, w.hdim),
                  (w.B, w.n_kvh, w.ksl, w.hdim)]
    return tuple(rng.standard_normal(s).astype(np.float16) for s in shapes)


def n_route_groups(ksl: int, tiles_per_bit: int, tile: int = TILE) -> int:
    n_kt = -(-ksl // tile)
    return -(-n_kt // tiles_per_bit)


def pack_bits(bits: np.ndarray) -> np.ndarray:
    """Pack a boolean [rows, n] array LSB-first into uint32 [rows, ceil(n/32)]."""
    bits = np.asarray(bits, dtype=bool)
    rows, n = bits.shape
    wpr = -(-n // 32)
    padded = np.zeros((rows, wpr * 32), dtype=np.uint64)
    padded[:, :n] = bits
    weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    words = (padded.reshape(rows, wpr, 32) * weights).sum(axis=2)
    return words.astype(np.uint32)


def draw_route(qsl: int, ksl: int, tiles_per_bit: int, p_int8: float, seed: int,
               tile: int = TILE) -> np.ndarray:
    """Bernoulli(p_int8) routing bits per (query tile, key-tile group), packed."""
    n_qt = -(-qsl // tile)
    n_g = n_route_groups(ksl, tiles_per_bit, tile)
    bits = np.random.default_rng(seed).random((n_qt, n_g)) < p_int8
    return pack_bits(bits)


def route_for(w: Workload) -> Optional[np.ndarray]:
    if not w.tiles_per_bit:
        return None
    return draw_route(w.qsl, w.ksl, w.tiles_per_bit, w.p_int8, w.mask_seed)


def metric_flop(B, n_qh, qsl, ksl, hdim, causal, seqlens=None) -> float:
    """The pages' throughput convention: 4*B*n_qh*qsl*ksl*hdim, halved if causal.

    A packed batch counts each sequence as its own (L x L) problem.
    """
    if seqlens is not None:
        f = sum(4.0 * n_qh * L * L * hdim for L in seqlens)
    else:
        f = 4.0 * B * n_qh * qsl * ksl * hdim
    return f / 2 if causal else f


def visited_pairs(qsl: int, ksl: int, causal: bool) -> int:
    """Number of (i, j) pairs a bottom-right causal mask leaves visible."""
    if not causal:
        return qsl * ksl
    off = ksl - qsl
    return sum(min(ksl, i + off + 1) for i in range(qsl))


def workload_flop(w: Workload):
    """(metric FLOP, visited FLOP) of one forward call on workload w."""
    metric = metric_flop(w.B, w.n_qh, w.qsl, w.ksl, w.hdim, w.causal, w.seqlens)
    if w.varlen:
        pairs = sum(visited_pairs(L, L, w.causal) for L in w.seqlens)
        visited = 4.0 * w.n_qh * w.hdim * pairs
    else:
        visited = 4.0 * w.B * w.n_qh * w.hdim * visited_pairs(w.qsl, w.ksl, w.causal)
    return metric, visited
