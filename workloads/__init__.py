"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module only draws numbers and arranges them: it holds none of the
quantization or attention arithmetic.  Both the HIP path (through torch
tensors) and the CPU oracle (through NumPy arrays) consume exactly the arrays
returned here.

Recipe (all draws from ``numpy.random.default_rng``):
  * values are fp32 N(0, 1) draws; "bf16" inputs are those draws rounded to
    bf16, nearest-even (rounding done by torch's CPU cast, a plumbing step);
  * order of draws inside one stream: K, then V, then outlier channels, then
    Q, then lengths, then the page permutation;
  * large workloads use one stream per (layer) or per (sequence), keyed as
    ``default_rng([seed, key...])`` so any block can be regenerated alone.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

try:  # torch is only used for the bf16 cast of inputs
    import torch
except Exception:  # pragma: no cover - torch is present in every supported env
    torch = None


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), nearest-even (torch CPU cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


@dataclass
class Workload:
    """Shapes of one synthetic decode/prefill workload."""
    name: str
    batch: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    group: int              # 0 = per-token scales, 32 = group-32 scales
    layout: str             # "contiguous" or "paged"
    kv_dtype: str           # "f32" or "bf16" for the appended K/V
    ctx: int                # tokens cached before the step (contiguous)
    n_new: int              # tokens appended by the step
    layers: int = 1
    outliers: int = 0       # outlier channels per (layer, kv head), x10
    seed: int = 0
    attn_scale: float = 0.0
    max_len: int = 0
    extra: dict = field(default_factory=dict)

    def __post_init__(self):
        if self.attn_scale == 0.0:
            self.attn_scale = float(1.0 / np.sqrt(self.head_dim))
        if self.max_len == 0:
            self.max_len = self.ctx + self.n_new


# The five workloads measured for this path (shapes as stated with the
# method's target metric; seeds: tiny decode uses 0, workload k uses k-1).
TINY = Workload("tiny_decode", 1, 8, 2, 64, 0, "contiguous", "f32", 255, 1, seed=0,
                attn_scale=0.125)
DECODE_8B = Workload("decode_8b", 16, 32, 8, 128, 0, "contiguous", "bf16", 4095, 1,
                     layers=32, outliers=4, seed=1)
Q8_GROUP32 = Workload("q8_group32", 8, 32, 8, 128, 32, "contiguous", "f32", 4095, 1,
                      layers=32, seed=2, max_len=4096)
PAGED = Workload("paged_decode", 64, 32, 8, 128, 0, "paged", "bf16", 0, 1, seed=3,
                 extra={"len_lo": 512, "len_hi": 32768, "page_size": 16})
CHUNK = Workload("chunked_prefill", 4, 32, 8, 128, 0, "contiguous", "bf16", 8192, 512,
                 seed=4)

# The 8B-shaped decode step on a recent-window hybrid cache: the last 128
# tokens of every sequence stay bf16 (the window the hybrid cache's default
# configuration keeps), the older ones are INT8.
RECENT = Workload("recent_window", 16, 32, 8, 128, 0, "contiguous", "bf16", 4095, 1,
                  layers=32, outliers=4, seed=5, extra={"window": 128})

# Sliding-window (local-layer) attention: a 1024-token window over 8192-token
# contexts, for decode (32 layers, K/V drawn on the device from a seeded
# generator: 9 GB of cache) and for the chunked-prefill shape.
SLIDING_DECODE = Workload("sliding_decode", 16, 32, 8, 128, 0, "contiguous", "bf16", 8191, 1,
                          layers=32, seed=6, extra={"sliding": 1024})
SLIDING_CHUNK = Workload("sliding_chunk", 4, 32, 8, 128, 0, "contiguous", "bf16", 8192, 512,
                         seed=7, extra={"sliding": 1024})

# The 8B-shaped decode step with per-token scales stored as bf16 (the GPU
# cache of abaddon kv_cache_quant_cuda.rs keeps them so).
BF16_SCALES = Workload("bf16_scales", 16, 32, 8, 128, 0, "contiguous", "bf16", 4095, 1,
                       layers=32, outliers=4, seed=8, extra={"scale_bf16": True})

# The 8B-shaped decode step on FP8 E4M3 codes with no scales (llama-gguf
# kv_quantized.rs `KVCacheFormat::Fp8E4M3`).
FP8_E4M3 = Workload("fp8_e4m3", 16, 32, 8, 128, 0, "contiguous", "bf16", 4095, 1,
                    layers=32, outliers=4, seed=9, extra={"fp8": "e4m3"})

# The chunked-prefill step on FP8 E4M3 codes.
FP8_CHUNK = Workload("fp8_chunk", 4, 32, 8, 128, 0, "contiguous", "bf16", 8192, 512,
                     seed=10, extra={"fp8": "e4m3"})

# The chunked-prefill step on group-32 scales (the Q8 layout of the decode
# workload above).
CHUNK_G32 = Workload("chunk_group32", 4, 32, 8, 128, 32, "contiguous", "bf16", 8192, 512, seed=11)

# The chunked-prefill step on a recent-window hybrid cache (W = 128): the
# chunk's rows enter through the hybrid append, and its queries attend to the
# INT8 rows and the ring.
RECENT_CHUNK = Workload("recent_chunk", 4, 32, 8, 128, 0, "contiguous", "bf16", 8192, 512, seed=12,
                        extra={"window": 128})

# The recent-window decode step with per-head and per-channel block scales
# (abaddon kv_cache_quant_cuda.rs `QuantGranularity`, over 16-row blocks).
RECENT_BLOCK_HEAD = Workload("recent_block_head", 16, 32, 8, 128, 0, "contiguous", "bf16", 4095, 1,
                             layers=32, outliers=4, seed=13, extra={"window": 128, "block": "head"})
RECENT_BLOCK_CHANNEL = Workload("recent_block_channel", 16, 32, 8, 128, 0, "contiguous", "bf16", 4095, 1,
                                layers=32, outliers=4, seed=14, extra={"window": 128, "block": "channel"})

# Chunked prefill at head dim 256 (local-attention layers of the Gemma
# family, which combs-models' sliding-window cache serves): 16 query heads on
# 8 KV heads, the chunked-prefill shape otherwise.
CHUNK_D256 = Workload("chunk_d256", 4, 16, 8, 256, 0, "contiguous", "bf16", 8192, 512, seed=15)
# Decode at head dim 256: the 8B-shaped decode's bytes per token (4 KV heads
# of 256 dims), 16 query heads.
DECODE_D256 = Workload("decode_d256", 16, 16, 4, 256, 0, "contiguous", "bf16", 4095, 1,
                       layers=32, outliers=4, seed=16)

ALL = {w.name: w for w in (TINY, DECODE_8B, Q8_GROUP32, PAGED, CHUNK, RECENT, SLIDING_DECODE, SLIDING_CHUNK,
                           BF16_SCALES, FP8_E4M3, FP8_CHUNK, CHUNK_G32, RECENT_CHUNK, RECENT_BLOCK_HEAD,
                           RECENT_BLOCK_CHANNEL, CHUNK_D256, DECODE_D256)}


# ----------------------------------------------------------------------------
# Generators
# ----------------------------------------------------------------------------

def _maybe_bf16(x: np.ndarray, dtype: str):
    """Returns (values fp32, raw) where raw is what the GPU receives: fp32
    array, or bf16 bit patterns."""
    if dtype == "bf16":
        bits = bf16_bits(x)
        return bits_to_f32(bits), bits
    return x, x


def layer_inputs(w: Workload, layer: int, tokens: int | None = None):
    """K/V for every cached + new token and Q of one layer (contiguous layouts).

    Returns dict with ``k``/``v`` fp32 values ``[B, KVH, T, D]`` (bf16-exact when
    the workload's K/V are bf16), ``k_raw``/``v_raw`` (what the device gets),
    ``q_bits`` bf16 ``[B, H, D]`` (or ``[B, H, n, D]`` when n_new > 1) and ``q``
    fp32 values.  One stream ``default_rng([seed, layer])``.
    """
    tokens = w.ctx + w.n_new if tokens is None else tokens
    rng = np.random.default_rng([w.seed, layer])
    shape = (w.batch, w.num_kv_heads, tokens, w.head_dim)
    k = normal(rng, shape)
    v = normal(rng, shape)
    if w.outliers:
        for arr in (k, v):
            for h in range(w.num_kv_heads):
                ch = rng.choice(w.head_dim, size=w.outliers, replace=False)
                arr[:, h, :, ch] *= np.float32(10.0)
    qshape = (w.batch, w.num_heads, w.head_dim) if w.n_new == 1 else \
        (w.batch, w.num_heads, w.n_new, w.head_dim)
    q_bits = bf16_bits(normal(rng, qshape))
    k, k_raw = _maybe_bf16(k, w.kv_dtype)
    v, v_raw = _maybe_bf16(v, w.kv_dtype)
    return {"k": k, "v": v, "k_raw": k_raw, "v_raw": v_raw,
            "q_bits": q_bits, "q": bits_to_f32(q_bits)}


def tiny_inputs():
    """Tiny decode: one stream ``default_rng(0)``: K [1,2,256,64] fp32, V, Q bf16 [1,8,64]."""
    w = TINY
    rng = np.random.default_rng(w.seed)
    shape = (w.batch, w.num_kv_heads, w.ctx + w.n_new, w.head_dim)
    k = normal(rng, shape)
    v = normal(rng, shape)
    q_bits = bf16_bits(normal(rng, (w.batch, w.num_heads, w.head_dim)))
    return {"k": k, "v": v, "k_raw": k, "v_raw": v, "q_bits": q_bits, "q": bits_to_f32(q_bits)}


def paged_layout(w: Workload = PAGED, batch: int | None = None, len_lo: int | None = None,
                 len_hi: int | None = None, seed: int | None = None):
    """Sequence lengths and block table for a paged workload.

    Lengths are integers uniform in [len_lo, len_hi] (inclusive; they count
    the appended token).  The arena holds P = sum ceil(L_b/16) pages; a random
    permutation of the P page ids is dealt out to the sequences in order, so
    sequence b's logical pages are scattered over the shared arena.
    Returns (lens int32 [B], block_table int32 [B, max_blocks] padded with -1,
    num_pages).
    """
    batch = w.batch if batch is None else batch
    lo = w.extra["len_lo"] if len_lo is None else len_lo
    hi = w.extra["len_hi"] if len_hi is None else len_hi
    ps = w.extra.get("page_size", 16)
    rng = np.random.default_rng([w.seed if seed is None else seed, 0])
    lens = rng.integers(lo, hi, endpoint=True, size=batch).astype(np.int32)
    npg = (lens.astype(np.int64) + ps - 1) // ps
    num_pages = int(npg.sum())
    perm = rng.permutation(num_pages).astype(np.int32)
    max_blocks = -(-hi // ps)
    table = np.full((batch, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(batch):
        table[b, :npg[b]] = perm[off:off + npg[b]]
        off += int(npg[b])
    return lens, table, num_pages


def sequence_kv(w: Workload, b: int, length: int):
    """K/V of one paged sequence, ``[KVH, length, D]``, stream ``[seed, 1 + b]``."""
    rng = np.random.default_rng([w.seed, 1 + b])
    shape = (w.num_kv_heads, length, w.head_dim)
    k = normal(rng, shape)
    v = normal(rng, shape)
    k, k_raw = _maybe_bf16(k, w.kv_dtype)
    v, v_raw = _maybe_bf16(v, w.kv_dtype)
    return {"k": k, "v": v, "k_raw": k_raw, "v_raw": v_raw}


def paged_q(w: Workload = PAGED, batch: int | None = None):
    batch = w.batch if batch is None else batch
    rng = np.random.default_rng([w.seed, 100000])
    q_bits = bf16_bits(normal(rng, (batch, w.num_heads, w.head_dim)))
    return q_bits, bits_to_f32(q_bits)


def random_kv(seed: int, shape, dtype: str = "f32", scale: float = 1.0):
    """Generic seeded N(0, scale^2) K/V pair for small test shapes."""
    rng = np.random.default_rng(seed)
    k = normal(rng, shape) * np.float32(scale)
    v = normal(rng, shape) * np.float32(scale)
    k, k_raw = _maybe_bf16(k, dtype)
    v, v_raw = _maybe_bf16(v, dtype)
    return {"k": k, "v": v, "k_raw": k_raw, "v_raw": v_raw}


def random_q(seed: int, shape):
    rng = np.random.default_rng(seed)
    q_bits = bf16_bits(normal(rng, shape))
    return q_bits, bits_to_f32(q_bits)
