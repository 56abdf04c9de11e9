"""CPU oracle for the INT8 KV-cache hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
module.  The product library never routes through it, and it shares no code
with the HIP kernels: it takes plain NumPy arrays and computes, slowly and
step by step, what the pages define.

Precision contract
  * quantization is emulated in IEEE fp32 (NumPy float32 division rounds to
    nearest; denormals are kept on x86 SSE), because the method produces
    integer codes from fp32 arithmetic and both sides must take that decision
    in the same precision;
  * rounding of the quotient is "half away from zero" and is evaluated in fp64
    on the fp32 quotient (``|y| + 0.5`` in fp32 would mis-round 0.49999997);
  * dequantization for attention is exact in fp64 ((code-128) * scale fits in
    31 significant bits);
  * attention is fp64 over those exact values, by its plain definition:
    scores, max-subtracted softmax, probability-weighted sum.

Sources (docs.rs source pages; a citation names the page and the Rust item):
  [P1] abaddon 0.2.0-rc.1, src/kv_cache_quant_cuda.rs
  [P2] realizar 0.8.5, src/cuda/executor/kv_cache_q8_init.rs
  [P3] abaddon 0.2.0-rc.2, src/kv_cache_quant.rs
  [P4] combs-models 0.2.2, src/kv.rs
  [P5] llama-gguf 0.14.0, src/model/kv_quantized.rs

Every function below is pinned by a ``-m "not gpu"`` test against a value the
pages fix, a closed form, or brute force; none is marked "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

# Smallest absmax the per-token quantizer allows (P1 `quantize_tensor`, the
# `.max(1e-8)` on the row's absolute maximum; P3 `QuantizedKvCache::quantize`,
# the `eps` tensor).  Applied identically for group-32 (reading documented in
# the P1 rule for both scale modes).
ABSMAX_FLOOR = np.float32(1e-8)
QMAX = np.float32(127.0)
CODE_OFFSET = 128
GROUP = 32
PAGE_SIZE = 16


# ----------------------------------------------------------------------------
# bf16 helpers (output rounding; [P1] kernel-source helpers `bf16_to_f32`,
# `f32_to_bf16`, which define bf16 as the upper half of an fp32 word rounded
# to nearest, ties to even)
# ----------------------------------------------------------------------------

def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp32 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 -> bf16, nearest with ties to even, as uint16 bit patterns.

    Written from the definition: the 16 dropped low bits are compared with the
    half-way point 0x8000; above it rounds up, below it truncates, and exactly
    at it the kept part is made even.  Finite inputs only.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    hi = u >> np.uint64(16)
    lo = u & np.uint64(0xFFFF)
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & np.uint64(1)) == 1))
    return (hi + up.astype(np.uint64)).astype(np.uint16)


# ----------------------------------------------------------------------------
# Quantizer
# ----------------------------------------------------------------------------

def round_half_away_from_zero(y: np.ndarray) -> np.ndarray:
    """Nearest integer, ties away from zero, of fp32 values, as int64.

    Rust's `f32::round`, used by the per-token quantizer of [P1]
    `CudaQuantizedKvCache::quantize_tensor` and by [P5] `quantize_int8`.
    """
    y64 = np.asarray(y, dtype=np.float32).astype(np.float64)
    return (np.sign(y64) * np.floor(np.abs(y64) + 0.5)).astype(np.int64)


def quantize(x: np.ndarray, group: int = 0):
    """Symmetric absmax/127 quantization to u8 codes with a +128 offset.

    ``x``: float32 array ``[..., D]``.  ``group``: 0 for one scale per row
    (per token and KV head) or 32 for one scale per 32 consecutive elements
    along the last axis.  Returns ``(codes uint8 [..., D], scales float32
    [..., G])`` with G = 1 or D/32.

    Steps, in the order [P1] `CudaQuantizedKvCache::quantize_tensor` takes
    them (group-32 granularity and fp32 scale storage from [P4] `kv_quantize`
    and [P2] `init_kv_cache_q8_gpu`):
      1. m = max(max_i |x_i|, 1e-8)            (exact in fp32)
      2. s = fl32(m / 127)                     (IEEE fp32 division)
      3. y = fl32(x_i / s)                     (IEEE fp32 division, not x*(1/s))
      4. q = round half away from zero (y), clamped to [-127, 127]
      5. code = q + 128                        (in [1, 255] for finite input)
    """
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    gsize = d if group == 0 else group
    if d % gsize != 0:
        raise ValueError("head_dim must be a multiple of the group size")
    g = x.reshape(x.shape[:-1] + (d // gsize, gsize))
    m = np.max(np.abs(g), axis=-1)
    m = np.maximum(m, ABSMAX_FLOOR).astype(np.float32)
    s = (m / QMAX).astype(np.float32)
    y = (g / s[..., None]).astype(np.float32)
    q = np.clip(round_half_away_from_zero(y), -127, 127)
    codes = (q + CODE_OFFSET).astype(np.uint8).reshape(x.shape)
    return codes, s


def quantize_bf16_scale(x: np.ndarray):
    """Per-token codes with the scale stored as bf16 ([P1]
    `CudaQuantizedKvCache::quantize_tensor`): the codes come from the fp32
    scale exactly as in :func:`quantize` (group 0), and the scale is kept as
    its bf16 rounding (the page's `f32_to_bf16`, nearest even), which is what
    dequantization then multiplies by.  Returns (codes uint8 [..., D],
    scale bit patterns uint16 [..., 1])."""
    codes, s = quantize(x, 0)
    return codes, f32_to_bf16_bits(s)


def _expand_scales(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    d = codes.shape[-1]
    gcount = scales.shape[-1]
    return np.repeat(scales.astype(np.float64), d // gcount, axis=-1)


def dequantize_exact(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """x_hat = (code - 128) * s, exact in fp64.

    [P1] module doc ("Dequantize K: (K_u8 - 128) * scale"), [P3]
    `QuantizedKvCache::dequantize`.  The group count is read from the trailing
    dimension of ``scales`` (1 = per token, D/32 = group-32).
    """
    c = np.asarray(codes).astype(np.float64) - CODE_OFFSET
    return c * _expand_scales(codes, scales)


def dequantize_f32(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """fl32((code - 128) * s): the exact product rounded once to fp32."""
    return dequantize_exact(codes, scales).astype(np.float32)


def dequantize_bf16_bits(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """bf16 (RNE) of the fp32 dequantized value, as uint16 bit patterns."""
    return f32_to_bf16_bits(dequantize_f32(codes, scales))


# ----------------------------------------------------------------------------
# FP8 codes ([P5] `KVCacheFormat::Fp8E4M3` / `Fp8E5M2`): each element is stored
# as one FP8 byte of its own value, with no scale; the page's converters
# `quantize_fp8_e4m3` / `quantize_fp8_e5m2` and `dequantize_fp8_*`
# ----------------------------------------------------------------------------

# (mantissa bits, exponent bias, code of a positive infinity input,
#  code of a positive overflow)
FP8_FORMATS = {
    "e4m3": (3, 7, 0x7F, 0x7E),
    "e5m2": (2, 15, 0x7C, 0x7C),
}


def fp8_encode(x: np.ndarray, fmt: str) -> np.ndarray:
    """fp32 -> FP8 byte, as [P5] `quantize_fp8_e4m3` / `quantize_fp8_e5m2`
    compute it (an encoding, so its steps are followed in order):
      1. NaN -> 0xFF;  +/-inf -> the format's infinity code (E4M3 0x7F / 0xFF,
         E5M2 0x7C / 0xFC);  +/-0 -> 0x00.
      2. Split the fp32 word: sign s, unbiased exponent e (raw field - 127),
         24-bit significand m (the implicit leading one added unless the raw
         exponent field is 0).
      3. Target exponent E = e + bias (7 or 15).
      4. E above the largest field (15 or 31): s | overflow code (E4M3 0x7E,
         the largest finite value 448; E5M2 0x7C, infinity).
      5. -M < E <= 0 (M = mantissa bits): a subnormal; the mantissa field is
         the top M + E bits of m, so the value is cut toward zero.
      6. E <= -M: s | 0 (a signed zero).
      7. Otherwise s | E << M | the top M fraction bits of m (cut toward
         zero, no rounding).
    Returns uint8 codes of ``x``'s shape.  Note step 7 at the largest
    exponent field can give the format's NaN or infinity patterns
    (E4M3 |x| in [480, 512); E5M2 |x| in [65536, 131072)), as on the page.
    """
    mbits, bias, inf_code, over_code = FP8_FORMATS[fmt]
    emax = (1 << (7 - mbits)) - 1
    xf = np.ascontiguousarray(x, dtype=np.float32)
    u = xf.view(np.uint32).astype(np.int64)
    sign = (u >> 31) & 1
    raw_e = (u >> 23) & 0xFF
    e = raw_e - 127
    m = (u & 0x7FFFFF) | np.where(raw_e != 0, 1 << 23, 0)
    E = e + bias
    s7 = sign << 7
    mask = (1 << mbits) - 1
    out = np.empty(xf.shape, dtype=np.int64)
    normal = (E >= 1) & (E <= emax)
    out[normal] = s7[normal] | (E[normal] << mbits) | ((m[normal] >> (23 - mbits)) & mask)
    sub = (E > -mbits) & (E <= 0)
    shift = 24 - (mbits + E[sub])
    out[sub] = s7[sub] | ((m[sub] >> shift) & (mask >> (-E[sub])))
    out[E <= -mbits] = s7[E <= -mbits]
    out[E > emax] = s7[E > emax] | over_code
    out[xf == 0] = 0
    isinf = np.isinf(xf)
    out[isinf] = np.where(xf[isinf] > 0, inf_code, 0x80 | inf_code)
    out[np.isnan(xf)] = 0xFF
    return out.astype(np.uint8)


def fp8_decode(codes: np.ndarray, fmt: str) -> np.ndarray:
    """FP8 byte -> value (fp64, exact), as [P5] `dequantize_fp8_e4m3` /
    `dequantize_fp8_e5m2` define it: a zero magnitude field is +0 (for either
    sign bit); E4M3 S.1111.111 is NaN; E5M2 S.11111.00 is +/-inf and
    S.11111.{01,10,11} NaN; an exponent field F > 0 gives
    (-1)^s 2^(F - bias) (1 + f / 2^M), and F = 0 the subnormal
    (-1)^s f 2^(1 - bias - M) (the page builds the same numbers case by case)."""
    mbits, bias, _, _ = FP8_FORMATS[fmt]
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    F = (c >> mbits) & ((1 << (7 - mbits)) - 1)
    f = c & ((1 << mbits) - 1)
    mag = np.where(F > 0, np.ldexp(1.0 + f / float(1 << mbits), F - bias),
                   np.ldexp(f.astype(np.float64), 1 - bias - mbits))
    val = sign * mag
    low = c & 0x7F
    val = np.where(low == 0, 0.0, val)
    if fmt == "e4m3":
        val = np.where(low == 0x7F, np.nan, val)
    else:
        val = np.where(low == 0x7C, sign * np.inf, val)
        val = np.where(low >= 0x7D, np.nan, val)
    return val


def fp8_decode_bf16_bits(codes: np.ndarray, fmt: str) -> np.ndarray:
    """bf16 (RNE) of the decoded value, as uint16 bit patterns (every finite
    E4M3 / E5M2 value fits fp32 exactly)."""
    return f32_to_bf16_bits(fp8_decode(codes, fmt).astype(np.float32))


# ----------------------------------------------------------------------------
# Cache layouts
# ----------------------------------------------------------------------------

def contiguous_append(k_codes, k_scales, v_codes, v_scales, k_new, v_new, start_pos, group):
    """Quantize ``[B, KVH, n, D]`` new rows and store them at positions
    ``start_pos[b] + i`` of a contiguous cache ``[B, KVH, max_len, D]``.

    Fixed-capacity slot write with a per-head ``max_len`` stride, as in [P2]
    `write_kv_q8` (offset head*max_len*head_dim + position*head_dim).
    Arrays are modified in place.
    """
    kc, ks = quantize(k_new, group)
    vc, vs = quantize(v_new, group)
    bsz, _, n, _ = k_new.shape
    max_len = k_codes.shape[2]
    for b in range(bsz):
        p0 = int(start_pos[b])
        if p0 < 0 or p0 + n > max_len:
            raise IndexError("append beyond capacity")
        k_codes[b, :, p0:p0 + n] = kc[b]
        k_scales[b, :, p0:p0 + n] = ks[b]
        v_codes[b, :, p0:p0 + n] = vc[b]
        v_scales[b, :, p0:p0 + n] = vs[b]


def page_slot(block_table: np.ndarray, b: int, p: int, page_size: int = PAGE_SIZE):
    """Logical position p of sequence b -> (physical page, slot).

    [P4] `PagedKVCache::attention_opts` write loop: slot = pos % page_size,
    phys = table[pos / page_size]; generalised to one table row per sequence.
    """
    return int(block_table[b, p // page_size]), p % page_size


def paged_append(k_codes, k_scales, v_codes, v_scales, block_table, k_new, v_new, start_pos, group):
    """Quantize new rows and write them into a paged arena
    ``[P, KVH, 16, D]`` (scales ``[P, KVH, 16, G]``) through the block table.

    [P4] `PagedKVCache::attention_opts` (quantized arena branch): quantize the
    incoming chunk once, then place each token with the page-slot arithmetic.
    """
    kc, ks = quantize(k_new, group)
    vc, vs = quantize(v_new, group)
    bsz, _, n, _ = k_new.shape
    for b in range(bsz):
        for i in range(n):
            phys, slot = page_slot(block_table, b, int(start_pos[b]) + i)
            k_codes[phys, :, slot] = kc[b, :, i]
            k_scales[phys, :, slot] = ks[b, :, i]
            v_codes[phys, :, slot] = vc[b, :, i]
            v_scales[phys, :, slot] = vs[b, :, i]


def paged_gather(arena, block_table, b, length, page_size=PAGE_SIZE):
    """Materialise sequence b's logical window ``[KVH, length, last]`` from a
    paged arena ``[P, KVH, page_size, last]``.

    [P4] `PagedKVCache::gather_window`: select the table's pages, put the
    head axis first, flatten pages x slots, keep the first ``length``.
    """
    npages = -(-length // page_size)
    pages = arena[block_table[b, :npages]]            # [npages, KVH, PS, last]
    win = np.swapaxes(pages, 0, 1)                   # [KVH, npages, PS, last]
    win = win.reshape(win.shape[0], npages * page_size, win.shape[-1])
    return win[:, :length]


# ----------------------------------------------------------------------------
# Attention (fp64, plain definition)
# ----------------------------------------------------------------------------

def kv_head_of(h: int, num_heads: int, num_kv_heads: int) -> int:
    """GQA mapping: query head h reads KV head h // (H / KVH).

    [P4] `repeat_kv` repeats each KV head n_rep times consecutively; [P1]
    kernels use h * num_kv_heads / num_heads, the same when H % KVH == 0.
    """
    return h // (num_heads // num_kv_heads)


def softmax_attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, attn_scale: float,
                   visible: np.ndarray | None = None) -> np.ndarray:
    """One query row: fp64 scaled dot-product attention.

    ``q`` [D], ``k``/``v`` [T, D] (fp64), ``visible`` optional bool [T].
    Scores q.k * scale; masked keys drop out (the [P1] causal branch fills
    -inf, [P4] `attend` fills -1e30: both vanish after exp); max-subtracted
    softmax; probability-weighted sum of values ([P4] `attend`, manual path;
    [P1] `forward_attention` softmax).
    """
    s = (k @ q) * float(attn_scale)
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    m = np.max(s)
    p = np.exp(s - m)
    p = p / np.sum(p)
    return p @ v


def window_visible(positions: np.ndarray, p: int, window: int) -> np.ndarray:
    """Keys a query at absolute position p may see: t <= p, and with a
    sliding window w also t > p - w ([P4] `KVCache::attention_opts` doc,
    keys in (p - w, p]; `attend`, `too_old` = k + w - 1 < p)."""
    vis = positions <= p
    if window > 0:
        vis &= positions > p - window
    return vis


def attention_decode(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray,
                     seq_lens, attn_scale: float, window: int = 0) -> np.ndarray:
    """Decode attention, one query token per sequence.

    ``q`` [B, H, D] (exact bf16 values as floats), ``k_hat``/``v_hat``
    [B, KVH, >=L, D] dequantized (fp64), ``seq_lens`` [B] attended lengths.
    The query sits at position L - 1.  Without a window it sees every cached
    token, so no mask applies ([P4] `attend`, the decode comment); a sliding
    window ``window`` > 0 keeps only keys in (L - 1 - window, L - 1].
    Returns [B, H, D] fp64.
    """
    bsz, nh, d = q.shape
    nkv = k_hat.shape[1]
    out = np.zeros((bsz, nh, d), dtype=np.float64)
    for b in range(bsz):
        length = int(seq_lens[b])
        vis = window_visible(np.arange(length), length - 1, window) if window > 0 else None
        for h in range(nh):
            g = kv_head_of(h, nh, nkv)
            out[b, h] = softmax_attend(q[b, h].astype(np.float64), k_hat[b, g, :length],
                                       v_hat[b, g, :length], attn_scale, vis)
    return out


def attention_chunk(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, ctx_lens,
                    causal: bool, attn_scale: float, window: int = 0) -> np.ndarray:
    """Chunked-prefill attention for n new queries per sequence.

    ``q`` [B, H, n, D]; ``k_hat``/``v_hat`` [B, KVH, >=L0+n, D] with the chunk
    already appended after ``ctx_lens[b] = L0`` cached tokens.  Query i sits at
    absolute position L0 + i and, when causal, sees keys t <= L0 + i
    (bottom-right alignment: [P1] `forward_attention`, cache_offset = seq_len
    - q_len; [P4] `attend`, keys > pos forbidden).  Non-causal queries see all
    L0 + n keys.  A sliding window ``window`` > 0 implies the causal bound
    and also hides keys t <= L0 + i - window ([P4] `attend`: the window mask
    is OR-ed onto the causal one).  Returns [B, H, n, D] fp64.
    """
    bsz, nh, n, d = q.shape
    nkv = k_hat.shape[1]
    out = np.zeros((bsz, nh, n, d), dtype=np.float64)
    for b in range(bsz):
        l0 = int(ctx_lens[b])
        total = l0 + n
        t = np.arange(total)
        for h in range(nh):
            g = kv_head_of(h, nh, nkv)
            kk = k_hat[b, g, :total]
            vv = v_hat[b, g, :total]
            for i in range(n):
                if window > 0:
                    vis = window_visible(t, l0 + i, window)
                else:
                    vis = (t <= l0 + i) if causal else None
                out[b, h, i] = softmax_attend(q[b, h, i].astype(np.float64), kk, vv,
                                              attn_scale, vis)
    return out


# ----------------------------------------------------------------------------
# Recent-window hybrid cache ([P1] `OptimizedQuantizedKvCache`): the last W
# tokens of a sequence stay unquantized (bf16), older tokens are INT8.
# ----------------------------------------------------------------------------

def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to bf16 (nearest even), returned as fp32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


class RecentWindowCache:
    """One sequence's hybrid cache, updated by the steps of [P1]
    `OptimizedQuantizedKvCache::append`:

      1. the new rows join the unquantized recent part (held as bf16 values:
         the page keeps its recent tensors in BF16, so an fp32 input row is
         rounded once, to nearest even, when it enters);
      2. if the recent part is longer than the window W, its oldest
         len - W rows are quantized (one row at a time, with this cache's
         quantizer and scale mode) and appended to the quantized part;
      3. the newest W rows stay recent.

    Arrays are ``[KVH, tokens, D]``.  ``window`` 0 quantizes every row on
    arrival (a plain INT8 cache).
    """

    def __init__(self, num_kv_heads: int, head_dim: int, window: int, group: int = 0):
        self.window = int(window)
        self.group = int(group)
        g = 1 if group == 0 else head_dim // group
        self.k_codes = np.zeros((num_kv_heads, 0, head_dim), np.uint8)
        self.v_codes = np.zeros((num_kv_heads, 0, head_dim), np.uint8)
        self.k_scales = np.zeros((num_kv_heads, 0, g), np.float32)
        self.v_scales = np.zeros((num_kv_heads, 0, g), np.float32)
        self.k_recent = np.zeros((num_kv_heads, 0, head_dim), np.float32)
        self.v_recent = np.zeros((num_kv_heads, 0, head_dim), np.float32)

    def append(self, k_new: np.ndarray, v_new: np.ndarray) -> None:
        k_rec = np.concatenate([self.k_recent, to_bf16_values(k_new)], axis=1)
        v_rec = np.concatenate([self.v_recent, to_bf16_values(v_new)], axis=1)
        n_old = k_rec.shape[1] - self.window
        if n_old > 0:
            kc, ks = quantize(k_rec[:, :n_old], self.group)
            vc, vs = quantize(v_rec[:, :n_old], self.group)
            self.k_codes = np.concatenate([self.k_codes, kc], axis=1)
            self.k_scales = np.concatenate([self.k_scales, ks], axis=1)
            self.v_codes = np.concatenate([self.v_codes, vc], axis=1)
            self.v_scales = np.concatenate([self.v_scales, vs], axis=1)
            k_rec, v_rec = k_rec[:, n_old:], v_rec[:, n_old:]
        self.k_recent, self.v_recent = k_rec, v_rec

    def quantized_len(self) -> int:
        return self.k_codes.shape[1]

    def recent_len(self) -> int:
        return self.k_recent.shape[1]

    def seq_len(self) -> int:
        return self.quantized_len() + self.recent_len()

    def kv(self):
        """[P1] `get_kv`: the dequantized old rows followed by the recent rows,
        as exact fp64 ``[KVH, L, D]`` K and V."""
        k = np.concatenate([dequantize_exact(self.k_codes, self.k_scales),
                            self.k_recent.astype(np.float64)], axis=1)
        v = np.concatenate([dequantize_exact(self.v_codes, self.v_scales),
                            self.v_recent.astype(np.float64)], axis=1)
        return k, v


# ----------------------------------------------------------------------------
# Per-head and per-channel granularity ([P1] `QuantGranularity`,
# `quantize_with_granularity`): the page takes one scale per head (the maximum
# over sequence and head_dim) or per (head, channel) (the maximum over the
# sequence) of whatever tensor one `append` hands over, so a row's codes
# depend on which rows were appended with it.  Reading used here (the design doc
# reading 20): the "sequence" is a fixed, position-aligned block of B rows
# (B = 16 in the kernels).  Block j (rows jB .. jB+B-1) is quantized, from its
# rows' bf16 values, at the append after which its first row has left the
# window (L > jB + W); W >= B - 1 guarantees that all B rows exist then.  Row
# p is read as INT8 when p < L - W, as on the page, so the quantized and
# recent counts are the page's; rows of a quantized block still inside the
# window are read from the recent part until they leave it.
# ----------------------------------------------------------------------------

def quantize_block(x: np.ndarray, granularity: str):
    """One block ``x`` [KVH, B, D] (fp32 values) with the per-token
    quantizer's steps (:func:`quantize`) applied over the page's reduction
    sets: ``"head"``, the maximum over the block's B rows and all D elements;
    ``"channel"``, the maximum over the B rows of each element index d.
    Returns (codes uint8 [KVH, B, D], scales float32: [KVH, 1] per head,
    [KVH, D] per channel)."""
    x = np.asarray(x, dtype=np.float32)
    kvh, nb, d = x.shape
    if granularity == "head":
        codes, s = quantize(x.reshape(kvh, nb * d), 0)        # one scale over B x D
        return codes.reshape(kvh, nb, d), s
    if granularity == "channel":
        codes, s = quantize(np.swapaxes(x, 1, 2), 0)          # [KVH, D, B]: one scale per d
        return np.ascontiguousarray(np.swapaxes(codes, 1, 2)), s[..., 0]
    raise ValueError("granularity is 'head' or 'channel'")


class BlockRecentCache:
    """One sequence's hybrid cache with per-head or per-channel block scales
    (reading above).  Rows enter as bf16 values, as in
    :class:`RecentWindowCache`; the quantized state is kept per block.

    ``codes``: [KVH, nq_blocks * B, D] for every quantized block (rows inside
    the window included).  ``scales``: per head [KVH, nq_blocks], per channel
    [KVH, nq_blocks, D].
    """

    def __init__(self, num_kv_heads: int, head_dim: int, window: int, granularity: str, block: int = 16):
        if granularity not in ("head", "channel"):
            raise ValueError("granularity is 'head' or 'channel'")
        if block < 1 or window < block - 1:
            raise ValueError("the window must be at least block - 1 rows")
        self.window, self.granularity, self.block = int(window), granularity, int(block)
        self.kvh, self.d = int(num_kv_heads), int(head_dim)
        self.rows = [np.zeros((num_kv_heads, 0, head_dim), np.float32) for _ in range(2)]  # every row, bf16 values
        self.codes = [np.zeros((num_kv_heads, 0, head_dim), np.uint8) for _ in range(2)]
        sshape = (num_kv_heads, 0) if granularity == "head" else (num_kv_heads, 0, head_dim)
        self.scales = [np.zeros(sshape, np.float32) for _ in range(2)]

    def append(self, k_new: np.ndarray, v_new: np.ndarray) -> None:
        for side, x in enumerate((k_new, v_new)):
            self.rows[side] = np.concatenate([self.rows[side], to_bf16_values(x)], axis=1)
        length = self.seq_len()
        for side in range(2):
            # every block whose first row has left the window is quantized
            while self.codes[side].shape[1] < length - self.window:
                j0 = self.codes[side].shape[1]
                blk = self.rows[side][:, j0:j0 + self.block]
                assert blk.shape[1] == self.block  # guaranteed by window >= block - 1
                c, sc = quantize_block(blk, self.granularity)
                self.codes[side] = np.concatenate([self.codes[side], c], axis=1)
                sc = sc[:, None] if self.granularity == "channel" else sc
                self.scales[side] = np.concatenate([self.scales[side], sc], axis=1)

    def seq_len(self) -> int:
        return self.rows[0].shape[1]

    def quantized_len(self) -> int:
        """Rows read as INT8 (the page's count)."""
        return recent_split(self.seq_len(), self.window)

    def recent_len(self) -> int:
        return self.seq_len() - self.quantized_len()

    def row_scales(self, side: int) -> np.ndarray:
        """Scales expanded to one entry per quantized row: [KVH, rows, 1] per
        head, [KVH, rows, D] per channel."""
        s = np.repeat(self.scales[side], self.block, axis=1)
        return s[..., None] if self.granularity == "head" else s

    def dequant(self, side: int) -> np.ndarray:
        """Exact fp64 (code - 128) * scale of every quantized row."""
        c = self.codes[side].astype(np.float64) - CODE_OFFSET
        return c * self.row_scales(side).astype(np.float64)

    def kv(self):
        """[P1] `get_kv`: dequantized rows below L - W, then the recent rows."""
        nq = self.quantized_len()
        out = []
        for side in range(2):
            old = self.dequant(side)[:, :nq]
            out.append(np.concatenate([old, self.rows[side][:, nq:].astype(np.float64)], axis=1))
        return out[0], out[1]


def attention_decode_recent(q: np.ndarray, caches, attn_scale: float) -> np.ndarray:
    """Decode attention over hybrid caches: ``q`` [B, H, D], ``caches`` one
    :class:`RecentWindowCache` per sequence; each query sees its sequence's
    `get_kv` view (all tokens, old ones dequantized).  Returns [B, H, D] fp64."""
    bsz, nh, d = q.shape
    out = np.zeros((bsz, nh, d), dtype=np.float64)
    for b, c in enumerate(caches):
        if c.seq_len() == 0:
            continue
        k, v = c.kv()
        for h in range(nh):
            g = kv_head_of(h, nh, k.shape[0])
            out[b, h] = softmax_attend(q[b, h].astype(np.float64), k[g], v[g], attn_scale)
    return out


def recent_memory_bytes(num_kv_heads: int, head_dim: int, length: int, window: int,
                        group: int = 0, scale_bytes: int = 2) -> int:
    """[P1] `OptimizedQuantizedKvCache::memory_bytes` for one sequence: one
    byte per quantized element, ``scale_bytes`` per scale (the page stores
    them as BF16, 2 bytes), two bytes per recent element; K and V."""
    nq = recent_split(length, window)
    nr = length - nq
    g = 1 if group == 0 else head_dim // group
    return 2 * (num_kv_heads * nq * head_dim + scale_bytes * num_kv_heads * nq * g
                + 2 * num_kv_heads * nr * head_dim)


def recent_split(length: int, window: int) -> int:
    """Number of INT8 rows of a hybrid sequence of ``length`` tokens: every
    position below length - W is quantized, the rest are recent."""
    return max(0, int(length) - int(window))


# ----------------------------------------------------------------------------
# Sizing
# ----------------------------------------------------------------------------

def cache_bytes(num_kv_heads: int, max_len: int, head_dim: int, group: int,
                batch: int = 1, layers: int = 1) -> int:
    """Bytes of u8 codes plus fp32 scales for K and V.

    [P2] `init_kv_cache_q8_gpu` / `kv_cache_q8_memory_bytes`:
    layers * 2 * (values + 4 * scales), with values = kvh*max_len*dim and
    scales = kvh*max_len*(dim/32) for group-32 (dim/dim = 1 per token).
    """
    per_row_scales = 1 if group == 0 else head_dim // group
    values = num_kv_heads * max_len * head_dim
    scales = num_kv_heads * max_len * per_row_scales
    return layers * batch * 2 * (values + 4 * scales)


def fp32_equivalent_bytes(num_kv_heads: int, max_len: int, head_dim: int,
                          batch: int = 1, layers: int = 1) -> int:
    """[P2] `kv_cache_fp32_equivalent_bytes`: layers*2*kvh*max_len*dim*4."""
    return layers * batch * 2 * num_kv_heads * max_len * head_dim * 4


def codes_bytes(num_kv_heads: int, max_len: int, head_dim: int,
                batch: int = 1, layers: int = 1) -> int:
    """u8 code bytes alone for K and V (also the whole of an FP8 cache, which
    keeps no scales: [P5] `KVCacheFormat::uses_scales`)."""
    return layers * batch * 2 * num_kv_heads * max_len * head_dim


def reference_attention_fp(q, k, v, attn_scale):
    """Unquantized fp64 decode attention on raw K/V (used to check the
    quantized path against the [P4] test tolerance); same definition as
    :func:`attention_decode` with K/V taken as given."""
    return attention_decode(q, np.asarray(k, np.float64), np.asarray(v, np.float64),
                            [k.shape[2]] * q.shape[0], attn_scale)


__all__ = [name for name in dir() if not name.startswith("_") and name not in ("math", "np", "annotations")]
