"""Pins for the CPU oracle: values the pages print, closed forms, brute force.

None of these tests retype the oracle's formulas: each checks it against
something fixed independently (a page's worked example and threshold, exact
rational arithmetic, an exhaustive search, a library cast, or a closed-form
attention result).
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_examples.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ----------------------------------------------------------------------------
# quantizer: page examples
# ----------------------------------------------------------------------------

def _grid_input():
    n = 2 * 3 * 64
    i = np.arange(n)
    q = (i * 37) % 255 - 127
    x = (q * 0.5).astype(np.float32)
    x[::32] = np.float32(63.5)
    return x.reshape(1, 2, 3, 64), q


@pytest.mark.parametrize("group", [32, 0])
def test_grid_roundtrip_exact(golden, group):
    """combs-models kv.rs `kv_quant_roundtrip_exact_on_grid_values`: absmax
    63.5 per group (and per row) forces scale 0.5, so codes are 2x+128 and the
    round trip is exact."""
    x, qgrid = _grid_input()
    codes, scales = orc.quantize(x, group)
    assert np.all(scales == np.float32(0.5))
    expect = (qgrid + 128).astype(np.uint8)
    expect[::32] = 255
    assert np.array_equal(codes.reshape(-1), expect)
    back = orc.dequantize_exact(codes, scales)
    assert np.max(np.abs(back - x)) < golden["grid_roundtrip"]["tolerance"]
    assert np.array_equal(orc.dequantize_f32(codes, scales), x)


def test_tie_rounding_half_away_from_zero():
    """Ties of x/s round away from zero (Rust `f32::round` in abaddon
    kv_cache_quant_cuda.rs `quantize_tensor`), and the rounding happens before
    the +128 offset: -0.5 -> -1 -> code 127 (rounding after the offset would
    give 128)."""
    row = np.zeros(32, np.float32)
    row[0] = 63.5                                   # s = 0.5 exactly
    row[1:9] = [0.25, -0.25, 0.75, -0.75, 1.25, -1.25, 0.0, -0.0]
    codes, s = orc.quantize(row[None], 32)
    assert s[0, 0] == np.float32(0.5)
    assert list(codes[0, :9]) == [255, 129, 127, 130, 126, 131, 125, 128, 128]


def test_half_step_bound(golden):
    """combs-models kv.rs `kv_quant_error_bounded_by_half_step`: error at
    most absmax/254 + 1e-6 per 32-group; also the tighter fp32 bound
    (s/2)(1 + 2^-15) per element."""
    n = 2 * 5 * 64
    i = np.arange(n, dtype=np.int64)
    x = (((i * 7919) % 1000).astype(np.float32) / np.float32(250.0) - np.float32(2.0)).astype(np.float32)
    x = x.reshape(1, 2, 5, 64)
    codes, scales = orc.quantize(x, 32)
    back = orc.dequantize_f32(codes, scales).astype(np.float64)
    xf = x.astype(np.float64).reshape(-1, 32)
    bf = back.reshape(-1, 32)
    absmax = np.max(np.abs(xf), axis=1, keepdims=True)
    assert np.all(np.abs(xf - bf) <= absmax / 254.0 + golden["half_step_bound"]["slack"])
    s = np.repeat(scales.reshape(-1, 1).astype(np.float64), 32, axis=1)
    assert np.all(np.abs(xf - bf) <= (s / 2) * (1 + 2.0 ** -15))


def test_candle_roundtrip(golden):
    """abaddon 0.2.0-rc.2 kv_cache_quant.rs roundtrip test: (1,2,8,8), x=(i-64)/64."""
    x = ((np.arange(128, dtype=np.float32) - np.float32(64)) / np.float32(64)).reshape(1, 2, 8, 8)
    codes, scales = orc.quantize(x, 0)
    assert scales.shape == (1, 2, 8, 1)
    err = np.abs(orc.dequantize_f32(codes, scales) - x)
    assert np.max(err) < golden["candle_roundtrip"]["tolerance"]


def test_int8_roundtrip_relative(golden):
    """llama-gguf kv_quantized.rs `test_int8_roundtrip`: 128 values 0.1 i - 6.4."""
    x = (np.arange(128, dtype=np.float32) * np.float32(0.1) - np.float32(6.4)).astype(np.float32)
    codes, scales = orc.quantize(x[None], 0)
    dec = orc.dequantize_f32(codes, scales)[0]
    for o, d in zip(x, dec):
        err = abs(float(o) - float(d))
        rel = err / abs(float(o)) if abs(float(o)) > 1e-6 else err
        assert rel < golden["int8_roundtrip"]["tolerance"]


def test_constant_tokens(golden):
    """llama-gguf kv_quantized.rs `test_shift_left` writes tokens whose
    elements all equal their position: codes are all 255 (128 at pos 0) and
    the read-back is within 0.01."""
    for pos in range(5):
        x = np.full((2, 4), pos, np.float32)
        codes, s = orc.quantize(x, 0)
        assert np.all(codes == (128 if pos == 0 else 255))
        assert np.max(np.abs(orc.dequantize_f32(codes, s) - x)) < golden["constant_tokens"]["tolerance"]


def test_zero_row():
    """All-zero row: absmax floor 1e-8 gives s = fl32(1e-8/127), codes 128, deq 0."""
    codes, s = orc.quantize(np.zeros((1, 64), np.float32), 0)
    assert np.all(codes == 128)
    assert s[0, 0] == np.float32(np.float32(1e-8) / np.float32(127))
    assert np.all(orc.dequantize_f32(codes, s) == 0)


# ----------------------------------------------------------------------------
# quantizer: exact-arithmetic and brute-force pins
# ----------------------------------------------------------------------------

def _is_nearest_f32(result: np.float32, exact: Fraction) -> bool:
    """True when ``result`` is a float32 nearest to ``exact`` (ties: even)."""
    r = Fraction(float(result))
    up = Fraction(float(np.nextafter(result, np.float32(np.inf), dtype=np.float32)))
    dn = Fraction(float(np.nextafter(result, np.float32(-np.inf), dtype=np.float32)))
    d = abs(r - exact)
    if d > abs(up - exact) or d > abs(dn - exact):
        return False
    if d == abs(up - exact) or d == abs(dn - exact):        # tie: mantissa even
        return (np.float32(result).view(np.uint32) & 1) == 0
    return True


def test_scale_and_quotient_are_correctly_rounded():
    """s and x/s are the fp32 values nearest to the exact rationals m/127 and
    x/s (IEEE division), checked with exact rational arithmetic."""
    rng = np.random.default_rng(123)
    x = (rng.standard_normal((40, 64)) * rng.choice([1e-3, 1.0, 37.0], size=(40, 1))).astype(np.float32)
    codes, s = orc.quantize(x, 0)
    for r in range(x.shape[0]):
        m = max(float(abs(v)) for v in x[r])
        assert _is_nearest_f32(s[r, 0], Fraction(m) / 127)
        for j in range(0, 64, 7):
            y = np.float32(x[r, j] / s[r, 0])
            assert _is_nearest_f32(y, Fraction(float(x[r, j])) / Fraction(float(s[r, 0])))


def test_rounding_brute_force():
    """Each code is the integer nearest the fp32 quotient (ties away from
    zero), found by exhaustive search over [-127, 127]."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 32)).astype(np.float32)
    # plant exact ties: quotients k + 1/2 need s with a short mantissa
    x[:8, 0] = np.float32(63.5)
    x[:8, 1:6] = np.float32([0.25, -0.75, 12.25, -30.75, 0.5])
    codes, s = orc.quantize(x, 32)
    cand = np.arange(-127, 128)
    for r in range(x.shape[0]):
        for j in range(32):
            y = float(np.float32(x[r, j] / s[r, 0]))
            dist = np.abs(cand - y)
            best = np.flatnonzero(dist == dist.min())
            q = cand[best[np.argmax(np.abs(cand[best]))]]
            assert codes[r, j] == q + 128, (r, j, y)


def _nearest_f32_of(exact: Fraction) -> np.float32:
    """The fp32 value nearest to an exact rational (ties to even), found by
    exact comparison among the neighbours of a first guess."""
    c = np.float32(float(exact))
    cands = [c]
    for _ in range(2):
        cands.append(np.nextafter(cands[-1], np.float32(np.inf), dtype=np.float32))
    dn = c
    for _ in range(2):
        dn = np.nextafter(dn, np.float32(-np.inf), dtype=np.float32)
        cands.append(dn)
    best = [v for v in cands if _is_nearest_f32(v, exact)]
    assert len(best) == 1
    return best[0]


def _round_away(y: float) -> int:
    return int(math.copysign(math.floor(abs(y) + 0.5), y))


def test_division_not_reciprocal_multiply():
    """Codes come from the correctly rounded quotient x/s.  With s = 3
    (absmax 381) some x just below (k + 1/2) * 3 round one way through x/s and
    the other way through x * fl32(1/s); expected codes are derived with exact
    rational arithmetic."""
    s = np.float32(3.0)
    recip = np.float32(1) / s
    picks = []
    for k in range(0, 126):
        x = np.float32((k + 0.5) * 3)
        for _ in range(30):
            x = np.nextafter(x, np.float32(-np.inf), dtype=np.float32)
        for _ in range(60):
            if _round_away(np.float32(x / s)) != _round_away(np.float32(x * recip)):
                picks.append(x)
            x = np.nextafter(x, np.float32(np.inf), dtype=np.float32)
    assert len(picks) >= 8
    row = np.zeros(len(picks) + 1 + (-(len(picks) + 1)) % 32, np.float32)
    row[0] = np.float32(381.0)
    row[1:len(picks) + 1] = picks
    row[len(picks) + 1:] = -np.float32(picks[0])
    codes, sc = orc.quantize(row[None], 0)
    assert sc[0, 0] == s
    for j, x in enumerate(row):
        y = _nearest_f32_of(Fraction(float(x)) / 3)
        assert codes[0, j] == _round_away(float(y)) + 128, (j, float(x))


def test_code_range_and_absmax_code():
    """Codes lie in [1, 255]; each row's absmax element maps to 1 or 255."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((256, 128)).astype(np.float32)
    codes, _ = orc.quantize(x, 0)
    assert codes.min() >= 1 and codes.max() <= 255
    am = np.argmax(np.abs(x), axis=1)
    assert np.all(np.isin(codes[np.arange(256), am], [1, 255]))
    codes32, _ = orc.quantize(x, 32)
    assert codes32.min() >= 1


def test_group_scales_independent():
    """Group-32 scales see only their own 32 elements (the [P4] group rule):
    changing one group leaves the others' codes and scales untouched."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 128)).astype(np.float32)
    c1, s1 = orc.quantize(x, 32)
    x2 = x.copy()
    x2[:, 32:64] *= np.float32(50.0)
    c2, s2 = orc.quantize(x2, 32)
    keep = np.r_[0:32, 64:128]
    assert np.array_equal(c1[:, keep], c2[:, keep])
    assert np.array_equal(s1[:, [0, 2, 3]], s2[:, [0, 2, 3]])
    assert np.all(s2[:, 1] > s1[:, 1])


def test_bf16_rounding_matches_library_cast():
    """The oracle's fp32->bf16 rounding equals torch's CPU cast (RNE),
    including exact ties on both parities."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    x = rng.standard_normal(100000).astype(np.float32) * np.float32(100)
    ties = (np.arange(0, 4096, dtype=np.uint32) << np.uint32(16)) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(np.float32)[10:2000], np.float32([0.0, -0.0, 1.0, -3.5])])
    ours = orc.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(orc.bf16_bits_to_f32(ours), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


# ----------------------------------------------------------------------------
# attention: closed forms and brute force
# ----------------------------------------------------------------------------

def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_single_token_gives_v():
    q = _rand((2, 4, 16), 0)
    k = _rand((2, 2, 1, 16), 1)
    v = _rand((2, 2, 1, 16), 2)
    out = orc.attention_decode(q, k, v, [1, 1], 0.25)
    for h in range(4):
        assert np.allclose(out[:, h], v[:, h // 2, 0], rtol=0, atol=1e-15)


def test_constant_keys_give_mean_v():
    k = np.repeat(_rand((1, 2, 1, 8), 3), 9, axis=2)
    v = _rand((1, 2, 9, 8), 4)
    q = _rand((1, 6, 8), 5)
    out = orc.attention_decode(q, k, v, [9], 0.7)
    for h in range(6):
        assert np.allclose(out[0, h], v[0, h // 3].mean(axis=0), atol=1e-14)


def test_zero_query_and_zero_scale_give_mean_v():
    k = _rand((1, 1, 5, 8), 6)
    v = _rand((1, 1, 5, 8), 7)
    q = np.zeros((1, 1, 8))
    assert np.allclose(orc.attention_decode(q, k, v, [5], 1.0)[0, 0], v[0, 0].mean(0), atol=1e-14)
    q = _rand((1, 1, 8), 8)
    assert np.allclose(orc.attention_decode(q, k, v, [5], 0.0)[0, 0], v[0, 0].mean(0), atol=1e-14)


def test_two_token_closed_form():
    q = _rand((1, 1, 4), 9)
    k = _rand((1, 1, 2, 4), 10)
    v = _rand((1, 1, 2, 4), 11)
    sc = 0.3
    s0 = sc * sum(q[0, 0, d] * k[0, 0, 0, d] for d in range(4))
    s1 = sc * sum(q[0, 0, d] * k[0, 0, 1, d] for d in range(4))
    p0 = 1.0 / (1.0 + math.exp(s1 - s0))
    expect = p0 * v[0, 0, 0] + (1 - p0) * v[0, 0, 1]
    assert np.allclose(orc.attention_decode(q, k, v, [2], sc)[0, 0], expect, atol=1e-14)


def test_gqa_head_mapping():
    """Query head h reads KV head h // (H/KVH): with V constant per KV head,
    each output equals its group's constant (h % KVH would fail)."""
    H, KVH, L, D = 8, 2, 5, 4
    v = np.zeros((1, KVH, L, D))
    v[0, 0] = 1.0
    v[0, 1] = -2.0
    out = orc.attention_decode(_rand((1, H, D), 12), _rand((1, KVH, L, D), 13), v, [L], 0.5)
    assert np.allclose(out[0, :4], 1.0) and np.allclose(out[0, 4:], -2.0)


def test_dominant_key_and_length_limit():
    """A key with a huge score takes all the weight; keys at t >= L are ignored."""
    D = 8
    q = np.ones((1, 1, D))
    k = np.zeros((1, 1, 6, D))
    k[0, 0, 2] = 100.0
    k[0, 0, 5] = 1000.0                       # beyond L = 4: must not matter
    v = _rand((1, 1, 6, D), 14)
    out = orc.attention_decode(q, k, v, [4], 1.0)
    assert np.allclose(out[0, 0], v[0, 0, 2], atol=1e-12)


def test_token_permutation_invariance():
    q = _rand((1, 2, 8), 15)
    k = _rand((1, 1, 11, 8), 16)
    v = _rand((1, 1, 11, 8), 17)
    perm = np.random.default_rng(0).permutation(11)
    a = orc.attention_decode(q, k, v, [11], 0.4)
    b = orc.attention_decode(q, k[:, :, perm], v[:, :, perm], [11], 0.4)
    assert np.allclose(a, b, atol=1e-13)


def _loop_attention(q, k, v, scale):
    """Brute force, scalar loops with math.exp (no NumPy reductions)."""
    scores = [scale * sum(q[d] * k[t][d] for d in range(len(q))) for t in range(len(k))]
    m = max(scores)
    w = [math.exp(s - m) for s in scores]
    z = sum(w)
    return [sum(w[t] * v[t][d] for t in range(len(k))) / z for d in range(len(q))]


def test_brute_force_tiny_decode_and_chunk():
    rng = np.random.default_rng(21)
    B, H, KVH, D, L0, n = 2, 4, 2, 5, 3, 4
    q = rng.standard_normal((B, H, n, D))
    k = rng.standard_normal((B, KVH, L0 + n, D))
    v = rng.standard_normal((B, KVH, L0 + n, D))
    out = orc.attention_chunk(q, k, v, [L0, L0], True, 0.37)
    for b in range(B):
        for h in range(H):
            g = h // 2
            for i in range(n):
                vis = L0 + i + 1
                ref = _loop_attention(list(q[b, h, i]), [list(r) for r in k[b, g, :vis]],
                                      [list(r) for r in v[b, g, :vis]], 0.37)
                assert np.allclose(out[b, h, i], ref, atol=1e-13)
    dec = orc.attention_decode(q[:, :, 0], k, v, [2, 5], 0.37)
    for b, length in enumerate([2, 5]):
        for h in range(H):
            ref = _loop_attention(list(q[b, h, 0]), [list(r) for r in k[b, h // 2, :length]],
                                  [list(r) for r in v[b, h // 2, :length]], 0.37)
            assert np.allclose(dec[b, h], ref, atol=1e-13)


def test_chunk_rows_equal_decode_and_noncausal():
    rng = np.random.default_rng(22)
    B, H, KVH, D, L0, n = 1, 2, 1, 8, 6, 5
    q = rng.standard_normal((B, H, n, D))
    k = rng.standard_normal((B, KVH, L0 + n, D))
    v = rng.standard_normal((B, KVH, L0 + n, D))
    ch = orc.attention_chunk(q, k, v, [L0], True, 0.5)
    for i in range(n):
        assert np.allclose(ch[:, :, i], orc.attention_decode(q[:, :, i], k, v, [L0 + i + 1], 0.5), atol=1e-14)
    nc = orc.attention_chunk(q, k, v, [L0], False, 0.5)
    for i in range(n):
        assert np.allclose(nc[:, :, i], orc.attention_decode(q[:, :, i], k, v, [L0 + n], 0.5), atol=1e-14)


# ----------------------------------------------------------------------------
# cache layouts and the page's end-to-end tolerance
# ----------------------------------------------------------------------------

def _kv_tok(i, n_kv, d, salt):
    j = np.arange(n_kv * d)
    return ((((i * 7 + j * 3 + salt) % 13) / 13.0) - 0.5).astype(np.float32).reshape(n_kv, d)


def _q_tok(i, n_q, d):
    j = np.arange(n_q * d)
    return ((((i * 11 + j * 5) % 17) / 17.0) - 0.5).astype(np.float32).reshape(n_q, d)


def test_quantized_paged_matches_fp(golden):
    """combs-models kv.rs `quantized_paged_cache_matches_fp_within_tolerance`:
    prefill 20 tokens (crossing the 16-token page boundary), then decode
    20..29; quantized (group-32) paged attention stays within 1e-2 of fp
    attention.  The paged arena, written through a scattered block table,
    also holds exactly the codes a contiguous cache holds."""
    g = golden["quantized_paged_vs_fp"]
    n_kv, n_q, d = g["n_kv"], g["n_q"], g["head_dim"]
    scale = 0.9 / math.sqrt(d)
    total = g["decode_to"]
    K = np.stack([_kv_tok(i, n_kv, d, 0) for i in range(total)], axis=1)[None]   # [1,KVH,T,D]
    V = np.stack([_kv_tok(i, n_kv, d, 5) for i in range(total)], axis=1)[None]
    Q = np.stack([_q_tok(i, n_q, d) for i in range(total)], axis=1)[None]        # [1,H,T,D]
    nblocks = 4
    table = np.array([[7, 2, 5, 0]], np.int32)
    arena = [np.zeros((8, n_kv, 16, d), np.uint8), np.zeros((8, n_kv, 16, 1), np.float32),
             np.zeros((8, n_kv, 16, d), np.uint8), np.zeros((8, n_kv, 16, 1), np.float32)]
    cont = [np.zeros((1, n_kv, nblocks * 16, d), np.uint8), np.zeros((1, n_kv, nblocks * 16, 1), np.float32),
            np.zeros((1, n_kv, nblocks * 16, d), np.uint8), np.zeros((1, n_kv, nblocks * 16, 1), np.float32)]
    # prefill chunk
    orc.paged_append(*arena, table, K[:, :, :20], V[:, :, :20], [0], 32)
    orc.contiguous_append(*cont, K[:, :, :20], V[:, :, :20], [0], 32)
    for pos in range(20, total):
        orc.paged_append(*arena, table, K[:, :, pos:pos + 1], V[:, :, pos:pos + 1], [pos], 32)
        orc.contiguous_append(*cont, K[:, :, pos:pos + 1], V[:, :, pos:pos + 1], [pos], 32)
    L = total
    kc = orc.paged_gather(arena[0], table, 0, L)
    ks = orc.paged_gather(arena[1], table, 0, L)
    vc = orc.paged_gather(arena[2], table, 0, L)
    vs = orc.paged_gather(arena[3], table, 0, L)
    assert np.array_equal(kc, cont[0][0, :, :L]) and np.array_equal(vs, cont[3][0, :, :L])
    k_hat = orc.dequantize_exact(kc, ks)[None]
    v_hat = orc.dequantize_exact(vc, vs)[None]
    # prefill rows 0..19 (causal chunk at ctx 0), then each decode step
    qp = Q[:, :, :20].astype(np.float64)
    a = orc.attention_chunk(qp, k_hat[:, :, :20], v_hat[:, :, :20], [0], True, scale)
    b = orc.attention_chunk(qp, K[:, :, :20].astype(np.float64), V[:, :, :20].astype(np.float64), [0], True, scale)
    assert np.max(np.abs(a - b)) < g["tolerance"]
    for pos in range(20, total):
        a = orc.attention_decode(Q[:, :, pos].astype(np.float64), k_hat, v_hat, [pos + 1], scale)
        b = orc.attention_decode(Q[:, :, pos].astype(np.float64), K.astype(np.float64), V.astype(np.float64),
                                 [pos + 1], scale)
        assert np.max(np.abs(a - b)) < g["tolerance"]


def test_page_slot_arithmetic():
    table = np.array([[3, 9, 1], [0, 2, 4]], np.int32)
    assert orc.page_slot(table, 0, 0) == (3, 0)
    assert orc.page_slot(table, 0, 15) == (3, 15)
    assert orc.page_slot(table, 0, 16) == (9, 0)
    assert orc.page_slot(table, 1, 47) == (4, 15)


def test_sizing_matches_printed_figures(golden):
    """realizar kv_cache_q8_init.rs: the byte formulas, and the printed
    "8.59 GB" / "2.15 GB" read as batch 8 (codes only for the Q8 figure)."""
    s = golden["sizing"]
    kw = dict(num_kv_heads=s["num_kv_heads"], max_len=s["max_len"], head_dim=s["head_dim"],
              layers=s["layers"])
    assert orc.fp32_equivalent_bytes(**kw) == s["per_sequence_fp32_bytes"]
    assert orc.cache_bytes(group=32, **kw) == s["per_sequence_q8_bytes"]
    assert orc.fp32_equivalent_bytes(batch=8, **kw) == s["batch8_fp32_bytes"]
    assert orc.codes_bytes(batch=8, **kw) == s["batch8_codes_bytes"]
    assert orc.cache_bytes(group=32, batch=8, **kw) == s["batch8_q8_total_bytes"]
    assert f"{s['batch8_fp32_bytes'] / 1e9:.2f} GB" == s["printed_fp32"]
    assert f"{s['batch8_codes_bytes'] / 1e9:.2f} GB" == s["printed_q8"]
    # the page's own product, evaluated, is 1.07e9 (garbled figure)
    assert 32 * 2 * 4096 * 8 * 128 * 4 == s["per_sequence_fp32_bytes"]


# ----------------------------------------------------------------------------
# recent-window hybrid cache (abaddon 0.2.0-rc.1 kv_cache_quant_cuda.rs,
# OptimizedQuantizedKvCache)
# ----------------------------------------------------------------------------

def _bf16_values_torch(x):
    """bf16 rounding by the library cast (independent of the oracle's)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def test_recent_window_counts(golden):
    """The quantized / recent split that the page's tests print."""
    for case in golden["recent_window_counts"]["cases"]:
        c = orc.RecentWindowCache(case["kv_heads"], case["head_dim"], case["window"])
        rng = np.random.default_rng(0)
        for n in case["appends"]:
            x = rng.standard_normal((case["kv_heads"], n, case["head_dim"])).astype(np.float32)
            c.append(x, x)
        assert (c.seq_len(), c.quantized_len(), c.recent_len()) == (case["seq_len"], case["quantized"],
                                                                     case["recent"])
        assert orc.recent_split(c.seq_len(), case["window"]) == case["quantized"]


@pytest.mark.parametrize("group", [0, 32])
def test_recent_window_state_is_path_independent(group):
    """Over random append sequences (chunks shorter and longer than the
    window), rows below L - W always hold the codes of their bf16-rounded
    values and the last W rows hold those bf16 values.  The fp32 inputs are
    chosen so that quantizing the raw value would give other codes."""
    rng = np.random.default_rng(1)
    W, KVH, D, T = 5, 2, 64, 41
    k = (rng.standard_normal((KVH, T, D)) * 3).astype(np.float32)
    v = (rng.standard_normal((KVH, T, D)) * 0.3).astype(np.float32)
    kb, vb = _bf16_values_torch(k), _bf16_values_torch(v)
    assert not np.array_equal(orc.quantize(k, group)[0], orc.quantize(kb, group)[0])
    for _ in range(10):
        c = orc.RecentWindowCache(KVH, D, W, group)
        L = 0
        while L < T:
            n = min(int(rng.integers(1, 13)), T - L)
            c.append(k[:, L:L + n], v[:, L:L + n])
            L += n
            nq = max(0, L - W)
            kc, ks = orc.quantize(kb[:, :nq], group)
            vc, vs = orc.quantize(vb[:, :nq], group)
            assert np.array_equal(c.k_codes, kc) and np.array_equal(c.v_codes, vc)
            assert np.array_equal(c.k_scales, ks) and np.array_equal(c.v_scales, vs)
            assert np.array_equal(c.k_recent, kb[:, nq:L]) and np.array_equal(c.v_recent, vb[:, nq:L])


def test_recent_window_zero_is_plain_int8():
    """W = 0 quantizes every row on arrival: the plain INT8 cache."""
    rng = np.random.default_rng(2)
    x = _bf16_values_torch(rng.standard_normal((2, 9, 32)))
    c = orc.RecentWindowCache(2, 32, 0)
    c.append(x[:, :4], x[:, :4])
    c.append(x[:, 4:], x[:, 4:])
    assert c.recent_len() == 0
    assert np.array_equal(c.k_codes, orc.quantize(x, 0)[0])


def test_recent_attention_all_recent_brute_force():
    """L <= W: attention over the bf16 rows, computed here with Python floats."""
    rng = np.random.default_rng(3)
    KVH, H, D, L = 1, 2, 8, 5
    k = rng.standard_normal((KVH, L, D)).astype(np.float32)
    v = rng.standard_normal((KVH, L, D)).astype(np.float32)
    q = _bf16_values_torch(rng.standard_normal((1, H, D)))
    c = orc.RecentWindowCache(KVH, D, 8)
    c.append(k, v)
    got = orc.attention_decode_recent(q, [c], 0.3)
    kb, vb = _bf16_values_torch(k)[0], _bf16_values_torch(v)[0]
    for h in range(H):
        s = [0.3 * sum(float(q[0, h, d]) * float(kb[t, d]) for d in range(D)) for t in range(L)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = sum(w)
        for d in range(D):
            ref = sum(w[t] * float(vb[t, d]) for t in range(L)) / z
            assert abs(got[0, h, d] - ref) < 1e-12


def test_recent_attention_equal_keys_give_mean_v():
    """Keys on the quantization grid and bf16-exact (integers, absmax 127)
    dequantize to themselves, so old and recent keys are equal, the weights
    are uniform, and the output is the mean of the old (dequantized) and
    recent (bf16) value rows."""
    rng = np.random.default_rng(4)
    KVH, D, L, W = 1, 32, 11, 4
    row = rng.integers(-127, 128, size=D).astype(np.float32)
    row[0] = 127.0
    k = np.repeat(row[None, None, :], L, axis=1)
    v = rng.standard_normal((KVH, L, D)).astype(np.float32)
    c = orc.RecentWindowCache(KVH, D, W)
    c.append(k[:, :6], v[:, :6])
    c.append(k[:, 6:], v[:, 6:])
    assert c.quantized_len() == L - W
    assert np.array_equal(orc.dequantize_exact(c.k_codes, c.k_scales)[0], k[0, :L - W].astype(np.float64))
    vb = _bf16_values_torch(v)[0]
    vc, vs = orc.quantize(vb[:L - W], 0)
    rows = np.concatenate([orc.dequantize_exact(vc, vs), vb[L - W:].astype(np.float64)])
    q = rng.standard_normal((1, 3, D))
    out = orc.attention_decode_recent(q, [c], 0.05)
    for h in range(3):
        assert np.allclose(out[0, h], rows.mean(axis=0), rtol=0, atol=1e-13)


def test_recent_memory_savings(golden):
    """test_memory_savings: W = 16, 8 KV heads, D = 128, 1000 tokens in BF16
    save more than 1.5x; by hand: 984 quantized rows (1 byte per element, a
    2-byte scale per row) and 16 recent rows (2 bytes per element), K and V."""
    g = golden["recent_window_savings"]
    got = orc.recent_memory_bytes(g["kv_heads"], g["head_dim"], g["tokens"], g["window"])
    by_hand = 2 * (8 * 984 * 128 + 2 * 8 * 984 + 2 * 8 * 16 * 128)
    assert got == by_hand == 2_112_256
    full = g["tokens"] * g["kv_heads"] * g["head_dim"] * 2 * 2
    assert full / got > g["min_savings"]


# ----------------------------------------------------------------------------
# per-head and per-channel block scales (abaddon kv_cache_quant_cuda.rs,
# QuantGranularity / quantize_with_granularity)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("gran", ["head", "channel"])
def test_block_modes_page_counts(golden, gran):
    """The page's test_per_head_quantization (W = 4, 10 tokens, 4 KV heads,
    head_dim 64: 6 quantized, 4 recent, a [4, 10, 64] get_kv view) and the
    other printed counts, with blocks of 4 rows (the reading needs B <= W + 1)."""
    for case in golden["recent_window_counts"]["cases"]:
        c = orc.BlockRecentCache(case["kv_heads"], case["head_dim"], case["window"], gran, block=4)
        rng = np.random.default_rng(0)
        for n in case["appends"]:
            x = rng.standard_normal((case["kv_heads"], n, case["head_dim"])).astype(np.float32)
            c.append(x, x)
        assert (c.seq_len(), c.quantized_len(), c.recent_len()) == (case["seq_len"], case["quantized"],
                                                                     case["recent"])
        k, v = c.kv()
        assert k.shape == v.shape == (case["kv_heads"], case["seq_len"], case["head_dim"])


def test_block_modes_need_a_window_of_block_minus_one():
    with pytest.raises(ValueError):
        orc.BlockRecentCache(1, 32, 14, "head", block=16)
    orc.BlockRecentCache(1, 32, 15, "head", block=16)


@pytest.mark.parametrize("gran", ["head", "channel"])
def test_block_scales_half_step_bound(gran):
    """Every dequantized element lies within (s/2)(1 + 2^-15) of its bf16
    input, s its own block (per head) or block-channel scale; per head that
    s is max over the block / 127, per channel max over the block's column."""
    rng = np.random.default_rng(11)
    KVH, D, B, W, T = 2, 64, 16, 20, 100
    x = (rng.standard_normal((KVH, T, D)) * np.exp(rng.uniform(-3, 3, (1, T, D)))).astype(np.float32)
    c = orc.BlockRecentCache(KVH, D, W, gran, block=B)
    c.append(x[:, :37], x[:, :37])
    c.append(x[:, 37:], x[:, 37:])
    xb = _bf16_values_torch(x).astype(np.float64)
    nrow = c.codes[0].shape[1]
    # the blocks are quantized from the rows' bf16 values (library cast),
    # with the per-token quantizer's steps over the block's reduction set
    blocks = xb[:, :nrow].astype(np.float32).reshape(KVH, nrow // B, B, D)
    if gran == "head":
        want_codes = orc.quantize(blocks.reshape(KVH, nrow // B, B * D), 0)[0].reshape(KVH, nrow, D)
    else:
        want_codes = np.swapaxes(orc.quantize(np.swapaxes(blocks, 2, 3), 0)[0], 2, 3).reshape(KVH, nrow, D)
    assert np.array_equal(c.codes[0], want_codes)
    err = np.abs(c.dequant(0) - xb[:, :nrow])
    s = c.row_scales(0).astype(np.float64)
    assert np.all(err <= s / 2 * (1 + 2.0 ** -15))
    for j in range(nrow // B):
        blk = np.abs(xb[:, j * B:(j + 1) * B])
        want = blk.max(axis=(1, 2)) if gran == "head" else blk.max(axis=1)
        got = c.scales[0][:, j]
        # s = fl32(max / 127): within half an fp32 ulp of the exact quotient
        assert np.all(np.abs(got.astype(np.float64) - want / 127) <= np.spacing(got) / 2 + 1e-300)


def test_block_head_with_one_row_blocks_is_per_token():
    """B = 1: the per-head block maximum is the row maximum, so codes and
    scales are those of the per-token quantizer."""
    rng = np.random.default_rng(12)
    x = _bf16_values_torch(rng.standard_normal((3, 20, 32)))
    c = orc.BlockRecentCache(3, 32, 0, "head", block=1)
    c.append(x, x)
    kc, ks = orc.quantize(x, 0)
    assert np.array_equal(c.codes[0], kc) and np.array_equal(c.scales[0], ks[..., 0])


def test_block_channel_constant_rows_closed_form():
    """A block of B equal rows u: per channel each scale is |u_d| / 127 and
    every code is 128 + 127 sign(u_d); per head the scale is max|u| / 127."""
    rng = np.random.default_rng(13)
    D, B = 32, 16
    u = _bf16_values_torch(rng.standard_normal(D))
    u[3] = 0.0
    x = np.repeat(u[None, None, :], 2 * B - 1, axis=1).astype(np.float32)
    c = orc.BlockRecentCache(1, D, B - 1, "channel", block=B)
    c.append(x, x)
    assert c.codes[0].shape[1] == B  # L - W = B: block 0 alone has started to leave
    want = np.where(u > 0, 255, np.where(u < 0, 1, 128))
    assert np.all(c.codes[0][0] == want[None, :])
    mag = np.maximum(np.abs(u), np.float32(1e-8))
    assert np.array_equal(c.scales[0][0, 0], (mag / np.float32(127)).astype(np.float32))
    h = orc.BlockRecentCache(1, D, B - 1, "head", block=B)
    h.append(x, x)
    assert h.scales[0][0, 0] == np.float32(np.max(np.abs(u)) / np.float32(127))


@pytest.mark.parametrize("gran", ["head", "channel"])
def test_block_state_is_history_independent(gran):
    """The state depends on the rows alone: any chunking of the appends gives
    the same codes, scales and get_kv view; and changing a row changes no
    code outside its block."""
    rng = np.random.default_rng(14)
    KVH, D, W, B, T = 2, 32, 17, 16, 90
    k = rng.standard_normal((KVH, T, D)).astype(np.float32)
    v = rng.standard_normal((KVH, T, D)).astype(np.float32)
    ref = orc.BlockRecentCache(KVH, D, W, gran, block=B)
    ref.append(k, v)
    for trial in range(6):
        c = orc.BlockRecentCache(KVH, D, W, gran, block=B)
        L = 0
        while L < T:
            n = min(int(rng.integers(1, 25)), T - L)
            c.append(k[:, L:L + n], v[:, L:L + n])
            L += n
        for side in range(2):
            assert np.array_equal(c.codes[side], ref.codes[side])
            assert np.array_equal(c.scales[side], ref.scales[side])
        assert all(np.array_equal(a, b) for a, b in zip(c.kv(), ref.kv()))
    k2 = k.copy()
    k2[:, 20] *= 8.0  # row 20: block 1
    c = orc.BlockRecentCache(KVH, D, W, gran, block=B)
    c.append(k2, v)
    diff = np.any(c.codes[0] != ref.codes[0], axis=(0, 2))
    assert diff[16:32].any() and not diff[:16].any() and not diff[32:].any()


# ----------------------------------------------------------------------------
# sliding-window attention (combs-models kv.rs, attention_opts window)
# ----------------------------------------------------------------------------

def _sliding_layer_outputs(K, V, Q, window, scale, prefill, steps):
    """The page's sliding layer, step by step with Python floats: a store of
    the last window - 1 (key, value) pairs; each call concatenates the store
    with the new tokens, re-bases the query positions by the first stored
    key's absolute position, masks keys after the query or at least window
    positions before it, attends, then keeps the trailing window - 1 tokens.
    K/V: [KVH, T, D]; Q: [H, T, D].  Returns {position: [H, D]}."""
    n_kv, _, d = K.shape
    n_q = Q.shape[0]
    store = []   # absolute positions held by the sliding store
    outs = {}
    calls = [(0, prefill)] + [(p, 1) for p in range(prefill, steps)]
    for pos, seq in calls:
        full = store + list(range(pos, pos + seq))
        kv_offset = pos + seq - len(full)
        for i in range(seq):
            qpos = pos - kv_offset + i          # query position in the concat
            o = np.zeros((n_q, d))
            for h in range(n_q):
                g = h // (n_q // n_kv)
                s = []
                for kpos in range(len(full)):
                    forbidden = kpos > qpos or kpos + window - 1 < qpos
                    s.append(-math.inf if forbidden else
                             scale * sum(float(Q[h, pos + i, e]) * float(K[g, full[kpos], e]) for e in range(d)))
                m = max(s)
                w = [math.exp(x - m) if x != -math.inf else 0.0 for x in s]
                z = sum(w)
                for e in range(d):
                    o[h, e] = sum(w[k] * float(V[g, full[k], e]) for k in range(len(full))) / z
            outs[pos + i] = o
        keep = min(len(full), window - 1)
        store = full[len(full) - keep:]
    return outs


def test_sliding_layer_matches_masked_global(golden):
    """combs-models `sliding_layer_matches_masked_global`: the evicting
    sliding layer equals attention over everything with the window applied
    as a mask (the oracle's definition), through a prefill chunk longer than
    the window and decode steps well past it."""
    g = golden["sliding_vs_masked_global"]
    n_kv, n_q, d, w = g["n_kv"], g["n_q"], g["head_dim"], g["window"]
    scale = 0.9 / math.sqrt(d)
    T = g["decode_to"]
    K = np.stack([_kv_tok(i, n_kv, d, 0) for i in range(T)], axis=1)   # [KVH, T, D]
    V = np.stack([_kv_tok(i, n_kv, d, 5) for i in range(T)], axis=1)
    Q = np.stack([_q_tok(i, n_q, d) for i in range(T)], axis=1)        # [H, T, D]
    sliding = _sliding_layer_outputs(K, V, Q, w, scale, g["prefill"], T)
    P = g["prefill"]
    chunk = orc.attention_chunk(Q[None, :, :P].astype(np.float64), K[None].astype(np.float64),
                                V[None].astype(np.float64), [0], True, scale, window=w)
    for i in range(P):
        assert np.allclose(chunk[0, :, i], sliding[i], rtol=0, atol=1e-12), i
    for pos in range(P, T):
        dec = orc.attention_decode(Q[None, :, pos].astype(np.float64), K[None].astype(np.float64),
                                   V[None].astype(np.float64), [pos + 1], scale, window=w)
        assert np.allclose(dec[0], sliding[pos], rtol=0, atol=1e-12), pos


def test_window_closed_forms():
    """Window 1: each query sees only its own key, so the output is its V
    row.  A window at least the length changes nothing."""
    rng = np.random.default_rng(61)
    k = rng.standard_normal((1, 2, 9, 8))
    v = rng.standard_normal((1, 2, 9, 8))
    q = rng.standard_normal((1, 4, 8))
    one = orc.attention_decode(q, k, v, [9], 0.5, window=1)
    for h in range(4):
        assert np.allclose(one[0, h], v[0, h // 2, 8], rtol=0, atol=1e-15)
    assert np.array_equal(orc.attention_decode(q, k, v, [9], 0.5, window=9), orc.attention_decode(q, k, v, [9], 0.5))
    qc = rng.standard_normal((1, 4, 3, 8))
    c1 = orc.attention_chunk(qc, k, v, [6], True, 0.5, window=1)
    for i in range(3):
        for h in range(4):
            assert np.allclose(c1[0, h, i], v[0, h // 2, 6 + i], rtol=0, atol=1e-15)
    assert np.array_equal(orc.attention_chunk(qc, k, v, [6], True, 0.5, window=9),
                          orc.attention_chunk(qc, k, v, [6], True, 0.5))


# ----------------------------------------------------------------------------
# bf16-stored per-token scales (abaddon 0.2.0-rc.1 kv_cache_quant_cuda.rs,
# CudaQuantizedKvCache::quantize_tensor)
# ----------------------------------------------------------------------------

def test_bf16_scale_storage():
    """The codes come from the fp32 scale (half-step bound against it), the
    stored scale is torch's bf16 rounding of it, and dequantizing with the
    stored scale stays within s/2 + 127 |s - s_bf16|, a bound that can
    exceed s/2 (the page's quantize/dequantize mismatch)."""
    import torch
    rng = np.random.default_rng(91)
    x = (rng.standard_normal((4, 3, 50, 128)) * rng.uniform(0.01, 30, (4, 3, 50, 1))).astype(np.float32)
    codes, sbits = orc.quantize_bf16_scale(x)
    m = np.maximum(np.abs(x).max(axis=-1, keepdims=True), np.float32(1e-8))
    s32 = (m / np.float32(127.0)).astype(np.float32)
    want_bits = torch.from_numpy(s32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(sbits, want_bits)
    c = codes.astype(np.float64) - 128
    assert np.all(np.abs(x - c * s32.astype(np.float64)) <= s32.astype(np.float64) * (0.5 + 2 ** -20))
    sb = orc.bf16_bits_to_f32(sbits).astype(np.float64)
    err = np.abs(x - orc.dequantize_exact(codes, orc.bf16_bits_to_f32(sbits)))
    bound = s32 * 0.5 + 127 * np.abs(s32 - sb)
    assert np.all(err <= bound * (1 + 2 ** -20))
    assert np.any(err > s32 * 0.5 * (1 + 2 ** -10))


# ----------------------------------------------------------------------------
# FP8 codes (llama-gguf 0.14.0 kv_quantized.rs, quantize_fp8_* / dequantize_fp8_*)
# ----------------------------------------------------------------------------

FP8_TORCH = {"e4m3": "float8_e4m3fn", "e5m2": "float8_e5m2"}
# below these magnitudes every finite input has a finite code on the page
FP8_FINITE_LIMIT = {"e4m3": 480.0, "e5m2": 65536.0}


def _torch_fp8_values(fmt):
    torch = pytest.importorskip("torch")
    c = np.arange(256, dtype=np.uint8)
    return torch.from_numpy(c).view(getattr(torch, FP8_TORCH[fmt])).float().numpy().astype(np.float64)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_decode_matches_library_cast(fmt):
    """All 256 codes decode to torch's OCP float8 value (NaN where it is NaN,
    +/-inf for E5M2's infinities); the page decodes negative zero as +0."""
    lib = _torch_fp8_values(fmt)
    ours = orc.fp8_decode(np.arange(256, dtype=np.uint8), fmt)
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert np.array_equal(ours[ok], lib[ok])
    assert ours[0x80] == 0.0 and not np.signbit(ours[0x80])


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_encode_cuts_toward_zero(fmt):
    """Below the format's NaN/inf band the code decodes to the representable
    value of largest magnitude not above |x|, with x's sign: truncation onto
    the grid that torch's cast defines (grid points, their fp32 neighbours,
    subnormals and random magnitudes over 10 decades)."""
    vals = _torch_fp8_values(fmt)
    grid = np.unique(vals[np.isfinite(vals) & (vals >= 0)])
    rng = np.random.default_rng(71)
    g32 = grid.astype(np.float32)
    x = np.concatenate([rng.standard_normal(100_000) * 10.0 ** rng.uniform(-6, 5, 100_000),
                        g32, -g32, np.nextafter(g32, np.float32(np.inf)), np.nextafter(g32, np.float32(0)),
                        -np.nextafter(g32, np.float32(np.inf))]).astype(np.float32)
    x = x[np.abs(x) < FP8_FINITE_LIMIT[fmt]]
    got = orc.fp8_decode(orc.fp8_encode(x, fmt), fmt)
    want = np.sign(x) * grid[np.searchsorted(grid, np.abs(x).astype(np.float64), side="right") - 1]
    assert np.array_equal(got, want)


def test_fp8_encode_special_inputs():
    """The page's explicit cases: NaN, infinities, zeros, overflow, the
    band just below overflow that lands on the NaN/inf patterns, and fp32
    denormals (a signed zero)."""
    f = np.float32
    e4 = lambda v: int(orc.fp8_encode(np.array([v], np.float32), "e4m3")[0])  # noqa: E731
    e5 = lambda v: int(orc.fp8_encode(np.array([v], np.float32), "e5m2")[0])  # noqa: E731
    assert e4(np.nan) == 0xFF and e5(np.nan) == 0xFF
    assert e4(np.inf) == 0x7F and e4(-np.inf) == 0xFF
    assert e5(np.inf) == 0x7C and e5(-np.inf) == 0xFC
    assert e4(0.0) == 0 and e4(-0.0) == 0 and e5(-0.0) == 0
    # overflow: E4M3 saturates to +/-448, E5M2 to +/-inf
    assert e4(512.0) == 0x7E and e4(-1e30) == 0xFE and e4(448.0) == 0x7E and e4(479.9) == 0x7E
    assert e5(131072.0) == 0x7C and e5(-3e38) == 0xFC
    # the top exponent field: E4M3 [480, 512) -> the NaN pattern; E5M2
    # [65536, 131072) -> inf and NaN patterns
    assert e4(480.0) == 0x7F and e4(-500.0) == 0xFF
    assert e5(65536.0) == 0x7C and e5(98304.0) == 0x7E
    # below the smallest subnormal: a signed zero; fp32 denormals too
    assert e4(f(2.0 ** -10)) == 0 and e4(-f(2.0 ** -10)) == 0x80
    assert e5(f(2.0 ** -17)) == 0 and e5(-f(1e-45)) == 0x80
    assert np.isnan(orc.fp8_decode(np.array([0x7F]), "e4m3")[0])


def _page_value(v):
    return 2.0 ** int(v[2:]) if isinstance(v, str) else float(v)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_page_roundtrips(golden, fmt):
    g = golden["fp8_roundtrip"][fmt]
    for v in map(_page_value, g["values"]):
        d = float(orc.fp8_decode(orc.fp8_encode(np.array([v], np.float32), fmt), fmt)[0])
        if v == 0.0:
            assert d == 0.0
        elif abs(v) < 1e-5:
            assert abs(d) < 0.01
        else:
            assert abs(v - d) / abs(v) < g["max_rel_err"], (v, d)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_page_cache_basic(golden, fmt):
    g = golden["fp8_cache_basic"]
    n = g["num_kv_heads"] * g["head_dim"]
    i = np.arange(n, dtype=np.float32)
    for x in (i * np.float32(0.01) - np.float32(1.0), i * np.float32(0.02) - np.float32(0.5)):
        head0 = x[:g["head_dim"]]
        d = orc.fp8_decode(orc.fp8_encode(head0, fmt), fmt)
        a = head0.astype(np.float64)
        err = np.where(np.abs(a) > 1e-6, np.abs(a - d) / np.maximum(np.abs(a), 1e-30), np.abs(a - d))
        assert np.all(err < g["max_rel_err"])


def test_fp8_memory_savings(golden):
    g = golden["fp8_memory_savings"]
    f32 = orc.fp32_equivalent_bytes(g["num_kv_heads"], g["max_seq_len"], g["head_dim"], layers=g["num_layers"])
    fp8 = orc.codes_bytes(g["num_kv_heads"], g["max_seq_len"], g["head_dim"], layers=g["num_layers"])
    assert fp8 < f32 // 2 + f32 // 4
    assert fp8 * 4 == f32
