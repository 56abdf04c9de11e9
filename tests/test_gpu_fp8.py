"""GPU parity of FP8 codes (llama-gguf kv_quantized.rs, E4M3 / E5M2): the
append's codes equal the oracle's encoder bit for bit (special inputs
included), dequantization equals the oracle's decoder bit for bit, and decode
attention (plain, paged, windowed, fused) is checked against the oracle
attending over the decoded values."""

import numpy as np
import pytest

import oracle as orc
import workloads as wl
from kvq_testlib import (assert_attention_close, bf16_dev, dev_tensor, kv_dev, log, random_block_table,
                         to_host_bits)

pytestmark = pytest.mark.gpu

FORMATS = ["e4m3", "e5m2"]


def _cache(kvq, fmt, B, H, KVH, D, T, paged, rng, fill=0):
    if paged:
        table, npages = random_block_table(rng, [T] * B)
        return kvq.Int8KVCache(B, H, KVH, D, num_pages=npages, block_table=dev_tensor(table), fill=fill,
                               fp8=fmt), table
    return kvq.Int8KVCache(B, H, KVH, D, max_len=T, fill=fill, fp8=fmt), None


def _rows(arena, table, b, n):
    return arena[b, :, :n] if table is None else orc.paged_gather(arena, table, b, n)


def _hat(x, fmt):
    return orc.fp8_decode(orc.fp8_encode(x, fmt), fmt)


def _special_values(rng, shape):
    """Magnitudes over twelve decades with the codec's edge cases planted:
    zeros of both signs, the subnormal bands, the values around each
    format's overflow and NaN/inf bands, infinities, NaN and fp32 denormals."""
    x = (rng.standard_normal(shape) * 10.0 ** rng.uniform(-7, 5.5, shape)).astype(np.float32)
    edge = np.array([0.0, -0.0, 2.0 ** -9, 2.0 ** -10, 1.5 * 2.0 ** -8, 2.0 ** -16, 2.0 ** -17, 3 * 2.0 ** -16,
                     448.0, 464.0, 479.9, 480.0, 500.0, 511.99, 512.0, 1e30, 57344.0, 61440.0, 65535.0, 65536.0,
                     98304.0, 131071.0, 131072.0, 3e38, np.inf, np.nan, 1e-45, 1e-39], np.float32)
    flat = x.reshape(-1)
    pos = rng.choice(flat.size, size=4 * edge.size, replace=False)
    flat[pos] = np.tile(edge, 4) * np.where(rng.random(4 * edge.size) < 0.5, -1, 1).astype(np.float32)
    return flat.reshape(shape)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("paged,dtype", [(False, "f32"), (True, "f32"), (False, "bf16")])
def test_append_codes_bit_exact(kvq, fmt, paged, dtype):
    B, H, KVH, D, T = 3, 8, 2, 128, 90
    log(f"fp8 append: fmt={fmt} paged={paged} dtype={dtype}")
    rng = np.random.default_rng(101 + paged)
    k = _special_values(rng, (B, KVH, T, D))
    v = _special_values(rng, (B, KVH, T, D))
    if dtype == "bf16":
        k_raw, v_raw = orc.f32_to_bf16_bits(k), orc.f32_to_bf16_bits(v)
        k, v = orc.bf16_bits_to_f32(k_raw), orc.bf16_bits_to_f32(v_raw)
    else:
        k_raw, v_raw = k, v
    cache, table = _cache(kvq, fmt, B, H, KVH, D, T, paged, rng)
    for p0, n in ((0, 40), (40, 1), (41, 49)):
        cache.append(kv_dev(np.ascontiguousarray(k_raw[:, :, p0:p0 + n])),
                     kv_dev(np.ascontiguousarray(v_raw[:, :, p0:p0 + n])), dev_tensor(np.full(B, p0, np.int32)))
    dk, dv = cache.k_codes.cpu().numpy(), cache.v_codes.cpu().numpy()
    wk, wv = orc.fp8_encode(k, fmt), orc.fp8_encode(v, fmt)
    for b in range(B):
        assert np.array_equal(_rows(dk, table, b, T), wk[b])
        assert np.array_equal(_rows(dv, table, b, T), wv[b])


@pytest.mark.parametrize("fmt", FORMATS)
def test_dequant_bit_exact(kvq, fmt):
    """Every byte value decodes as the page does, in fp32 and in bf16 (NaN as
    the canonical quiet NaN, negative zero as +0), zeros past each length."""
    import torch
    B, H, KVH, D, T = 2, 4, 2, 64, 8
    cache, _ = _cache(kvq, fmt, B, H, KVH, D, T, False, None)
    codes = np.arange(B * KVH * T * D, dtype=np.int64).reshape(B, KVH, T, D) % 256
    cache.k_codes.copy_(torch.from_numpy(codes.astype(np.uint8)))
    lens = [8, 5]
    want = orc.fp8_decode(codes, fmt).astype(np.float32)
    got = cache.dequant(0, dev_tensor(np.asarray(lens, np.int32)), T).cpu().numpy()
    gotb = to_host_bits(cache.dequant(0, dev_tensor(np.asarray(lens, np.int32)), T, bf16=True))
    wantb = orc.fp8_decode_bf16_bits(codes, fmt)
    for b, L in enumerate(lens):
        assert np.array_equal(got[b, :, :L].view(np.uint32), want[b, :, :L].view(np.uint32))
        assert np.array_equal(gotb[b, :, :L], wantb[b, :, :L])
        assert np.all(got[b, :, L:] == 0)


DECODE_CASES = [
    # fmt, D, H, KVH, lens, paged, window
    ("e4m3", 128, 32, 8, [1, 17, 63, 64, 65, 300, 2000], False, 0),
    ("e5m2", 128, 32, 8, [2, 129, 511, 1537], False, 0),
    ("e4m3", 128, 32, 8, [5, 600, 1025], True, 0),
    ("e5m2", 128, 32, 8, [70, 333], True, 0),
    ("e4m3", 64, 8, 2, [3, 129, 257], False, 0),
    ("e5m2", 32, 4, 4, [16, 200], False, 0),
    ("e4m3", 256, 16, 4, [9, 300], False, 0),
    ("e5m2", 256, 16, 4, [40, 77], True, 0),     # paged
    ("e4m3", 128, 32, 8, [50, 700, 2500], False, 100),
    ("e5m2", 128, 64, 8, [76, 600], True, 77),
]


@pytest.mark.parametrize("fmt,D,H,KVH,lens,paged,window", DECODE_CASES)
def test_decode_fp8(kvq, fmt, D, H, KVH, lens, paged, window):
    """Rows past each length hold NaN codes (bytes 0xFF): the masked tokens
    of partial blocks must not reach the result."""
    import torch
    log(f"fp8 decode: fmt={fmt} D={D} H={H} KVH={KVH} lens={lens} paged={paged} window={window}")
    B, T = len(lens), max(lens)
    rng = np.random.default_rng(D + len(lens) + paged + window)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "bf16", scale=2.0)
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, D))
    cap = -(-T // 64) * 64 + 64
    cache, table = _cache(kvq, fmt, B, H, KVH, D, cap, paged, rng, fill=0xFF)
    cache.append(kv_dev(x["k_raw"]), kv_dev(x["v_raw"]), dev_tensor(np.zeros(B, np.int32)))
    # rows past each length back to NaN codes
    kc, vc = cache.k_codes.cpu().numpy(), cache.v_codes.cpu().numpy()
    for b, L in enumerate(lens):
        for t in range(L, cap):
            if table is None:
                kc[b, :, t] = 0xFF
                vc[b, :, t] = 0xFF
            else:
                pg = table[b, t // 16]
                if pg >= 0:
                    kc[pg, :, t % 16] = 0xFF
                    vc[pg, :, t % 16] = 0xFF
    cache.k_codes.copy_(torch.from_numpy(kc))
    cache.v_codes.copy_(torch.from_numpy(vc))
    scale = 1.0 / np.sqrt(D)
    out = cache.decode(bf16_dev(qb), dev_tensor(np.asarray(lens, np.int32)), scale, cap, window=window)
    torch.cuda.synchronize()
    ref = orc.attention_decode(qv, _hat(x["k"], fmt), _hat(x["v"], fmt), lens, scale, window=window)
    assert_attention_close(to_host_bits(out), ref, f"fp8 {fmt} decode")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("paged", [False, True])
def test_fused_fp8_equals_two_launches(kvq, fmt, paged):
    import torch
    lens = [1, 64, 65, 700, 2049]
    B, H, KVH, D = len(lens), 32, 8, 128
    T = max(lens)
    log(f"fp8 fused: fmt={fmt} paged={paged}")
    rng = np.random.default_rng(121 + paged)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "f32", scale=3.0)
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, D))
    a, _ = _cache(kvq, fmt, B, H, KVH, D, T, paged, np.random.default_rng(3))
    f, _ = _cache(kvq, fmt, B, H, KVH, D, T, paged, np.random.default_rng(3))
    for c in (a, f):
        c.append(kv_dev(x["k_raw"]), kv_dev(x["v_raw"]), dev_tensor(np.zeros(B, np.int32)))
    idx = np.asarray(lens) - 1
    k_new = kv_dev(np.ascontiguousarray(x["k_raw"][np.arange(B), :, idx][:, :, None, :]))
    v_new = kv_dev(np.ascontiguousarray(x["v_raw"][np.arange(B), :, idx][:, :, None, :]))
    L = dev_tensor(np.asarray(lens, np.int32))
    q = bf16_dev(qb)
    a.append(k_new, v_new, dev_tensor(idx.astype(np.int32)))
    out_a = a.decode(q, L, 0.088, T)
    out_f = f.append_decode(k_new, v_new, q, L, 0.088, T)
    torch.cuda.synchronize()
    assert torch.equal(a.k_codes, f.k_codes) and torch.equal(a.v_codes, f.v_codes)
    assert np.array_equal(to_host_bits(out_a), to_host_bits(out_f))
    assert_attention_close(to_host_bits(out_f),
                           orc.attention_decode(qv, _hat(x["k"], fmt), _hat(x["v"], fmt), lens, 0.088), "fp8 fused")


CHUNK_CASES = [
    # fmt, D, H, KVH, L0s, n, paged, window
    ("e4m3", 128, 32, 8, [300, 17], 100, False, 0),
    ("e5m2", 128, 32, 8, [700], 130, True, 0),
    ("e4m3", 64, 8, 2, [200, 513], 50, False, 0),
    ("e5m2", 64, 16, 4, [0, 90], 77, True, 0),
    ("e4m3", 128, 32, 8, [1000], 64, False, 129),
]


@pytest.mark.parametrize("fmt,D,H,KVH,L0s,n,paged,window", CHUNK_CASES)
def test_chunk_fp8(kvq, fmt, D, H, KVH, L0s, n, paged, window):
    import torch
    log(f"fp8 chunk: fmt={fmt} D={D} L0={L0s} n={n} paged={paged} window={window}")
    B = len(L0s)
    T = max(L0s) + n
    rng = np.random.default_rng(D + n + paged + window)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "bf16", scale=2.0)
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, n, D))
    cache, _ = _cache(kvq, fmt, B, H, KVH, D, T, paged, rng)
    cache.append(kv_dev(x["k_raw"]), kv_dev(x["v_raw"]), dev_tensor(np.zeros(B, np.int32)))
    scale = 1.0 / np.sqrt(D)
    out = cache.chunk(bf16_dev(qb), dev_tensor(np.asarray(L0s, np.int32)), True, scale, max(L0s), window=window)
    torch.cuda.synchronize()
    ref = orc.attention_chunk(qv, _hat(x["k"], fmt), _hat(x["v"], fmt), L0s, True, scale, window=window)
    assert_attention_close(to_host_bits(out), ref, f"fp8 {fmt} chunk")


def test_fp8_recent_unsupported(kvq):
    import torch
    q = torch.zeros((1, 8, 128), dtype=torch.bfloat16, device="cuda")
    # (the workspace query fails first; sizes report errors as 0, which the
    # binding raises with the library's message)
    with pytest.raises(kvq.KvqError, match="recent window over FP8 codes is not supported"):
        kvq.Int8KVCache(1, 8, 2, 128, max_len=64, fp8="e5m2", recent_window=4).decode(
            q, dev_tensor(np.ones(1, np.int32)), 0.1, 64)
