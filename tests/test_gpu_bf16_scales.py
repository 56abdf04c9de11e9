"""GPU parity of bf16-stored per-token scales (KVQ_SCALE_PER_TOKEN_BF16):
codes equal the fp32 per-token codes and the stored scales equal the
oracle's bf16 bits, bit for bit; attention (decode, fused step, chunk) is
checked against the oracle dequantizing with the stored bf16 scales."""

import numpy as np
import pytest

import oracle as orc
import workloads as wl
from kvq_testlib import (assert_attention_close, bf16_dev, dev_tensor, kv_dev, log, random_block_table,
                         to_host_bits)

pytestmark = pytest.mark.gpu


def _cache(kvq, B, H, KVH, D, T, paged, rng):
    if paged:
        table, npages = random_block_table(rng, [T] * B)
        return kvq.Int8KVCache(B, H, KVH, D, num_pages=npages, block_table=dev_tensor(table), fill=0,
                               scale_bf16=True), table
    return kvq.Int8KVCache(B, H, KVH, D, max_len=T, fill=0, scale_bf16=True), None


def _rows(arena, table, b, n):
    return arena[b, :, :n] if table is None else orc.paged_gather(arena, table, b, n)


def _oracle(x):
    kc, ksb = orc.quantize_bf16_scale(x["k"])
    vc, vsb = orc.quantize_bf16_scale(x["v"])
    return kc, ksb, vc, vsb


def _hat(codes, sbits):
    return orc.dequantize_exact(codes, orc.bf16_bits_to_f32(sbits))


def _scale_bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("paged,dtype", [(False, "bf16"), (True, "f32"), (False, "f32")])
def test_append_codes_and_bf16_scales(kvq, paged, dtype):
    B, H, KVH, D, T = 3, 8, 2, 128, 150
    log(f"bf16 scales append: paged={paged} dtype={dtype}")
    rng = np.random.default_rng(11 + paged)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), dtype, scale=3.0)
    cache, table = _cache(kvq, B, H, KVH, D, T, paged, rng)
    for p0, n in ((0, 70), (70, 1), (71, 79)):
        cache.append(kv_dev(np.ascontiguousarray(x["k_raw"][:, :, p0:p0 + n])),
                     kv_dev(np.ascontiguousarray(x["v_raw"][:, :, p0:p0 + n])), dev_tensor(np.full(B, p0, np.int32)))
    kc, ksb, vc, vsb = _oracle(x)
    dkc, dvc = cache.k_codes.cpu().numpy(), cache.v_codes.cpu().numpy()
    dks, dvs = _scale_bits(cache.k_scales), _scale_bits(cache.v_scales)
    for b in range(B):
        assert np.array_equal(_rows(dkc, table, b, T), kc[b])
        assert np.array_equal(_rows(dvc, table, b, T), vc[b])
        assert np.array_equal(_rows(dks, table, b, T), ksb[b])
        assert np.array_equal(_rows(dvs, table, b, T), vsb[b])
    # the codes are those of fp32 per-token scales
    assert np.array_equal(kc, orc.quantize(x["k"], 0)[0])


DECODE_CASES = [
    # D, H, KVH, lens, paged
    (128, 32, 8, [1, 17, 300, 511, 512, 513, 2000], False),
    (128, 32, 8, [5, 600, 1025], True),
    (64, 8, 2, [3, 129, 257], False),
    (256, 16, 4, [9, 300], False),
]


@pytest.mark.parametrize("D,H,KVH,lens,paged", DECODE_CASES)
def test_decode_bf16_scales(kvq, D, H, KVH, lens, paged):
    import torch
    log(f"bf16 scales decode: D={D} lens={lens} paged={paged}")
    B, T = len(lens), max(lens)
    rng = np.random.default_rng(D + len(lens) + paged)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "bf16")
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, D))
    cache, _ = _cache(kvq, B, H, KVH, D, T, paged, rng)
    cache.append(kv_dev(x["k_raw"]), kv_dev(x["v_raw"]), dev_tensor(np.zeros(B, np.int32)))
    scale = 1.0 / np.sqrt(D)
    out = cache.decode(bf16_dev(qb), dev_tensor(np.asarray(lens, np.int32)), scale, T)
    torch.cuda.synchronize()
    kc, ksb, vc, vsb = _oracle(x)
    ref = orc.attention_decode(qv, _hat(kc, ksb), _hat(vc, vsb), lens, scale)
    assert_attention_close(to_host_bits(out), ref, "bf16 scales decode")


@pytest.mark.parametrize("paged", [False, True])
def test_fused_bf16_scales_equals_two_launches(kvq, paged):
    """The fused step stores the bf16 scale and attends with that stored value."""
    import torch
    lens = [1, 64, 65, 700, 2049]
    B, H, KVH, D = len(lens), 32, 8, 128
    T = max(lens)
    rng = np.random.default_rng(21 + paged)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "f32")
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, D))
    a, table = _cache(kvq, B, H, KVH, D, T, paged, np.random.default_rng(3))
    f, _ = _cache(kvq, B, H, KVH, D, T, paged, np.random.default_rng(3))
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
    for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
        assert torch.equal(getattr(a, name), getattr(f, name)), name
    assert np.array_equal(to_host_bits(out_a), to_host_bits(out_f))
    kc, ksb, vc, vsb = _oracle(x)
    assert_attention_close(to_host_bits(out_f), orc.attention_decode(qv, _hat(kc, ksb), _hat(vc, vsb), lens, 0.088),
                           "fused bf16 scales")


@pytest.mark.parametrize("paged", [False, True])
def test_chunk_bf16_scales(kvq, paged):
    import torch
    L0s, n = [300, 17], 100
    B, H, KVH, D = 2, 32, 8, 128
    T = max(L0s) + n
    rng = np.random.default_rng(31 + paged)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "bf16")
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, n, D))
    cache, _ = _cache(kvq, B, H, KVH, D, T, paged, rng)
    cache.append(kv_dev(x["k_raw"]), kv_dev(x["v_raw"]), dev_tensor(np.zeros(B, np.int32)))
    out = cache.chunk(bf16_dev(qb), dev_tensor(np.asarray(L0s, np.int32)), True, 0.088, max(L0s))
    torch.cuda.synchronize()
    kc, ksb, vc, vsb = _oracle(x)
    ref = orc.attention_chunk(qv, _hat(kc, ksb), _hat(vc, vsb), L0s, True, 0.088)
    assert_attention_close(to_host_bits(out), ref, "bf16 scales chunk")


def test_dequant_bf16_scales_exact(kvq):
    """fl32((c - 128) s_bf16), zeros past each length."""
    lens = [5, 90]
    B, H, KVH, D, T = 2, 8, 2, 64, 96
    x = wl.random_kv(41, (B, KVH, T, D), "f32")
    cache, _ = _cache(kvq, B, H, KVH, D, T, False, None)
    cache.append(kv_dev(x["k_raw"]), kv_dev(x["v_raw"]), dev_tensor(np.zeros(B, np.int32)))
    kc, ksb, vc, vsb = _oracle(x)
    for which, (c, sb) in enumerate(((kc, ksb), (vc, vsb))):
        got = cache.dequant(which, dev_tensor(np.asarray(lens, np.int32)), T).cpu().numpy()
        want = _hat(c, sb).astype(np.float32)
        for b, L in enumerate(lens):
            assert np.array_equal(got[b, :, :L], want[b, :, :L])
            assert np.all(got[b, :, L:] == 0)
