"""GPU parity of sliding-window attention (a query at position p sees keys
in (p - w, p]) against the oracle, for decode, the fused decode step and
chunked prefill."""

import numpy as np
import pytest

import oracle as orc
import workloads as wl
from kvq_testlib import (assert_attention_close, bf16_dev, dev_tensor, kv_dev, log, random_block_table,
                         to_host_bits)

pytestmark = pytest.mark.gpu


def _build(kvq, x, H, group, paged, rng):
    B, KVH, T, D = x["k"].shape
    if paged:
        table, npages = random_block_table(rng, [T] * B)
        cache = kvq.Int8KVCache(B, H, KVH, D, num_pages=npages, block_table=dev_tensor(table),
                                group32=(group == 32), fill=0)
    else:
        cache = kvq.Int8KVCache(B, H, KVH, D, max_len=T, group32=(group == 32), fill=0)
    cache.append(kv_dev(x["k_raw"]), kv_dev(x["v_raw"]), dev_tensor(np.zeros(B, np.int32)))
    return cache


def _oracle_hat(x, group):
    kc, ks = orc.quantize(x["k"], group)
    vc, vs = orc.quantize(x["v"], group)
    return orc.dequantize_exact(kc, ks), orc.dequantize_exact(vc, vs)


DECODE_CASES = [
    # D, H, KVH, group, window, lens, paged
    (128, 32, 8, 0, 100, [1, 50, 99, 100, 101, 163, 164, 700, 2500], False),
    (128, 32, 8, 32, 64, [63, 64, 65, 128, 129, 1000], False),
    (128, 32, 8, 0, 1, [1, 2, 17, 300], True),
    (128, 32, 8, 0, 1000, [5, 999, 1000, 1001, 3000], True),
    (64, 8, 2, 0, 5, [3, 5, 6, 90], False),
    (32, 4, 4, 0, 17, [16, 17, 18, 200], False),
    (256, 16, 4, 0, 40, [20, 41, 300], False),
    (128, 64, 8, 0, 77, [76, 600], False),        # two workgroups per KV head
]


@pytest.mark.parametrize("D,H,KVH,group,window,lens,paged", DECODE_CASES)
def test_decode_window(kvq, D, H, KVH, group, window, lens, paged):
    import torch
    log(f"decode window: D={D} H={H} KVH={KVH} group={group} w={window} lens={lens} paged={paged}")
    B, T = len(lens), max(lens)
    rng = np.random.default_rng(D + H + window + group + paged)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "bf16")
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, D))
    cache = _build(kvq, x, H, group, paged, rng)
    scale = 1.0 / np.sqrt(D)
    out = cache.decode(bf16_dev(qb), dev_tensor(np.asarray(lens, np.int32)), scale, T, window=window)
    torch.cuda.synchronize()
    k_hat, v_hat = _oracle_hat(x, group)
    ref = orc.attention_decode(qv, k_hat, v_hat, lens, scale, window=window)
    assert_attention_close(to_host_bits(out), ref, "decode window")


def test_window_covering_everything_is_plain_decode(kvq):
    """window >= the hint: the same launch as plain decode, bit for bit."""
    import torch
    lens = [7, 500, 1300]
    B, H, KVH, D = 3, 32, 8, 128
    T = max(lens)
    x = wl.random_kv(71, (B, KVH, T, D), "bf16")
    qb, _ = wl.random_q(72, (B, H, D))
    cache = _build(kvq, x, H, 0, False, np.random.default_rng(0))
    q, L = bf16_dev(qb), dev_tensor(np.asarray(lens, np.int32))
    a = cache.decode(q, L, 0.09, T)
    b = cache.decode(q, L, 0.09, T, window=T)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(a), to_host_bits(b))


@pytest.mark.parametrize("paged,group", [(False, 0), (True, 32)])
def test_fused_window_equals_append_then_decode(kvq, paged, group):
    import torch
    lens = [1, 64, 65, 300, 1500]
    window = 128
    B, H, KVH, D = len(lens), 32, 8, 128
    T = max(lens)
    log(f"fused window: paged={paged} group={group}")
    rng = np.random.default_rng(81 + paged + group)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "bf16")
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, D))
    a = _build(kvq, x, H, group, paged, np.random.default_rng(5))
    f = _build(kvq, x, H, group, paged, np.random.default_rng(5))
    idx = np.asarray(lens) - 1
    k_new = kv_dev(np.ascontiguousarray(x["k_raw"][np.arange(B), :, idx][:, :, None, :]))
    v_new = kv_dev(np.ascontiguousarray(x["v_raw"][np.arange(B), :, idx][:, :, None, :]))
    L = dev_tensor(np.asarray(lens, np.int32))
    q = bf16_dev(qb)
    a.append(k_new, v_new, dev_tensor(idx.astype(np.int32)))
    out_a = a.decode(q, L, 0.088, T, window=window)
    out_f = f.append_decode(k_new, v_new, q, L, 0.088, T, window=window)
    torch.cuda.synchronize()
    for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
        assert torch.equal(getattr(a, name), getattr(f, name)), name
    assert np.array_equal(to_host_bits(out_a), to_host_bits(out_f))
    k_hat, v_hat = _oracle_hat(x, group)
    assert_attention_close(to_host_bits(out_f), orc.attention_decode(qv, k_hat, v_hat, lens, 0.088, window=window),
                           "fused window")


CHUNK_CASES = [
    # D, H, KVH, L0s, n, window, paged
    (128, 32, 8, [300, 17], 100, 40, False),
    (128, 32, 8, [700], 130, 64, False),
    (128, 32, 8, [90, 0], 77, 1, True),
    (64, 8, 2, [200, 513], 50, 129, False),
    (128, 24, 8, [1000], 64, 5000, False),      # window past everything: plain causal
    (128, 64, 8, [256], 96, 200, True),
]


@pytest.mark.parametrize("D,H,KVH,L0s,n,window,paged", CHUNK_CASES)
def test_chunk_window(kvq, D, H, KVH, L0s, n, window, paged):
    import torch
    log(f"chunk window: D={D} H={H} KVH={KVH} L0={L0s} n={n} w={window} paged={paged}")
    B = len(L0s)
    T = max(L0s) + n
    rng = np.random.default_rng(D + n + window + paged)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "bf16")
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, n, D))
    cache = _build(kvq, x, H, 0, paged, rng)
    scale = 1.0 / np.sqrt(D)
    out = cache.chunk(bf16_dev(qb), dev_tensor(np.asarray(L0s, np.int32)), True, scale, max(L0s), window=window)
    torch.cuda.synchronize()
    k_hat, v_hat = _oracle_hat(x, 0)
    ref = orc.attention_chunk(qv, k_hat, v_hat, L0s, True, scale, window=window)
    assert_attention_close(to_host_bits(out), ref, "chunk window")


@pytest.mark.parametrize("group,fused,D", [(0, False, 128), (32, True, 128), (0, True, 64)])
def test_rolling_store(kvq, group, fused, D):
    """A sliding-window layer on a rolling store: a paged cache whose block
    table maps each sequence's logical pages onto ceil((w + n - 1) / 16)
    physical ones in turn, so rows overwrite rows that left the window.  The
    sequences grow to 700 tokens through appends of 1 to n rows; after each
    append the decode (fused for single rows when ``fused``) and, after a
    chunk, chunked prefill over the chunk's queries match the oracle's
    sliding attention over the whole history."""
    import torch
    B, H, KVH, w, n = 2, 8, 2, 100, 29
    T = 700
    log(f"rolling store: group={group} fused={fused} D={D}")
    table, npages = kvq.rolling_block_table(B, T, w, n)
    assert npages * 16 < T // 2
    rng = np.random.default_rng(91 + group + D)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "bf16")
    k_hat, v_hat = _oracle_hat(x, group)
    cache = kvq.Int8KVCache(B, H, KVH, D, num_pages=npages, block_table=table.cuda(), group32=(group == 32), fill=0)
    scale = 1.0 / np.sqrt(D)
    ws = cache.workspace(T, 1, w)      # decode
    wsc = cache.workspace(T, n, w)     # chunks of up to n rows
    sizes = [1, 29, 7, 1, 1, 13, 29, 2, 1]
    L, i, checked = 0, 0, 0
    while L < T:
        m = min(sizes[i % len(sizes)], T - L)
        i += 1
        rows = lambda a: np.ascontiguousarray(a[:, :, L:L + m])
        start = dev_tensor(np.full(B, L, np.int32))
        lens = dev_tensor(np.full(B, L + m, np.int32))
        qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, D))
        if m == 1 and fused:
            out = cache.append_decode(kv_dev(rows(x["k_raw"])), kv_dev(rows(x["v_raw"])), bf16_dev(qb), lens, scale, T,
                                      workspace=ws, window=w)
        else:
            cache.append(kv_dev(rows(x["k_raw"])), kv_dev(rows(x["v_raw"])), start)
            out = cache.decode(bf16_dev(qb), lens, scale, T, workspace=ws, window=w)
        torch.cuda.synchronize()
        L += m
        ref = orc.attention_decode(qv, k_hat, v_hat, [L] * B, scale, window=w)
        assert_attention_close(to_host_bits(out), ref, f"rolling decode at L={L}")
        if m > 1:
            cb, cv = wl.random_q(int(rng.integers(1 << 30)), (B, H, m, D))
            out = cache.chunk(bf16_dev(cb), start, True, scale, L - m, workspace=wsc, window=w)
            torch.cuda.synchronize()
            ref = orc.attention_chunk(cv, k_hat, v_hat, [L - m] * B, True, scale, window=w)
            assert_attention_close(to_host_bits(out), ref, f"rolling chunk at L={L}")
        checked += 1
    assert checked > 50
