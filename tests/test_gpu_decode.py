"""GPU parity of kvq_attention_decode against the fp64 oracle, plus the
closed forms and invariants that hold at any size."""

import os

import numpy as np
import pytest

import oracle as orc
import workloads as wl
from kvq_testlib import (assert_attention_close, bf16_dev, dev_tensor, kv_dev, log, random_block_table,
                         to_host_bits)

pytestmark = pytest.mark.gpu


def _build(kvq, k_raw, v_raw, H, group, max_len=None, paged=False, rng=None, lens=None, chunks=None):
    """Append full K/V [B, KVH, T, D] into a fresh cache (in chunks)."""
    B, KVH, T, D = k_raw.shape
    if paged:
        table, npages = random_block_table(rng, [T] * B)
        cache = kvq.Int8KVCache(B, H, KVH, D, num_pages=npages, block_table=dev_tensor(table),
                                group32=(group == 32), fill=0)
    else:
        cache = kvq.Int8KVCache(B, H, KVH, D, max_len=max_len or T, group32=(group == 32), fill=0)
    pos = 0
    for n in (chunks or [T]):
        cache.append(kv_dev(np.ascontiguousarray(k_raw[:, :, pos:pos + n])),
                     kv_dev(np.ascontiguousarray(v_raw[:, :, pos:pos + n])),
                     dev_tensor(np.full(B, pos, np.int32)))
        pos += n
    return cache


def _oracle_decode(k_vals, v_vals, q_vals, lens, scale, group):
    kc, ks = orc.quantize(k_vals, group)
    vc, vs = orc.quantize(v_vals, group)
    return orc.attention_decode(q_vals, orc.dequantize_exact(kc, ks), orc.dequantize_exact(vc, vs), lens, scale)


def _decode(cache, q_bits, lens, scale, hint):
    import torch
    out = cache.decode(bf16_dev(q_bits), dev_tensor(np.asarray(lens, np.int32)), scale, hint)
    torch.cuda.synchronize()
    return to_host_bits(out)


def test_tiny_workload(kvq):
    """Tiny decode: B1, 8 q / 2 KV heads, D64, 255 cached + 1 appended, scale 1/8, seed 0."""
    log("decode: tiny workload")
    w = wl.TINY
    x = wl.tiny_inputs()
    cache = _build(kvq, x["k_raw"], x["v_raw"], w.num_heads, 0, chunks=[255, 1])
    got = _decode(cache, x["q_bits"], [256], w.attn_scale, 256)
    ref = _oracle_decode(x["k"], x["v"], x["q"], [256], w.attn_scale, 0)
    assert_attention_close(got, ref, "tiny")


CASES = [
    # D, H, KVH, group, lens, paged
    (128, 32, 8, 0, [1, 2, 15, 16, 17, 300, 511, 512, 513, 1000], False),
    (128, 32, 8, 32, [7, 64, 700, 1025], False),
    (64, 8, 2, 0, [3, 129, 257, 1], False),
    (32, 4, 4, 0, [5, 90, 333], False),
    (256, 16, 2, 32, [9, 200, 513], False),     # head dim 256: 32-token blocks
    (256, 16, 4, 0, [1, 31, 32, 33, 600, 1025], False),
    (256, 8, 4, 0, [17, 256, 257, 700], True),  # GQA 2: two heads per workgroup, paged
    (256, 12, 4, 32, [64, 300], True),          # GQA 3: one head per workgroup
    (128, 24, 8, 0, [100, 517], False),        # GQA 3: one head per workgroup
    (128, 64, 8, 0, [77, 600], False),         # GQA 8: two workgroups per KV head
    (128, 16, 16, 0, [40, 41], False),         # MHA
    (128, 32, 8, 0, [1, 17, 300, 1000, 16, 32], True),
    (64, 8, 2, 32, [31, 64, 65], True),
]


@pytest.mark.parametrize("D,H,KVH,group,lens,paged", CASES)
def test_decode_ragged(kvq, D, H, KVH, group, lens, paged):
    log(f"decode: D={D} H={H} KVH={KVH} group={group} lens={lens} paged={paged}")
    B = len(lens)
    T = max(lens)
    rng = np.random.default_rng(D * 7 + H + group + (1 if paged else 0))
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "bf16")
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, D))
    scale = 1.0 / np.sqrt(D)
    cache = _build(kvq, x["k_raw"], x["v_raw"], H, group, paged=paged, rng=rng)
    got = _decode(cache, qb, lens, scale, T)
    ref = _oracle_decode(x["k"], x["v"], qv, lens, scale, group)
    assert_attention_close(got, ref, f"D{D} H{H} KVH{KVH} g{group} paged={paged}")


def test_single_token_gives_v(kvq):
    """L = 1: the output is the dequantized V row, rounded to bf16."""
    log("decode: single cached token")
    B, H, KVH, D = 2, 8, 2, 128
    x = wl.random_kv(5, (B, KVH, 1, D), "bf16")
    qb, _ = wl.random_q(6, (B, H, D))
    cache = _build(kvq, x["k_raw"], x["v_raw"], H, 0)
    got = _decode(cache, qb, [1, 1], 0.1, 1)
    vc, vs = orc.quantize(x["v"], 0)
    vhat = orc.dequantize_bf16_bits(vc, vs)
    for h in range(H):
        assert np.array_equal(got[:, h], vhat[:, h // 4, 0]), h


def test_constant_keys_give_mean_v(kvq):
    """Identical keys at every position give uniform weights: out = mean V."""
    log("decode: constant keys")
    B, H, KVH, D, L = 1, 4, 1, 128, 777
    x = wl.random_kv(8, (B, KVH, L, D), "bf16")
    k = np.repeat(x["k_raw"][:, :, :1], L, axis=2)
    qb, _ = wl.random_q(9, (B, H, D))
    cache = _build(kvq, k, x["v_raw"], H, 0)
    got = _decode(cache, qb, [L], 0.3, L)
    vc, vs = orc.quantize(x["v"], 0)
    mean = orc.dequantize_exact(vc, vs)[0, 0].mean(axis=0)
    for h in range(H):
        assert_attention_close(got[0, h], mean, "constant keys")


def test_zero_length_gives_zeros(kvq):
    log("decode: zero length")
    B, H, KVH, D = 2, 4, 1, 64
    x = wl.random_kv(10, (B, KVH, 8, D), "f32")
    qb, qv = wl.random_q(11, (B, H, D))
    cache = _build(kvq, x["k_raw"], x["v_raw"], H, 0)
    got = _decode(cache, qb, [0, 8], 0.125, 8)
    assert np.all(got[0] == 0)
    ref = _oracle_decode(x["k"][1:], x["v"][1:], qv[1:], [8], 0.125, 0)
    assert_attention_close(got[1:], ref, "second sequence")


def test_split_count_invariance(kvq, monkeypatch):
    """The split-K result does not depend on the number of splits."""
    log("decode: split invariance")
    B, H, KVH, D, L = 2, 32, 8, 128, 3000
    x = wl.random_kv(12, (B, KVH, L, D), "bf16")
    qb, qv = wl.random_q(13, (B, H, D))
    cache = _build(kvq, x["k_raw"], x["v_raw"], H, 0)
    outs = []
    for ns in (1, 2, 7, 64):
        monkeypatch.setenv("KVQ_NUM_SPLITS", str(ns))
        outs.append(orc.bf16_bits_to_f32(_decode(cache, qb, [L, 1234], 0.088, L)).astype(np.float64))
    monkeypatch.delenv("KVQ_NUM_SPLITS")
    for ns, o in zip((2, 7, 64), outs[1:]):
        # equal up to one bf16 rounding step of the fp32 result, plus fp32
        # association noise near zero (100x below the attention tolerance)
        dev = np.abs(o - outs[0])
        log(f"  splits={ns}: max |diff| {dev.max():.3e}")
        assert np.all(dev <= 2.0 ** -7 * np.abs(outs[0]) + 1e-4)
    ref = _oracle_decode(x["k"], x["v"], qv, [L, 1234], 0.088, 0)
    assert_attention_close(to_bits(outs[0]), ref, "split invariance")


def to_bits(vals):
    return orc.f32_to_bf16_bits(vals.astype(np.float32))


def test_paged_equals_contiguous(kvq):
    """The same logical tokens in a scattered paged arena and in a contiguous
    cache give bit-identical outputs."""
    log("decode: paged == contiguous")
    B, H, KVH, D = 3, 32, 8, 128
    lens = [1000, 16, 513]
    T = max(lens)
    rng = np.random.default_rng(14)
    x = wl.random_kv(15, (B, KVH, T, D), "bf16")
    qb, _ = wl.random_q(16, (B, H, D))
    c1 = _build(kvq, x["k_raw"], x["v_raw"], H, 0)
    c2 = _build(kvq, x["k_raw"], x["v_raw"], H, 0, paged=True, rng=rng)
    assert np.array_equal(_decode(c1, qb, lens, 0.09, T), _decode(c2, qb, lens, 0.09, T))


def test_large_scores_lazy_rescale(kvq):
    """Scores that grow along the sequence force the running-max rescale."""
    log("decode: growing scores")
    B, H, KVH, D, L = 1, 4, 1, 128, 2000
    rng = np.random.default_rng(17)
    k = rng.standard_normal((B, KVH, L, D)).astype(np.float32)
    k *= np.linspace(0.1, 6.0, L, dtype=np.float32)[None, None, :, None]
    v = rng.standard_normal((B, KVH, L, D)).astype(np.float32)
    qb, qv = wl.random_q(18, (B, H, D))
    cache = _build(kvq, k, v, H, 0)
    got = _decode(cache, qb, [L], 1.0 / np.sqrt(D), L)
    ref = _oracle_decode(k, v, qv, [L], 1.0 / np.sqrt(D), 0)
    assert_attention_close(got, ref, "growing scores")


@pytest.mark.parametrize("paged,fused", [(False, False), (True, False), (False, True), (True, True)])
def test_longest_first_order(kvq, monkeypatch, paged, fused):
    """Workgroups that take sequences longest first (ties, an empty sequence
    and several splits per sequence included) give the same bits as the
    natural order, and match the oracle."""
    import torch
    log(f"decode: longest-first order paged={paged} fused={fused}")
    lens = [700, 3, 1500, 700, 0, 1499, 64, 1500, 65]
    B, H, KVH, D = len(lens), 32, 8, 128
    T = max(lens)
    rng = np.random.default_rng(21 + 2 * paged + fused)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "bf16")
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, D))
    scale = 1.0 / np.sqrt(D)
    lens_np = np.asarray(lens, np.int32)
    idx = np.maximum(lens_np - 1, 0)
    k_new = np.ascontiguousarray(x["k_raw"][np.arange(B), :, idx][:, :, None, :])
    v_new = np.ascontiguousarray(x["v_raw"][np.arange(B), :, idx][:, :, None, :])
    monkeypatch.setenv("KVQ_SPLIT_LEN", "512")
    outs = {}
    for lf in ("0", "1"):
        monkeypatch.setenv("KVQ_LONGEST_FIRST", lf)
        cache = _build(kvq, x["k_raw"], x["v_raw"], H, 0, paged=paged, rng=np.random.default_rng(5))
        if fused:
            out = cache.append_decode(kv_dev(k_new), kv_dev(v_new), bf16_dev(qb), dev_tensor(lens_np), scale, T)
            torch.cuda.synchronize()
            outs[lf] = to_host_bits(out)
        else:
            outs[lf] = _decode(cache, qb, lens, scale, T)
    assert np.array_equal(outs["0"], outs["1"])
    live = lens_np > 0
    assert np.all(outs["1"][~live] == 0)
    ref = _oracle_decode(x["k"][live], x["v"][live], qv[live], lens_np[live], scale, 0)
    assert_attention_close(outs["1"][live], ref, "longest first")


@pytest.mark.parametrize("group,paged", [(32, False), (0, False), (32, True)])
def test_short_sequences_in_unwritten_cache(kvq, group, paged):
    """Sequences much shorter than a zero-initialised cache: the first block's
    loads run ahead of the length and read rows never written (zero scales),
    which must not reach the result."""
    import torch
    lens = [10, 1, 63, 65]
    B, H, KVH, D = len(lens), 32, 8, 128
    cap = 512
    log(f"decode: short sequences in an unwritten cache, group={group} paged={paged}")
    rng = np.random.default_rng(51 + group + paged)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, max(lens), D), "bf16")
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, D))
    if paged:
        table, npages = random_block_table(rng, [cap] * B)
        cache = kvq.Int8KVCache(B, H, KVH, D, num_pages=npages, block_table=dev_tensor(table),
                                group32=(group == 32), fill=0)
    else:
        cache = kvq.Int8KVCache(B, H, KVH, D, max_len=cap, group32=(group == 32), fill=0)
    # only each sequence's own rows are written: row i of sequence b for i < lens[b]
    for i in range(max(lens)):
        live = np.asarray([i < L for L in lens])
        if not live.any():
            break
        pos = np.where(live, i, cap + 10).astype(np.int32)   # rows past the capacity are not written
        cache.append(kv_dev(np.ascontiguousarray(x["k_raw"][:, :, i:i + 1])),
                     kv_dev(np.ascontiguousarray(x["v_raw"][:, :, i:i + 1])), dev_tensor(pos))
    out = cache.decode(bf16_dev(qb), dev_tensor(np.asarray(lens, np.int32)), 0.088, cap)
    torch.cuda.synchronize()
    ref = _oracle_decode(x["k"], x["v"], qv, lens, 0.088, group)
    assert_attention_close(to_host_bits(out), ref, "short sequences")
