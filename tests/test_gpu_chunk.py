"""GPU parity of kvq_attention_chunk (f16 MFMA on the INT8 cache) against the
fp64 oracle, and the invariants of chunked prefill: row i of a causal chunk
equals decode attention over L0 + i + 1 tokens, paged equals contiguous."""

import numpy as np
import pytest

import oracle as orc
import workloads as wl
from kvq_testlib import assert_attention_close, bf16_dev, dev_tensor, kv_dev, log, random_block_table, to_host_bits

pytestmark = pytest.mark.gpu

CASES = [
    # D, H, KVH, ctx_lens, n, causal, paged
    (128, 32, 8, [0, 100], 37, True, False),      # first chunk of a prompt; ragged n
    (128, 32, 8, [513, 64], 96, True, False),     # several key tiles and query blocks
    (128, 32, 8, [200, 3], 64, False, False),     # non-causal
    (64, 8, 2, [0, 77, 300], 33, True, False),
    (64, 8, 8, [65, 1], 40, True, False),         # MHA: four position blocks per workgroup
    (128, 6, 2, [130], 70, True, False),          # 3 query heads per KV head
    (128, 16, 2, [255], 50, True, False),         # 8 query heads per KV head
    (128, 32, 8, [40, 500], 45, True, True),      # paged
    (64, 8, 2, [17, 130], 100, False, True),      # paged, non-causal
    (128, 8, 2, [1000], 1, True, False),          # n = 1
    (256, 16, 4, [513, 64], 96, True, False),     # head dim 256: 32-token tiles
    (256, 8, 2, [40, 300], 70, False, True),      # head dim 256, paged, non-causal
]


def _setup(kvq, D, H, KVH, ctx, n, paged, seed, dtype="bf16"):
    B = len(ctx)
    T = max(ctx) + n
    rng = np.random.default_rng(seed)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), dtype)
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, n, D))
    if paged:
        table, npages = random_block_table(rng, [T] * B)
        cache = kvq.Int8KVCache(B, H, KVH, D, num_pages=npages, block_table=dev_tensor(table), fill=0)
    else:
        cache = kvq.Int8KVCache(B, H, KVH, D, max_len=T, fill=0)
    cache.append(kv_dev(x["k_raw"]), kv_dev(x["v_raw"]), dev_tensor(np.zeros(B, np.int32)))
    return x, qb, qv, cache, T


def _chunk(cache, qb, ctx, causal, scale, hint):
    import torch
    out = cache.chunk(bf16_dev(qb), dev_tensor(np.asarray(ctx, np.int32)), causal, scale, hint)
    torch.cuda.synchronize()
    return to_host_bits(out)


def _oracle(x, qv, ctx, causal, scale):
    kc, ks = orc.quantize(x["k"], 0)
    vc, vs = orc.quantize(x["v"], 0)
    return orc.attention_chunk(qv, orc.dequantize_exact(kc, ks), orc.dequantize_exact(vc, vs), ctx, causal, scale)


@pytest.mark.parametrize("D,H,KVH,ctx,n,causal,paged", CASES)
def test_chunk_matches_oracle(kvq, D, H, KVH, ctx, n, causal, paged):
    log(f"chunk: D={D} H={H} KVH={KVH} ctx={ctx} n={n} causal={causal} paged={paged}")
    x, qb, qv, cache, T = _setup(kvq, D, H, KVH, ctx, n, paged, seed=D + H + n + len(ctx))
    scale = 1.0 / np.sqrt(D)
    got = _chunk(cache, qb, ctx, causal, scale, max(ctx))
    ref = _oracle(x, qv, ctx, causal, scale)
    assert_attention_close(got, ref, "chunk")


def test_chunk_rows_equal_decode(kvq):
    """Causal row i == decode over L0 + i + 1 tokens (same cache, same query)."""
    import torch
    log("chunk: rows vs decode")
    D, H, KVH, ctx, n = 128, 32, 8, [300, 1200], 80
    x, qb, qv, cache, T = _setup(kvq, D, H, KVH, ctx, n, False, seed=11)
    scale = 1.0 / np.sqrt(D)
    got = orc.bf16_bits_to_f32(_chunk(cache, qb, ctx, True, scale, max(ctx))).astype(np.float64)
    for i in (0, 1, 31, 32, 63, 79):
        lens = np.asarray(ctx, np.int32) + i + 1
        q_i = np.ascontiguousarray(qb[:, :, i])
        out = cache.decode(bf16_dev(q_i), dev_tensor(lens), scale, int(lens.max()))
        torch.cuda.synchronize()
        assert_attention_close(to_host_bits(out), got[:, :, i], f"decode vs chunk row {i}")


def test_chunk_paged_equals_contiguous(kvq):
    """Identical logical content in both layouts gives identical bits."""
    log("chunk: paged == contiguous")
    D, H, KVH, ctx, n = 128, 32, 8, [77, 640], 65
    outs = []
    for paged in (False, True):
        x, qb, qv, cache, T = _setup(kvq, D, H, KVH, ctx, n, paged, seed=5)
        outs.append(_chunk(cache, qb, ctx, True, 0.09, max(ctx)))
    assert np.array_equal(outs[0], outs[1])


def test_chunk_single_token_context(kvq):
    """ctx 0, n 1: the only visible key is the query's own row, so out = V-hat."""
    log("chunk: single visible token")
    D, H, KVH = 128, 8, 2
    x, qb, qv, cache, T = _setup(kvq, D, H, KVH, [0, 0], 1, False, seed=9)
    got = _chunk(cache, qb, [0, 0], True, 0.1, 0)
    vc, vs = orc.quantize(x["v"], 0)
    vhat = orc.dequantize_exact(vc, vs)[:, :, 0]                 # [B, KVH, D]
    ref = np.repeat(vhat, H // KVH, axis=1)[:, :, None, :]       # [B, H, 1, D]
    assert_attention_close(got, ref, "single token")


def test_chunk_full_size_sampled(kvq):
    """Chunked-prefill workload at full size (B4, 32/8 heads, D128, 8192
    cached + 512 new, causal), in the launch configuration the benchmark
    times: codes bit-exact, sampled rows against the oracle."""
    import torch
    w = wl.CHUNK
    log("chunk: full-size workload, sampled rows")
    x = wl.layer_inputs(w, 0)
    B, KVH, T, D = x["k"].shape
    cache = kvq.Int8KVCache(B, w.num_heads, KVH, D, max_len=w.max_len, fill=0)
    # prefill, then append the chunk's own rows, as the step does
    cache.append(kv_dev(np.ascontiguousarray(x["k_raw"][:, :, :w.ctx])),
                 kv_dev(np.ascontiguousarray(x["v_raw"][:, :, :w.ctx])), dev_tensor(np.zeros(B, np.int32)))
    cache.append(kv_dev(np.ascontiguousarray(x["k_raw"][:, :, w.ctx:])),
                 kv_dev(np.ascontiguousarray(x["v_raw"][:, :, w.ctx:])),
                 dev_tensor(np.full(B, w.ctx, np.int32)))
    ctx = [w.ctx] * B
    got = _chunk(cache, x["q_bits"], ctx, True, w.attn_scale, w.ctx)
    kc, ks = orc.quantize(x["k"], 0)
    vc, vs = orc.quantize(x["v"], 0)
    torch.cuda.synchronize()
    assert np.array_equal(cache.k_codes.cpu().numpy(), kc)
    assert np.array_equal(cache.v_codes.cpu().numpy(), vc)
    rng = np.random.default_rng(123)
    hpg = w.num_heads // KVH
    picks = [(int(rng.integers(B)), int(rng.integers(w.num_heads)), int(i))
             for i in list(rng.integers(w.n_new, size=40)) + [0, 31, 32, 511]]
    ref = np.empty((len(picks), D))
    gsel = np.empty((len(picks), D), np.uint16)
    for j, (b, h, i) in enumerate(picks):
        g = h // hpg
        total = w.ctx + i + 1
        kh = orc.dequantize_exact(kc[b, g, :total], ks[b, g, :total])
        vh = orc.dequantize_exact(vc[b, g, :total], vs[b, g, :total])
        ref[j] = orc.softmax_attend(x["q"][b, h, i].astype(np.float64), kh, vh, w.attn_scale, None)
        gsel[j] = got[b, h, i]
    assert_attention_close(gsel, ref, "full-size chunk")


G32_CASES = [
    # D, H, KVH, ctx_lens, n, causal, paged, window
    (128, 32, 8, [0, 100], 37, True, False, 0),
    (128, 32, 8, [513, 64], 96, True, True, 0),
    (64, 8, 2, [17, 300], 70, False, False, 0),
    (64, 16, 4, [200], 33, True, True, 0),
    (128, 32, 8, [700], 130, True, False, 129),
]


@pytest.mark.parametrize("D,H,KVH,ctx,n,causal,paged,window", G32_CASES)
def test_chunk_group32(kvq, D, H, KVH, ctx, n, causal, paged, window):
    """Group-32 scales (realizar kv_cache_q8_init.rs layout): the oracle
    dequantizes each 32-element group with its own scale.  Inputs carry a
    different magnitude per group, so the group scales differ widely."""
    import torch
    log(f"chunk group-32: D={D} H={H} KVH={KVH} ctx={ctx} n={n} causal={causal} paged={paged} w={window}")
    B = len(ctx)
    T = max(ctx) + n
    rng = np.random.default_rng(D + n + paged + window)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "f32")
    gain = np.repeat(np.float32(2.0) ** rng.integers(-4, 5, size=(1, KVH, 1, D // 32)).astype(np.float32), 32, -1)
    k, v = (x["k"] * gain).astype(np.float32), (x["v"] * gain[..., ::-1]).astype(np.float32)
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, n, D))
    if paged:
        table, npages = random_block_table(rng, [T] * B)
        cache = kvq.Int8KVCache(B, H, KVH, D, num_pages=npages, block_table=dev_tensor(table), fill=0, group32=True)
    else:
        cache = kvq.Int8KVCache(B, H, KVH, D, max_len=T, fill=0, group32=True)
    cache.append(kv_dev(k), kv_dev(v), dev_tensor(np.zeros(B, np.int32)))
    scale = 1.0 / np.sqrt(D)
    out = cache.chunk(bf16_dev(qb), dev_tensor(np.asarray(ctx, np.int32)), causal, scale, max(ctx), window=window)
    torch.cuda.synchronize()
    kc, ks = orc.quantize(k, 32)
    vc, vs = orc.quantize(v, 32)
    ref = orc.attention_chunk(qv, orc.dequantize_exact(kc, ks), orc.dequantize_exact(vc, vs), ctx, causal, scale,
                              window=window)
    assert_attention_close(to_host_bits(out), ref, "chunk group-32")


GENERIC_CASES = [
    # D, H, KVH, ctx_lens, n, causal, paged, window, mode
    (256, 16, 4, [0, 100], 37, True, False, 0, "token"),
    (256, 8, 2, [300], 20, False, True, 0, "token"),
    (32, 8, 2, [513, 64], 45, True, False, 0, "token"),
    (32, 4, 4, [90], 33, True, True, 17, "token"),
    (256, 16, 4, [200], 30, True, False, 0, "group32"),
    (32, 8, 2, [130, 7], 25, True, False, 0, "bf16"),
    (256, 8, 2, [150], 40, True, True, 64, "e4m3"),
    (32, 8, 2, [70], 19, False, False, 0, "e5m2"),
]


@pytest.mark.parametrize("D,H,KVH,ctx,n,causal,paged,window,mode", GENERIC_CASES)
def test_chunk_generic_head_dims(kvq, D, H, KVH, ctx, n, causal, paged, window, mode):
    """Every scale mode at head dims 32 (no MFMA chunk kernel: each
    (sequence, query) pair runs as a decode over the keys it sees, with the
    same masks) and 256 (the MFMA kernel with 32-token tiles)."""
    import torch
    log(f"chunk generic: D={D} H={H} KVH={KVH} ctx={ctx} n={n} causal={causal} paged={paged} w={window} {mode}")
    B = len(ctx)
    T = max(ctx) + n
    rng = np.random.default_rng(D + n + paged + window + len(mode))
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "bf16", scale=1.5)
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, n, D))
    kw = dict(group32=mode == "group32", scale_bf16=mode == "bf16", fp8=mode if mode in ("e4m3", "e5m2") else None)
    if paged:
        table, npages = random_block_table(rng, [T] * B)
        cache = kvq.Int8KVCache(B, H, KVH, D, num_pages=npages, block_table=dev_tensor(table), fill=0, **kw)
    else:
        cache = kvq.Int8KVCache(B, H, KVH, D, max_len=T, fill=0, **kw)
    cache.append(kv_dev(x["k_raw"]), kv_dev(x["v_raw"]), dev_tensor(np.zeros(B, np.int32)))
    scale = 1.0 / np.sqrt(D)
    out = cache.chunk(bf16_dev(qb), dev_tensor(np.asarray(ctx, np.int32)), causal, scale, max(ctx), window=window)
    torch.cuda.synchronize()
    if mode in ("e4m3", "e5m2"):
        kh = orc.fp8_decode(orc.fp8_encode(x["k"], mode), mode)
        vh = orc.fp8_decode(orc.fp8_encode(x["v"], mode), mode)
    elif mode == "bf16":
        kc, ksb = orc.quantize_bf16_scale(x["k"])
        vc, vsb = orc.quantize_bf16_scale(x["v"])
        kh = orc.dequantize_exact(kc, orc.bf16_bits_to_f32(ksb))
        vh = orc.dequantize_exact(vc, orc.bf16_bits_to_f32(vsb))
    else:
        grp = 32 if mode == "group32" else 0
        kc, ks = orc.quantize(x["k"], grp)
        vc, vs = orc.quantize(x["v"], grp)
        kh, vh = orc.dequantize_exact(kc, ks), orc.dequantize_exact(vc, vs)
    ref = orc.attention_chunk(qv, kh, vh, ctx, causal, scale, window=window)
    assert_attention_close(to_host_bits(out), ref, f"chunk generic D={D} {mode}")
