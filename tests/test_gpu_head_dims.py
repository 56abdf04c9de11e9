"""GPU parity at the head dims whose 16-byte lane count is not a power of two
(96, 160, 192, 224: realizar's cache takes any head_dim that is a multiple
of 32), against the fp64 oracle: decode (contiguous and paged, every scale
mode), the fused step, chunked prefill and the recent-window cache.  These
run on the generic kernel, whose lane groups are padded to a power of two."""

import numpy as np
import pytest

import oracle as orc
import workloads as wl
from kvq_testlib import assert_attention_close, bf16_dev, dev_tensor, kv_dev, log, random_block_table, to_host_bits

pytestmark = pytest.mark.gpu

DIMS = [96, 160, 192, 224]


def _cache(kvq, B, H, KVH, D, T, mode, paged, rng):
    kw = dict(group32=(mode == "g32"), scale_bf16=(mode == "bf16"), fp8=("e4m3" if mode == "fp8" else None), fill=0)
    if paged:
        table, npages = random_block_table(rng, [T] * B)
        return kvq.Int8KVCache(B, H, KVH, D, num_pages=npages, block_table=dev_tensor(table), **kw)
    return kvq.Int8KVCache(B, H, KVH, D, max_len=T, **kw)


def _oracle_kv(x, mode):
    if mode == "fp8":
        return (orc.fp8_decode(orc.fp8_encode(x["k"], "e4m3"), "e4m3"),
                orc.fp8_decode(orc.fp8_encode(x["v"], "e4m3"), "e4m3"))
    if mode == "bf16":
        kc, ks = orc.quantize_bf16_scale(x["k"])
        vc, vs = orc.quantize_bf16_scale(x["v"])
        return (orc.dequantize_exact(kc, orc.bf16_bits_to_f32(ks)), orc.dequantize_exact(vc, orc.bf16_bits_to_f32(vs)))
    g = 32 if mode == "g32" else 0
    kc, ks = orc.quantize(x["k"], g)
    vc, vs = orc.quantize(x["v"], g)
    return orc.dequantize_exact(kc, ks), orc.dequantize_exact(vc, vs)


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("mode,paged", [("token", False), ("g32", False), ("bf16", False), ("fp8", False),
                                        ("token", True)])
def test_decode(kvq, D, mode, paged):
    import torch
    log(f"head dims: decode D={D} mode={mode} paged={paged}")
    lens = [1, 63, 64, 65, 700]
    B, H, KVH, T = len(lens), 8, 2, max(lens)
    rng = np.random.default_rng(D + len(mode) + paged)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "bf16")
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, D))
    cache = _cache(kvq, B, H, KVH, D, T, mode, paged, rng)
    cache.append(kv_dev(x["k_raw"]), kv_dev(x["v_raw"]), dev_tensor(np.zeros(B, np.int32)))
    scale = 1.0 / np.sqrt(D)
    out = cache.decode(bf16_dev(qb), dev_tensor(np.asarray(lens, np.int32)), scale, T)
    torch.cuda.synchronize()
    kh, vh = _oracle_kv(x, mode)
    assert_attention_close(to_host_bits(out), orc.attention_decode(qv, kh, vh, lens, scale), f"decode D={D}")


@pytest.mark.parametrize("D", DIMS)
def test_fused_step_and_chunk(kvq, D):
    """The fused append + decode (append launch, then the generic kernel) and a
    causal chunk, per-token scales, against the oracle."""
    import torch
    log(f"head dims: fused step and chunk D={D}")
    B, H, KVH, ctx, n = 2, 8, 2, [130, 7], 40
    T = max(ctx) + n
    rng = np.random.default_rng(3 * D)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "bf16")
    cache = kvq.Int8KVCache(B, H, KVH, D, max_len=T, fill=0)
    cache.append(kv_dev(x["k_raw"]), kv_dev(x["v_raw"]), dev_tensor(np.zeros(B, np.int32)))
    kh, vh = _oracle_kv(x, "token")
    scale = 1.0 / np.sqrt(D)
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, n, D))
    out = cache.chunk(bf16_dev(qb), dev_tensor(np.asarray(ctx, np.int32)), True, scale, max(ctx))
    torch.cuda.synchronize()
    assert_attention_close(to_host_bits(out), orc.attention_chunk(qv, kh, vh, ctx, True, scale), f"chunk D={D}")
    # fused step: the last token of each sequence, re-appended by the step
    lens = np.asarray([T, T - 5], np.int32)
    idx = lens - 1
    k_new = np.ascontiguousarray(x["k_raw"][np.arange(B), :, idx][:, :, None, :])
    v_new = np.ascontiguousarray(x["v_raw"][np.arange(B), :, idx][:, :, None, :])
    qd, qdv = wl.random_q(int(rng.integers(1 << 30)), (B, H, D))
    out = cache.append_decode(kv_dev(k_new), kv_dev(v_new), bf16_dev(qd), dev_tensor(lens), scale, T)
    torch.cuda.synchronize()
    assert_attention_close(to_host_bits(out), orc.attention_decode(qdv, kh, vh, lens, scale), f"fused D={D}")


@pytest.mark.parametrize("D", [96, 224])
def test_recent_window(kvq, D):
    """Hybrid cache (last 16 tokens bf16, older ones INT8) decode against the
    oracle's RecentWindowCache, after one append of the whole history."""
    import torch
    log(f"head dims: recent window D={D}")
    B, H, KVH, W, T = 2, 8, 2, 16, 100
    rng = np.random.default_rng(5 * D)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "f32")
    cache = kvq.Int8KVCache(B, H, KVH, D, max_len=T, recent_window=W, fill=0)
    cache.append(kv_dev(x["k"]), kv_dev(x["v"]), dev_tensor(np.zeros(B, np.int32)))
    refs = []
    for b in range(B):
        rc = orc.RecentWindowCache(KVH, D, W)
        rc.append(x["k"][b], x["v"][b])
        refs.append(rc)
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, D))
    scale = 1.0 / np.sqrt(D)
    out = cache.decode(bf16_dev(qb), dev_tensor(np.full(B, T, np.int32)), scale, T)
    torch.cuda.synchronize()
    assert_attention_close(to_host_bits(out), orc.attention_decode_recent(qv, refs, scale), f"recent D={D}")
