"""Parity at the full sizes of the cache variants' workloads (recent window,
sliding window, bf16-stored scales, FP8 codes), in the launch configuration
the benchmark times: a kvq_append prefill, then the fused decode step (or
the chunk append and chunked attention) with the workload's hint.  Codes
(and scales) of sampled sequences are checked bit-exact against the oracle,
attention on sampled (sequence, head[, query]) rows that the oracle computes
one by one, and every output must be finite."""

import numpy as np
import pytest

import oracle as orc
import workloads as wl
from kvq_testlib import assert_attention_close, bf16_dev, dev_tensor, kv_dev, log, to_host_bits

pytestmark = pytest.mark.gpu


def _prefill(cache, x, upto, chunk=1024):
    B = x["k"].shape[0]
    for p0 in range(0, upto, chunk):
        n = min(chunk, upto - p0)
        cache.append(kv_dev(np.ascontiguousarray(x["k_raw"][:, :, p0:p0 + n])),
                     kv_dev(np.ascontiguousarray(x["v_raw"][:, :, p0:p0 + n])),
                     dev_tensor(np.full(B, p0, np.int32)))


def _fused_step(cache, w, x, **kw):
    import torch
    B, _, T, _ = x["k"].shape
    out = cache.append_decode(kv_dev(np.ascontiguousarray(x["k_raw"][:, :, w.ctx:])),
                              kv_dev(np.ascontiguousarray(x["v_raw"][:, :, w.ctx:])),
                              bf16_dev(x["q_bits"]), dev_tensor(np.full(B, T, np.int32)), w.attn_scale, T, **kw)
    torch.cuda.synchronize()
    got = to_host_bits(out)
    assert np.all(np.isfinite(orc.bf16_bits_to_f32(got)))
    return got


def _picks(seed, B, H):
    rng = np.random.default_rng(seed)
    return sorted({(int(rng.integers(B)), int(rng.integers(H))) for _ in range(24)} | {(0, 0), (B - 1, H - 1)})


def _check_rows(got, x, picks, hpg, kv_of, scale, what, visible=None):
    """kv_of(b, g) -> (k_hat, v_hat) fp64 [L, D] of the sequence's KV head;
    visible(L) -> first visible key (sliding window)."""
    refs, sels = [], []
    cache_kv = {}
    for b, h in picks:
        g = h // hpg
        if (b, g) not in cache_kv:
            cache_kv[(b, g)] = kv_of(b, g)
        kh, vh = cache_kv[(b, g)]
        lo = visible(kh.shape[0]) if visible else 0
        refs.append(orc.softmax_attend(x["q"][b, h].astype(np.float64), kh[lo:], vh[lo:], scale, None))
        sels.append(got[b, h])
    err, rel = assert_attention_close(np.stack(sels), np.stack(refs), what)
    log(f"  {len(picks)} sampled rows: max abs err {err:.2e}, rel L2 {rel:.2e}")


@pytest.mark.parametrize("name", ["bf16_scales", "fp8_e4m3"])
def test_decode_variant_full_size(kvq, name):
    w = wl.ALL[name]
    fp8 = w.extra.get("fp8")
    log(f"full size {name}: B={w.batch} L={w.ctx + w.n_new}")
    x = wl.layer_inputs(w, 0)
    B, KVH, T, D = x["k"].shape
    cache = kvq.Int8KVCache(B, w.num_heads, KVH, D, max_len=w.max_len, scale_bf16=bool(w.extra.get("scale_bf16")),
                            fp8=fp8)
    _prefill(cache, x, w.ctx)
    got = _fused_step(cache, w, x)
    dk, dv = cache.k_codes.cpu().numpy(), cache.v_codes.cpu().numpy()
    if not fp8:
        import torch
        dks = cache.k_scales.view(torch.int16).cpu().numpy().view(np.uint16)
        dvs = cache.v_scales.view(torch.int16).cpu().numpy().view(np.uint16)
    hat = {}
    for b in sorted({0, B // 2, B - 1}):
        if fp8:
            kc, vc = orc.fp8_encode(x["k"][b], fp8), orc.fp8_encode(x["v"][b], fp8)
            hat[b] = (orc.fp8_decode(kc, fp8), orc.fp8_decode(vc, fp8))
        else:
            kc, ksb = orc.quantize_bf16_scale(x["k"][b])
            vc, vsb = orc.quantize_bf16_scale(x["v"][b])
            assert np.array_equal(dks[b], ksb) and np.array_equal(dvs[b], vsb), f"scales of sequence {b}"
            hat[b] = (orc.dequantize_exact(kc, orc.bf16_bits_to_f32(ksb)),
                      orc.dequantize_exact(vc, orc.bf16_bits_to_f32(vsb)))
        assert np.array_equal(dk[b], kc) and np.array_equal(dv[b], vc), f"codes of sequence {b}"
    picks = [(b, h) for b, h in _picks(5, B, w.num_heads) if b in hat]
    picks += [(b, h) for b in hat for h in (0, w.num_heads - 1)]
    _check_rows(got, x, sorted(set(picks)), w.num_heads // KVH,
                lambda b, g: (hat[b][0][g], hat[b][1][g]), w.attn_scale, name)


def test_recent_window_full_size(kvq):
    """8B-shaped decode on the hybrid cache (W = 128): prefill through the
    hybrid append in 1024-row chunks, then the fused step; sampled sequences
    rebuilt by the oracle's hybrid cache from the same rows."""
    w = wl.RECENT
    W = w.extra["window"]
    x = wl.layer_inputs(w, 0)
    B, KVH, T, D = x["k"].shape
    log(f"full size recent_window: B={B} L={T} W={W}")
    cache = kvq.Int8KVCache(B, w.num_heads, KVH, D, max_len=w.max_len, recent_window=W)
    _prefill(cache, x, w.ctx)
    got = _fused_step(cache, w, x)
    dk = cache.k_codes.cpu().numpy()
    hat = {}
    for b in sorted({0, B - 1}):
        rc = orc.RecentWindowCache(KVH, D, W)
        rc.append(x["k"][b], x["v"][b])
        assert rc.quantized_len() == T - W
        assert np.array_equal(dk[b, :, :T - W], rc.k_codes), f"INT8 rows of sequence {b}"
        hat[b] = rc.kv()
    picks = [(b, h) for b in hat for h in range(0, w.num_heads, 5)]
    _check_rows(got, x, picks, w.num_heads // KVH, lambda b, g: (hat[b][0][g], hat[b][1][g]), w.attn_scale,
                "recent window")


def test_sliding_decode_full_size(kvq):
    """Context 8192, window 1024, fused step with the window."""
    w = wl.SLIDING_DECODE
    win = w.extra["sliding"]
    x = wl.layer_inputs(w, 0)
    B, KVH, T, D = x["k"].shape
    log(f"full size sliding_decode: B={B} L={T} window={win}")
    cache = kvq.Int8KVCache(B, w.num_heads, KVH, D, max_len=w.max_len)
    _prefill(cache, x, w.ctx)
    got = _fused_step(cache, w, x, window=win)
    dk = cache.k_codes.cpu().numpy()
    hat = {}

    def kv_of(b, g):
        kc, ks = orc.quantize(x["k"][b, g], 0)
        vc, vs = orc.quantize(x["v"][b, g], 0)
        if (b, g) == (0, 0):
            assert np.array_equal(dk[0, 0], kc), "codes of sequence 0, KV head 0"
        return orc.dequantize_exact(kc, ks), orc.dequantize_exact(vc, vs)

    _check_rows(got, x, _picks(6, B, w.num_heads), w.num_heads // KVH, kv_of, w.attn_scale, "sliding decode",
                visible=lambda L: max(L - win, 0))
    del hat


@pytest.mark.parametrize("name", ["sliding_chunk", "fp8_chunk", "chunk_group32", "recent_chunk", "chunk_d256"])
def test_chunk_variant_full_size(kvq, name):
    """512 new queries after 8192 cached tokens: with a window of 1024, on
    FP8 E4M3 codes, with group-32 scales, on a hybrid cache whose last 128
    rows are bf16, or at head dim 256."""
    import torch
    w = wl.ALL[name]
    win = w.extra.get("sliding", 0)
    rw = w.extra.get("window", 0)
    fp8 = w.extra.get("fp8")
    x = wl.layer_inputs(w, 0)
    B, KVH, T, D = x["k"].shape
    log(f"full size {name}: B={B} ctx={w.ctx} n={w.n_new} window={win} fp8={fp8} recent={rw}")
    cache = kvq.Int8KVCache(B, w.num_heads, KVH, D, max_len=w.max_len, fp8=fp8, group32=(w.group == 32),
                            recent_window=rw)
    _prefill(cache, x, w.ctx)
    cache.append(kv_dev(np.ascontiguousarray(x["k_raw"][:, :, w.ctx:])),
                 kv_dev(np.ascontiguousarray(x["v_raw"][:, :, w.ctx:])), dev_tensor(np.full(B, w.ctx, np.int32)))
    out = cache.chunk(bf16_dev(x["q_bits"]), dev_tensor(np.full(B, w.ctx, np.int32)), True, w.attn_scale, w.ctx,
                      window=win)
    torch.cuda.synchronize()
    got = to_host_bits(out)
    assert np.all(np.isfinite(orc.bf16_bits_to_f32(got)))
    dk = cache.k_codes.cpu().numpy()
    hpg = w.num_heads // KVH
    rng = np.random.default_rng(17)
    picks = sorted({(int(rng.integers(B)), int(rng.integers(w.num_heads)), int(i))
                    for i in list(rng.integers(w.n_new, size=30)) + [0, 31, 32, w.n_new - 1]})
    hat = {}
    refs, sels = [], []
    for b, h, i in picks:
        g = h // hpg
        if (b, g) not in hat:
            if rw:  # the oracle's hybrid cache holding the same rows
                rc = orc.RecentWindowCache(1, D, rw, w.group)
                rc.append(x["k"][b, g:g + 1], x["v"][b, g:g + 1])
                assert np.array_equal(dk[b, g, :T - rw], rc.k_codes[0]), f"INT8 rows of sequence {b}, KV head {g}"
                hat[(b, g)] = tuple(a[0] for a in rc.kv())
            elif fp8:
                kc, vc = orc.fp8_encode(x["k"][b, g], fp8), orc.fp8_encode(x["v"][b, g], fp8)
                hat[(b, g)] = (orc.fp8_decode(kc, fp8), orc.fp8_decode(vc, fp8))
            else:
                kc, ks = orc.quantize(x["k"][b, g], w.group)
                vc, vs = orc.quantize(x["v"][b, g], w.group)
                hat[(b, g)] = (orc.dequantize_exact(kc, ks), orc.dequantize_exact(vc, vs))
            if not rw:
                assert np.array_equal(dk[b, g], kc), f"codes of sequence {b}, KV head {g}"
        kh, vh = hat[(b, g)]
        total = w.ctx + i + 1
        lo = max(total - win, 0) if win else 0
        refs.append(orc.softmax_attend(x["q"][b, h, i].astype(np.float64), kh[lo:total], vh[lo:total],
                                       w.attn_scale, None))
        sels.append(got[b, h, i])
    err, rel = assert_attention_close(np.stack(sels), np.stack(refs), name)
    log(f"  {len(picks)} sampled rows: max abs err {err:.2e}, rel L2 {rel:.2e}")
