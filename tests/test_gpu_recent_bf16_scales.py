"""GPU parity of a recent-window cache whose INT8 rows keep bf16-stored
per-token scales (KVQ_SCALE_PER_TOKEN_BF16): the append state (codes equal to
the oracle hybrid cache's, scales equal to the bf16 rounding of its fp32
scales, ring rows its bf16 values) after every call; decode, the fused step
and chunked prefill against the oracle's attention over the get_kv view in
which the old rows are dequantized with the stored bf16 scales."""

import numpy as np
import pytest

import oracle as orc
import workloads as wl
from kvq_testlib import (assert_attention_close, bf16_dev, dev_tensor, kv_dev, log, random_block_table,
                         to_host_bits)

pytestmark = pytest.mark.gpu


def _new_cache(kvq, B, H, KVH, D, W, cap, paged, T, rng, lens=None):
    if paged:
        table, npages = random_block_table(rng, lens if lens is not None else [T] * B)
        return kvq.Int8KVCache(B, H, KVH, D, num_pages=npages, block_table=dev_tensor(table), fill=0,
                               scale_bf16=True, recent_window=W, recent_capacity=cap), table
    return kvq.Int8KVCache(B, H, KVH, D, max_len=T, fill=0, scale_bf16=True, recent_window=W,
                           recent_capacity=cap), None


def _u16(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _rows(arena, table, b, n):
    return arena[b, :, :n] if table is None else orc.paged_gather(arena, table, b, n)


class _Bf16View:
    """The oracle hybrid cache read with its scales rounded to bf16, as the
    device stores them."""

    def __init__(self, ref):
        self.ref = ref

    def seq_len(self):
        return self.ref.seq_len()

    def kv(self):
        r = self.ref
        rnd = lambda s: orc.bf16_bits_to_f32(orc.f32_to_bf16_bits(s))
        k = np.concatenate([orc.dequantize_exact(r.k_codes, rnd(r.k_scales)), r.k_recent.astype(np.float64)], axis=1)
        v = np.concatenate([orc.dequantize_exact(r.v_codes, rnd(r.v_scales)), r.v_recent.astype(np.float64)], axis=1)
        return k, v


def _check_state(cache, table, refs, what):
    kc, vc = cache.k_codes.cpu().numpy(), cache.v_codes.cpu().numpy()
    ks, vs = _u16(cache.k_scales), _u16(cache.v_scales)
    kr, vr = _u16(cache.k_recent), _u16(cache.v_recent)
    cap = kr.shape[2]
    for b, ref in enumerate(refs):
        nq, L = ref.quantized_len(), ref.seq_len()
        if nq:
            assert np.array_equal(_rows(kc, table, b, nq), ref.k_codes), f"{what}: K codes of sequence {b}"
            assert np.array_equal(_rows(vc, table, b, nq), ref.v_codes), f"{what}: V codes of sequence {b}"
            assert np.array_equal(_rows(ks, table, b, nq), orc.f32_to_bf16_bits(ref.k_scales)), f"{what}: K scales"
            assert np.array_equal(_rows(vs, table, b, nq), orc.f32_to_bf16_bits(ref.v_scales)), f"{what}: V scales"
        slots = [t % cap for t in range(nq, L)]
        assert np.array_equal(kr[b][:, slots], orc.f32_to_bf16_bits(ref.k_recent)), f"{what}: K ring {b}"
        assert np.array_equal(vr[b][:, slots], orc.f32_to_bf16_bits(ref.v_recent)), f"{what}: V ring {b}"


def _write_state(cache, table, refs):
    """Place oracle states (any lengths) into the device cache, scales as bf16 bits."""
    import torch
    kc, vc = cache.k_codes.cpu().numpy(), cache.v_codes.cpu().numpy()
    ks, vs = _u16(cache.k_scales), _u16(cache.v_scales)
    kr, vr = _u16(cache.k_recent), _u16(cache.v_recent)
    cap = kr.shape[2]
    for b, ref in enumerate(refs):
        nq, L = ref.quantized_len(), ref.seq_len()
        ksb, vsb = orc.f32_to_bf16_bits(ref.k_scales), orc.f32_to_bf16_bits(ref.v_scales)
        for t in range(nq):
            if table is None:
                at = (b, slice(None), t)
            else:
                phys, slot = orc.page_slot(table, b, t)
                at = (phys, slice(None), slot)
            kc[at], ks[at] = ref.k_codes[:, t], ksb[:, t]
            vc[at], vs[at] = ref.v_codes[:, t], vsb[:, t]
        for i, t in enumerate(range(nq, L)):
            kr[b, :, t % cap] = orc.f32_to_bf16_bits(ref.k_recent[:, i])
            vr[b, :, t % cap] = orc.f32_to_bf16_bits(ref.v_recent[:, i])
    cache.k_codes.copy_(torch.from_numpy(kc))
    cache.v_codes.copy_(torch.from_numpy(vc))
    for t, a in ((cache.k_scales, ks), (cache.v_scales, vs), (cache.k_recent, kr), (cache.v_recent, vr)):
        t.view(torch.int16).copy_(torch.from_numpy(a.view(np.int16)))


def _oracle_states(x, lens, W):
    refs = []
    for b, L in enumerate(lens):
        c = orc.RecentWindowCache(x["k"].shape[1], x["k"].shape[3], W, 0)
        pos = 0
        for n in (L // 3, 1, L):
            n = min(n, L - pos)
            if n > 0:
                c.append(x["k"][b, :, pos:pos + n], x["v"][b, :, pos:pos + n])
                pos += n
        refs.append(c)
    return refs


@pytest.mark.parametrize("D,dtype,W,cap,paged,chunks", [
    (128, "bf16", 16, 17, False, [3, 1, 7, 1, 1, 20, 1, 40]),
    (64, "f32", 8, 13, True, [30, 1, 1, 8, 1]),
    (256, "f32", 4, 9, False, [1, 1, 1, 2, 5, 1, 13]),
])
def test_append_state(kvq, D, dtype, W, cap, paged, chunks):
    """After every append call: INT8 rows below L - W with bf16 scales, and the
    window's bf16 rows in their ring slots (the row leaving the window is
    quantized with the fp32 scale; the stored scale is its bf16 rounding)."""
    B, H, KVH = 3, 8, 2
    T = sum(chunks)
    log(f"recent bf16 scales append: D={D} dtype={dtype} W={W} cap={cap} paged={paged}")
    rng = np.random.default_rng(D + W + cap + paged)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), dtype, scale=2.0)
    cache, table = _new_cache(kvq, B, H, KVH, D, W, cap, paged, T, rng)
    refs = [orc.RecentWindowCache(KVH, D, W, 0) for _ in range(B)]
    pos = 0
    for n in chunks:
        cache.append(kv_dev(np.ascontiguousarray(x["k_raw"][:, :, pos:pos + n])),
                     kv_dev(np.ascontiguousarray(x["v_raw"][:, :, pos:pos + n])),
                     dev_tensor(np.full(B, pos, np.int32)))
        for b in range(B):
            refs[b].append(x["k"][b, :, pos:pos + n], x["v"][b, :, pos:pos + n])
        pos += n
        _check_state(cache, table, refs, f"after {pos} tokens")


@pytest.mark.parametrize("D,H,KVH,W,lens,paged", [
    (128, 32, 8, 128, [1, 5, 127, 128, 129, 300, 2100], False),   # streaming kernel
    (128, 32, 8, 16, [16, 17, 700, 1025], True),
    (64, 8, 2, 8, [3, 9, 300], False),
    (256, 16, 4, 16, [1, 17, 300, 1100], False),                   # generic kernel
])
def test_decode(kvq, D, H, KVH, W, lens, paged):
    import torch
    log(f"recent bf16 scales decode: D={D} W={W} lens={lens} paged={paged}")
    B, T = len(lens), max(lens)
    rng = np.random.default_rng(D + H + W + paged)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "bf16")
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, D))
    refs = _oracle_states(x, lens, W)
    cache, table = _new_cache(kvq, B, H, KVH, D, W, W + 3, paged, T, rng, lens)
    _write_state(cache, table, refs)
    out = cache.decode(bf16_dev(qb), dev_tensor(np.asarray(lens, np.int32)), 1.0 / np.sqrt(D), T)
    torch.cuda.synchronize()
    ref = orc.attention_decode_recent(qv, [_Bf16View(r) for r in refs], 1.0 / np.sqrt(D))
    assert_attention_close(to_host_bits(out), ref, "decode, recent window, bf16 scales")


@pytest.mark.parametrize("D,paged,dtype", [(128, False, "bf16"), (128, True, "f32"), (256, False, "bf16")])
def test_fused_equals_two_steps(kvq, D, paged, dtype):
    """The fused step equals append-then-decode bit for bit (outputs, codes,
    scales, rings), and both match the oracle."""
    import torch
    lens = [1, 2, 16, 17, 18, 100, 1500, 2049]
    W = 16
    B, H, KVH = len(lens), 32, 8
    T = max(lens)
    log(f"recent bf16 scales fused: D={D} paged={paged} dtype={dtype}")
    rng = np.random.default_rng(17 + D + paged)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), dtype)
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, D))
    before = _oracle_states(x, [L - 1 for L in lens], W)
    caches = []
    for _ in range(2):
        c, table = _new_cache(kvq, B, H, KVH, D, W, W + 1, paged, T, np.random.default_rng(5), lens)
        _write_state(c, table, before)
        caches.append(c)
    idx = np.asarray(lens) - 1
    k_new = kv_dev(np.ascontiguousarray(x["k_raw"][np.arange(B), :, idx][:, :, None, :]))
    v_new = kv_dev(np.ascontiguousarray(x["v_raw"][np.arange(B), :, idx][:, :, None, :]))
    lens_dev = dev_tensor(np.asarray(lens, np.int32))
    q = bf16_dev(qb)
    scale = 0.071
    a, f = caches
    a.append(k_new, v_new, dev_tensor(idx.astype(np.int32)))
    out_a = a.decode(q, lens_dev, scale, T)
    out_f = f.append_decode(k_new, v_new, q, lens_dev, scale, T)
    torch.cuda.synchronize()
    for name in ("k_codes", "v_codes", "k_scales", "v_scales", "k_recent", "v_recent"):
        assert torch.equal(getattr(a, name), getattr(f, name)), name
    assert np.array_equal(to_host_bits(out_a), to_host_bits(out_f))
    for b, ref in enumerate(before):
        ref.append(x["k"][b, :, lens[b] - 1:lens[b]], x["v"][b, :, lens[b] - 1:lens[b]])
    _check_state(f, table, before, "fused step")
    assert_attention_close(to_host_bits(out_f), orc.attention_decode_recent(qv, [_Bf16View(r) for r in before], scale),
                           "fused, recent window, bf16 scales")


@pytest.mark.parametrize("D,H,KVH,W,ctx,n,paged", [
    (128, 32, 8, 128, [0, 700, 2000], 300, False),   # MFMA kernel, ring inside the chunk
    (128, 16, 8, 64, [10, 300], 70, True),
    (64, 8, 2, 16, [3, 100, 0], 37, False),
    (32, 4, 4, 8, [0, 5, 40], 13, False),            # generic kernel
])
def test_chunk(kvq, D, H, KVH, W, ctx, n, paged):
    import torch
    B = len(ctx)
    lens = [c + n for c in ctx]
    T = max(lens)
    log(f"recent bf16 scales chunk: D={D} W={W} ctx={ctx} n={n} paged={paged}")
    rng = np.random.default_rng(D * 3 + W + n + paged)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "bf16")
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, n, D))
    refs = _oracle_states(x, ctx, W)
    cache, table = _new_cache(kvq, B, H, KVH, D, W, W + 5, paged, T, rng, lens)
    _write_state(cache, table, refs)
    rows = lambda a: np.ascontiguousarray(np.stack([a[b, :, c:c + n] for b, c in enumerate(ctx)]))
    ctx_dev = dev_tensor(np.asarray(ctx, np.int32))
    cache.append(kv_dev(rows(x["k_raw"])), kv_dev(rows(x["v_raw"])), ctx_dev)
    for b, ref in enumerate(refs):
        ref.append(x["k"][b, :, ctx[b]:lens[b]], x["v"][b, :, ctx[b]:lens[b]])
    _check_state(cache, table, refs, "chunk append")
    scale = 1.0 / np.sqrt(D)
    out = cache.chunk(bf16_dev(qb), ctx_dev, True, scale, max(ctx))
    torch.cuda.synchronize()
    kh = np.zeros((B, KVH, T, D))
    vh = np.zeros((B, KVH, T, D))
    for b, ref in enumerate(refs):
        kh[b, :, :lens[b]], vh[b, :, :lens[b]] = _Bf16View(ref).kv()
    o = to_host_bits(out)
    assert np.all(np.isfinite(orc.bf16_bits_to_f32(o)))
    assert_attention_close(o, orc.attention_chunk(qv, kh, vh, ctx, True, scale), "chunk, recent window, bf16 scales")
