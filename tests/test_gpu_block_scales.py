"""GPU parity of the block-scale modes (abaddon kv_cache_quant_cuda.rs,
QuantGranularity PerHead / PerChannel, taken over position-aligned blocks of
16 rows of a hybrid cache) against the oracle's BlockRecentCache: the append
state bit-exact after every call (codes of every quantized block, its scales
and the window's bf16 ring rows), the get_kv view exact, and decode, the
fused step and chunked prefill within the attention bar.  Per-head scales
run on the per-token kernels (streaming decode and MFMA chunk at 64 and
128); per-channel scales on the generic kernel."""

import numpy as np
import pytest

import oracle as orc
import workloads as wl
from kvq_testlib import (assert_attention_close, bf16_dev, dev_tensor, kv_dev, log, random_block_table,
                         to_host_bits)

pytestmark = pytest.mark.gpu
BLK = 16


def _bits(values):
    return orc.f32_to_bf16_bits(np.asarray(values, np.float32))


def _new_cache(kvq, B, H, KVH, D, gran, W, cap, paged, capacity, rng=None, lens=None):
    capacity = -(-capacity // BLK) * BLK
    if paged:
        table, npages = random_block_table(rng, lens if lens is not None else [capacity] * B)
        return kvq.Int8KVCache(B, H, KVH, D, num_pages=npages, block_table=dev_tensor(table), fill=0,
                               recent_window=W, recent_capacity=cap, block_scales=gran), table
    return kvq.Int8KVCache(B, H, KVH, D, max_len=capacity, fill=0, recent_window=W, recent_capacity=cap,
                           block_scales=gran), None


def _rows(arena, table, b, n):
    return arena[b, :, :n] if table is None else orc.paged_gather(arena, table, b, n)


def _block_scales(sc, table, b, nblk):
    """Per-channel scales of sequence b's first nblk blocks as [KVH, nblk, D]."""
    if table is None:
        return sc[b, :, :nblk]
    return np.stack([sc[table[b, j]] for j in range(nblk)], axis=1)


def _check_state(cache, table, refs, gran, what):
    import torch
    codes = [t.cpu().numpy() for t in (cache.k_codes, cache.v_codes)]
    scales = [t.cpu().numpy() for t in (cache.k_scales, cache.v_scales)]
    rings = [t.view(torch.int16).cpu().numpy().view(np.uint16) for t in (cache.k_recent, cache.v_recent)]
    cap = rings[0].shape[2]
    for b, ref in enumerate(refs):
        L, nq = ref.seq_len(), ref.quantized_len()
        for side in range(2):
            nrow = ref.codes[side].shape[1]
            if nrow:
                assert np.array_equal(_rows(codes[side], table, b, nrow), ref.codes[side]), \
                    f"{what}: codes side {side} sequence {b}"
                if gran == "head":
                    got = _rows(scales[side], table, b, nrow)
                    assert np.array_equal(got.view(np.uint32), ref.row_scales(side).view(np.uint32)), \
                        f"{what}: per-head scales side {side} sequence {b}"
                else:
                    got = _block_scales(scales[side], table, b, nrow // BLK)
                    assert np.array_equal(got.view(np.uint32), ref.scales[side].view(np.uint32)), \
                        f"{what}: per-channel scales side {side} sequence {b}"
            slots = [t % cap for t in range(nq, L)]
            assert np.array_equal(rings[side][b][:, slots], _bits(ref.rows[side][:, nq:L])), \
                f"{what}: ring side {side} sequence {b}"


def _write_state(cache, table, refs, gran):
    """Place oracle states (ragged lengths) into the device cache."""
    import torch
    codes = [t.cpu().numpy() for t in (cache.k_codes, cache.v_codes)]
    scales = [t.cpu().numpy() for t in (cache.k_scales, cache.v_scales)]
    rings = [t.view(torch.int16).cpu().numpy().view(np.uint16) for t in (cache.k_recent, cache.v_recent)]
    cap = rings[0].shape[2]
    for b, ref in enumerate(refs):
        L, nq = ref.seq_len(), ref.quantized_len()
        for side in range(2):
            nrow = ref.codes[side].shape[1]
            rs = ref.row_scales(side)
            for t in range(nrow):
                if table is None:
                    codes[side][b, :, t] = ref.codes[side][:, t]
                    if gran == "head":
                        scales[side][b, :, t] = rs[:, t]
                else:
                    phys, slot = orc.page_slot(table, b, t)
                    codes[side][phys, :, slot] = ref.codes[side][:, t]
                    if gran == "head":
                        scales[side][phys, :, slot] = rs[:, t]
            if gran == "channel":
                for j in range(nrow // BLK):
                    if table is None:
                        scales[side][b, :, j] = ref.scales[side][:, j]
                    else:
                        scales[side][table[b, j]] = ref.scales[side][:, j]
            for t in range(nq, L):
                rings[side][b, :, t % cap] = _bits(ref.rows[side][:, t])
    for dst, src in zip((cache.k_codes, cache.v_codes, cache.k_scales, cache.v_scales), codes + scales):
        dst.copy_(torch.from_numpy(src))
    cache.k_recent.view(torch.int16).copy_(torch.from_numpy(rings[0].view(np.int16)))
    cache.v_recent.view(torch.int16).copy_(torch.from_numpy(rings[1].view(np.int16)))


def _oracle_states(x, lens, W, gran):
    refs = []
    for b, L in enumerate(lens):
        c = orc.BlockRecentCache(x["k"].shape[1], x["k"].shape[3], W, gran, block=BLK)
        pos = 0
        for n in (L // 3, 1, L):
            n = min(n, L - pos)
            if n > 0:
                c.append(x["k"][b, :, pos:pos + n], x["v"][b, :, pos:pos + n])
                pos += n
        refs.append(c)
    return refs


APPEND_CASES = [
    # gran, D, dtype, W, cap, paged, chunks
    ("head", 64, "bf16", 15, 16, False, [3, 1, 20, 1, 1, 40, 5, 17, 1]),
    ("channel", 64, "f32", 15, 19, False, [1, 1, 14, 1, 33, 2, 16, 16]),
    ("head", 128, "f32", 20, 24, True, [30, 1, 1, 8, 1, 50]),
    ("channel", 96, "bf16", 17, 18, True, [16, 1, 47, 3]),
]


@pytest.mark.parametrize("gran,D,dtype,W,cap,paged,chunks", APPEND_CASES)
def test_append_block_state(kvq, gran, D, dtype, W, cap, paged, chunks):
    """After every kvq_append_recent call: every quantized block's codes and
    scales, and the window's ring rows, equal the oracle's."""
    B, H, KVH = 3, 8, 2
    T = sum(chunks)
    log(f"block append: {gran} D={D} dtype={dtype} W={W} cap={cap} paged={paged} chunks={chunks}")
    rng = np.random.default_rng(W * 7 + cap + D + len(gran))
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), dtype, scale=2.0)
    cache, table = _new_cache(kvq, B, H, KVH, D, gran, W, cap, paged, T, rng)
    refs = [orc.BlockRecentCache(KVH, D, W, gran, block=BLK) for _ in range(B)]
    pos = 0
    for n in chunks:
        cache.append(kv_dev(np.ascontiguousarray(x["k_raw"][:, :, pos:pos + n])),
                     kv_dev(np.ascontiguousarray(x["v_raw"][:, :, pos:pos + n])),
                     dev_tensor(np.full(B, pos, np.int32)))
        for b in range(B):
            refs[b].append(x["k"][b, :, pos:pos + n], x["v"][b, :, pos:pos + n])
        pos += n
        _check_state(cache, table, refs, gran, f"after {pos} tokens")


DECODE_CASES = [
    # gran, D, H, KVH, W, lens, paged
    ("head", 128, 32, 8, 16, [1, 15, 16, 17, 33, 300, 1000], False),
    ("channel", 128, 32, 8, 16, [1, 16, 17, 40, 700], False),
    ("head", 64, 8, 2, 31, [5, 47, 48, 600], True),
    ("channel", 64, 8, 2, 15, [16, 31, 32, 333], True),
    ("head", 96, 8, 2, 20, [21, 36, 500], False),
    ("channel", 256, 8, 2, 15, [3, 100, 257], False),
]


@pytest.mark.parametrize("gran,D,H,KVH,W,lens,paged", DECODE_CASES)
def test_decode_block(kvq, gran, D, H, KVH, W, lens, paged):
    import torch
    log(f"block decode: {gran} D={D} H={H} KVH={KVH} W={W} lens={lens} paged={paged}")
    B, T = len(lens), max(lens)
    rng = np.random.default_rng(D + H + W + paged + len(gran))
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "bf16")
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, D))
    refs = _oracle_states(x, lens, W, gran)
    cache, table = _new_cache(kvq, B, H, KVH, D, gran, W, W + 3, paged, T, rng, lens)
    _write_state(cache, table, refs, gran)
    scale = 1.0 / np.sqrt(D)
    out = cache.decode(bf16_dev(qb), dev_tensor(np.asarray(lens, np.int32)), scale, T)
    torch.cuda.synchronize()
    assert_attention_close(to_host_bits(out), orc.attention_decode_recent(qv, refs, scale), "block decode")


@pytest.mark.parametrize("gran,D,paged,W", [("head", 128, False, 15), ("channel", 128, True, 15), ("head", 64, True, 15),
                                            ("channel", 96, False, 15), ("head", 128, True, 20), ("head", 128, False, 33)])
def test_fused_step_block(kvq, gran, D, paged, W):
    """kvq_append_decode_recent on block scales: the step that moves a
    block's first row out of the window quantizes the whole block (per-head
    scales: inside the fused decode kernel, which with W = 15 takes the
    block's last row from the step's input); state and attention against the
    oracle over steps that cross block edges, and the same state and output,
    bit for bit, as kvq_append_recent followed by kvq_attention_decode_recent."""
    import torch
    B, H, KVH = 3, 8, 2
    lens0 = [14, 16, 40]
    steps = 20 + W
    T = max(lens0) + steps
    log(f"block fused: {gran} D={D} paged={paged} W={W}")
    rng = np.random.default_rng(D + paged + len(gran) + W)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "f32")
    refs = _oracle_states(x, lens0, W, gran)
    caches = []
    for _ in range(2):
        c, table = _new_cache(kvq, B, H, KVH, D, gran, W, W + 1, paged, T, np.random.default_rng(9), [T] * B)
        _write_state(c, table, refs, gran)
        caches.append(c)
    cache, two = caches
    lens = np.asarray(lens0, np.int32)
    scale = 1.0 / np.sqrt(D)
    for s in range(steps):
        lens = lens + 1
        idx = lens - 1
        k_new = np.ascontiguousarray(np.stack([x["k"][b, :, idx[b]:idx[b] + 1] for b in range(B)]))
        v_new = np.ascontiguousarray(np.stack([x["v"][b, :, idx[b]:idx[b] + 1] for b in range(B)]))
        for b in range(B):
            refs[b].append(k_new[b], v_new[b])
        qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, D))
        out = cache.append_decode(kv_dev(k_new), kv_dev(v_new), bf16_dev(qb), dev_tensor(lens), scale, T)
        two.append(kv_dev(k_new), kv_dev(v_new), dev_tensor(idx.astype(np.int32)))
        out2 = two.decode(bf16_dev(qb), dev_tensor(lens), scale, T)
        torch.cuda.synchronize()
        _check_state(cache, table, refs, gran, f"step {s}")
        for name in ("k_codes", "v_codes", "k_scales", "v_scales", "k_recent", "v_recent"):
            assert torch.equal(getattr(cache, name), getattr(two, name)), f"step {s}: {name}"
        assert np.array_equal(to_host_bits(out), to_host_bits(out2)), f"step {s}: fused and two-step outputs"
        assert_attention_close(to_host_bits(out), orc.attention_decode_recent(qv, refs, scale), f"step {s}")


@pytest.mark.parametrize("gran,D,paged", [("head", 128, False), ("head", 64, True), ("channel", 128, False),
                                          ("channel", 64, True)])
def test_chunk_block(kvq, gran, D, paged):
    """A causal chunk appended through kvq_append_recent (blocks triggered
    inside the chunk), then kvq_attention_chunk_recent over the get_kv view."""
    import torch
    B, H, KVH, W = 2, 8, 2, 16
    ctx, n = [37, 160], 40
    lens = [c + n for c in ctx]
    T = max(lens)
    log(f"block chunk: {gran} D={D} paged={paged}")
    rng = np.random.default_rng(3 * D + paged + len(gran))
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "bf16")
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, n, D))
    refs = _oracle_states(x, ctx, W, gran)
    cache, table = _new_cache(kvq, B, H, KVH, D, gran, W, W + 5, paged, T, rng, lens)
    _write_state(cache, table, refs, gran)
    rows = lambda a: np.ascontiguousarray(np.stack([a[b, :, c:c + n] for b, c in enumerate(ctx)]))
    ctx_dev = dev_tensor(np.asarray(ctx, np.int32))
    cache.append(kv_dev(rows(x["k_raw"])), kv_dev(rows(x["v_raw"])), ctx_dev)
    for b, ref in enumerate(refs):
        ref.append(x["k"][b, :, ctx[b]:lens[b]], x["v"][b, :, ctx[b]:lens[b]])
    _check_state(cache, table, refs, gran, "chunk append")
    scale = 1.0 / np.sqrt(D)
    out = cache.chunk(bf16_dev(qb), ctx_dev, True, scale, max(ctx))
    torch.cuda.synchronize()
    kh = np.zeros((B, KVH, T, D))
    vh = np.zeros((B, KVH, T, D))
    for b, ref in enumerate(refs):
        kh[b, :, :lens[b]], vh[b, :, :lens[b]] = ref.kv()
    assert_attention_close(to_host_bits(out), orc.attention_chunk(qv, kh, vh, ctx, True, scale), "block chunk")


@pytest.mark.parametrize("gran,paged", [("head", False), ("channel", True), ("channel", False)])
def test_dequant_block_view(kvq, gran, paged):
    """kvq_dequant_recent gives the get_kv view exactly: INT8 rows as
    fl32((c - 128) s) with each element's block scale, recent rows as their
    bf16 values, zeros past L."""
    import torch
    lens = [3, 16, 31, 90]
    W, B, H, KVH, D = 15, 4, 8, 2, 64
    T = 96
    x = wl.random_kv(33, (B, KVH, T, D), "f32")
    refs = _oracle_states(x, lens, W, gran)
    cache, table = _new_cache(kvq, B, H, KVH, D, gran, W, 20, paged, T, np.random.default_rng(4), [T] * B)
    _write_state(cache, table, refs, gran)
    lens_dev = dev_tensor(np.asarray(lens, np.int32))
    for which in (0, 1):
        got = cache.dequant(which, lens_dev, T).cpu().numpy()
        for b, ref in enumerate(refs):
            k, v = ref.kv()
            want = (k if which == 0 else v).astype(np.float32)
            assert np.array_equal(got[b, :, :lens[b]], want), (which, b)
            assert np.all(got[b, :, lens[b]:] == 0)
    torch.cuda.synchronize()
