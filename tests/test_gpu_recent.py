"""GPU parity of the recent-window hybrid cache (the last W positions of a
sequence in bf16, older ones INT8) against the oracle's RecentWindowCache:
append state bit-exact after every call, decode within the attention bar,
the fused step equal to append-then-decode bit for bit, the get_kv view
exact, and chunked prefill over the view within the attention bar at every
head size (one MFMA kernel, its tiles holding INT8 and ring rows, at 64 and
128; the generic kernel's
ring loop at 32 and 256)."""

import numpy as np
import pytest

import oracle as orc
import workloads as wl
from kvq_testlib import (assert_attention_close, bf16_dev, dev_tensor, kv_dev, log, random_block_table,
                         to_host_bits)

pytestmark = pytest.mark.gpu


def _bits(values: np.ndarray) -> np.ndarray:
    return orc.f32_to_bf16_bits(np.asarray(values, np.float32))


def _new_cache(kvq, B, H, KVH, D, group, W, cap, paged, capacity, rng=None, lens=None):
    if paged:
        table, npages = random_block_table(rng, lens if lens is not None else [capacity] * B)
        return kvq.Int8KVCache(B, H, KVH, D, num_pages=npages, block_table=dev_tensor(table),
                               group32=(group == 32), fill=0, recent_window=W, recent_capacity=cap), table
    return kvq.Int8KVCache(B, H, KVH, D, max_len=capacity, group32=(group == 32), fill=0,
                           recent_window=W, recent_capacity=cap), None


def _device_state(cache, table):
    """Host copies of codes, scales and rings, with a per-sequence row reader."""
    kc, ks = cache.k_codes.cpu().numpy(), cache.k_scales.cpu().numpy()
    vc, vs = cache.v_codes.cpu().numpy(), cache.v_scales.cpu().numpy()
    kr = cache.k_recent.view(__import__("torch").int16).cpu().numpy().view(np.uint16)
    vr = cache.v_recent.view(__import__("torch").int16).cpu().numpy().view(np.uint16)

    def rows(arena, b, n):
        if table is None:
            return arena[b, :, :n]
        return orc.paged_gather(arena, table, b, n)
    return kc, ks, vc, vs, kr, vr, rows


def _check_state(cache, table, refs, what):
    """Device INT8 rows below L - W and ring rows of the window equal the oracle."""
    kc, ks, vc, vs, kr, vr, rows = _device_state(cache, table)
    cap = kr.shape[2]
    for b, ref in enumerate(refs):
        nq, L = ref.quantized_len(), ref.seq_len()
        if nq:
            assert np.array_equal(rows(kc, b, nq), ref.k_codes), f"{what}: K codes of sequence {b}"
            assert np.array_equal(rows(vc, b, nq), ref.v_codes), f"{what}: V codes of sequence {b}"
            assert np.array_equal(rows(ks, b, nq).view(np.uint32), ref.k_scales.view(np.uint32)), f"{what}: K scales"
            assert np.array_equal(rows(vs, b, nq).view(np.uint32), ref.v_scales.view(np.uint32)), f"{what}: V scales"
        slots = [t % cap for t in range(nq, L)]
        assert np.array_equal(kr[b][:, slots], _bits(ref.k_recent)), f"{what}: K ring of sequence {b}"
        assert np.array_equal(vr[b][:, slots], _bits(ref.v_recent)), f"{what}: V ring of sequence {b}"


def _write_state(cache, table, refs):
    """Place oracle states (one per sequence, any lengths) into the device cache."""
    import torch
    kc, ks, vc, vs = (t.cpu().numpy() for t in (cache.k_codes, cache.k_scales, cache.v_codes, cache.v_scales))
    kr = cache.k_recent.view(torch.int16).cpu().numpy().view(np.uint16)
    vr = cache.v_recent.view(torch.int16).cpu().numpy().view(np.uint16)
    cap = kr.shape[2]
    for b, ref in enumerate(refs):
        nq, L = ref.quantized_len(), ref.seq_len()
        for t in range(nq):
            if table is None:
                kc[b, :, t], ks[b, :, t] = ref.k_codes[:, t], ref.k_scales[:, t]
                vc[b, :, t], vs[b, :, t] = ref.v_codes[:, t], ref.v_scales[:, t]
            else:
                phys, slot = orc.page_slot(table, b, t)
                kc[phys, :, slot], ks[phys, :, slot] = ref.k_codes[:, t], ref.k_scales[:, t]
                vc[phys, :, slot], vs[phys, :, slot] = ref.v_codes[:, t], ref.v_scales[:, t]
        for i, t in enumerate(range(nq, L)):
            kr[b, :, t % cap] = _bits(ref.k_recent[:, i])
            vr[b, :, t % cap] = _bits(ref.v_recent[:, i])
    for t, a in ((cache.k_codes, kc), (cache.k_scales, ks), (cache.v_codes, vc), (cache.v_scales, vs)):
        t.copy_(torch.from_numpy(a))
    cache.k_recent.view(torch.int16).copy_(torch.from_numpy(kr.view(np.int16)))
    cache.v_recent.view(torch.int16).copy_(torch.from_numpy(vr.view(np.int16)))


def _oracle_states(x, lens, W, group):
    """One RecentWindowCache per sequence holding its first lens[b] tokens,
    appended in a few uneven chunks."""
    refs = []
    for b, L in enumerate(lens):
        c = orc.RecentWindowCache(x["k"].shape[1], x["k"].shape[3], W, group)
        pos = 0
        for n in (L // 3, 1, L):
            n = min(n, L - pos)
            if n > 0:
                c.append(x["k"][b, :, pos:pos + n], x["v"][b, :, pos:pos + n])
                pos += n
        refs.append(c)
    return refs


APPEND_CASES = [
    # group, dtype, W, cap, paged, chunks
    (0, "bf16", 16, 17, False, [3, 1, 7, 1, 1, 20, 1, 40]),
    (32, "f32", 4, 9, False, [1, 1, 1, 2, 5, 1, 13]),
    (0, "f32", 8, 8 + 5, True, [30, 1, 1, 8, 1]),
    (32, "bf16", 1, 2, True, [2, 1, 1, 5]),
]


@pytest.mark.parametrize("group,dtype,W,cap,paged,chunks", APPEND_CASES)
def test_append_recent_state(kvq, group, dtype, W, cap, paged, chunks):
    """After every kvq_append_recent call the device holds the oracle's state:
    INT8 rows below L - W (quantized from bf16 values) and the window's bf16
    rows in their ring slots."""
    B, H, KVH, D = 3, 8, 2, 64
    T = sum(chunks)
    log(f"append recent: group={group} dtype={dtype} W={W} cap={cap} paged={paged} chunks={chunks}")
    rng = np.random.default_rng(W * 13 + cap + group)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), dtype, scale=2.0)
    cache, table = _new_cache(kvq, B, H, KVH, D, group, W, cap, paged, T, rng)
    refs = [orc.RecentWindowCache(KVH, D, W, group) for _ in range(B)]
    pos = 0
    for n in chunks:
        cache.append(kv_dev(np.ascontiguousarray(x["k_raw"][:, :, pos:pos + n])),
                     kv_dev(np.ascontiguousarray(x["v_raw"][:, :, pos:pos + n])),
                     dev_tensor(np.full(B, pos, np.int32)))
        for b in range(B):
            refs[b].append(x["k"][b, :, pos:pos + n], x["v"][b, :, pos:pos + n])
        pos += n
        _check_state(cache, table, refs, f"after {pos} tokens")


DECODE_CASES = [
    # D, H, KVH, group, W, lens, paged
    (128, 32, 8, 0, 128, [1, 5, 127, 128, 129, 300, 2100, 3000], False),
    (128, 32, 8, 32, 16, [16, 17, 700, 1025], False),
    (128, 32, 8, 0, 64, [1, 65, 200, 1000, 16, 33], True),
    (64, 8, 2, 0, 8, [3, 9, 300], False),
    (32, 4, 4, 0, 5, [5, 6, 90], False),
    (128, 24, 8, 0, 32, [40, 517], False),        # one head per workgroup
    (128, 64, 8, 0, 32, [77, 600], False),        # two workgroups per KV head
    (256, 16, 4, 0, 16, [1, 17, 300, 1100], False),  # generic kernel: the ring is its second loop
    (256, 8, 2, 32, 8, [9, 64, 600], True),
]


@pytest.mark.parametrize("D,H,KVH,group,W,lens,paged", DECODE_CASES)
def test_decode_recent(kvq, D, H, KVH, group, W, lens, paged):
    """kvq_attention_decode_recent over ragged hybrid states against the
    oracle's attention over the get_kv view."""
    log(f"decode recent: D={D} H={H} KVH={KVH} group={group} W={W} lens={lens} paged={paged}")
    B, T = len(lens), max(lens)
    rng = np.random.default_rng(D + H + W + group + paged)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "bf16")
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, D))
    refs = _oracle_states(x, lens, W, group)
    cache, table = _new_cache(kvq, B, H, KVH, D, group, W, W + 3, paged, T, rng, lens)
    _write_state(cache, table, refs)
    import torch
    out = cache.decode(bf16_dev(qb), dev_tensor(np.asarray(lens, np.int32)), 1.0 / np.sqrt(D), T)
    torch.cuda.synchronize()
    ref = orc.attention_decode_recent(qv, refs, 1.0 / np.sqrt(D))
    assert_attention_close(to_host_bits(out), ref, "decode recent")


@pytest.mark.parametrize("paged,group,dtype,D", [(False, 0, "bf16", 128), (True, 0, "f32", 128),
                                                 (False, 32, "f32", 128), (True, 32, "bf16", 128),
                                                 (False, 0, "bf16", 256), (True, 32, "f32", 256)])
def test_fused_recent_equals_two_steps(kvq, paged, group, dtype, D):
    """kvq_append_decode_recent == kvq_append_recent (one row at L - 1) then
    kvq_attention_decode_recent, bit for bit (outputs, codes, scales, rings),
    and both match the oracle's state after the step."""
    import torch
    lens = [1, 2, 16, 17, 18, 100, 1500, 2049]
    W = 16
    B, H, KVH = len(lens), 32, 8
    T = max(lens)
    log(f"fused recent: paged={paged} group={group} dtype={dtype} D={D} lens={lens}")
    rng = np.random.default_rng(7 + paged + group)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), dtype)
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, D))
    before = _oracle_states(x, [L - 1 for L in lens], W, group)
    caches = []
    for _ in range(2):
        c, table = _new_cache(kvq, B, H, KVH, D, group, W, W + 1, paged, T,
                              np.random.default_rng(99), lens)
        _write_state(c, table, before)
        caches.append(c)
    idx = np.asarray(lens) - 1
    k_new = kv_dev(np.ascontiguousarray(x["k_raw"][np.arange(B), :, idx][:, :, None, :]))
    v_new = kv_dev(np.ascontiguousarray(x["v_raw"][np.arange(B), :, idx][:, :, None, :]))
    lens_dev = dev_tensor(np.asarray(lens, np.int32))
    q = bf16_dev(qb)
    scale = 0.088
    a, f = caches
    a.append(k_new, v_new, dev_tensor(idx.astype(np.int32)))
    out_a = a.decode(q, lens_dev, scale, T)
    out_f = f.append_decode(k_new, v_new, q, lens_dev, scale, T)
    torch.cuda.synchronize()
    for name in ("k_codes", "v_codes", "k_scales", "v_scales", "k_recent", "v_recent"):
        assert torch.equal(getattr(a, name), getattr(f, name)), name
    assert np.array_equal(to_host_bits(out_a), to_host_bits(out_f))
    after = []
    for b, ref in enumerate(before):
        ref.append(x["k"][b, :, lens[b] - 1:lens[b]], x["v"][b, :, lens[b] - 1:lens[b]])
        after.append(ref)
    _check_state(f, table, after, "fused step")
    assert_attention_close(to_host_bits(out_f), orc.attention_decode_recent(qv, after, scale), "fused recent")


def test_dequant_recent_view(kvq):
    """kvq_dequant_recent gives the get_kv view exactly: INT8 rows as
    fl32((c - 128) s), recent rows as their bf16 values, zeros past L."""
    import torch
    lens = [3, 40, 41, 90]
    W, B, H, KVH, D = 40, 4, 8, 2, 64
    T = 96
    x = wl.random_kv(31, (B, KVH, T, D), "f32")
    refs = _oracle_states(x, lens, W, 32)
    cache, table = _new_cache(kvq, B, H, KVH, D, 32, W, 48, True, T, np.random.default_rng(3), [T] * B)
    _write_state(cache, table, refs)
    lens_dev = dev_tensor(np.asarray(lens, np.int32))
    for which in (0, 1):
        got = cache.dequant(which, lens_dev, T).cpu().numpy()
        for b, ref in enumerate(refs):
            k, v = ref.kv()
            want = (k if which == 0 else v).astype(np.float32)
            assert np.array_equal(got[b, :, :lens[b]], want), (which, b)
            assert np.all(got[b, :, lens[b]:] == 0)
    torch.cuda.synchronize()


def test_recent_longest_first_and_splits(kvq, monkeypatch):
    """Longest-first order and forced short splits leave the hybrid result
    bit-identical."""
    import torch
    lens = [900, 3, 1700, 128, 0, 129, 1700, 64]
    W, B, H, KVH, D = 128, len(lens), 32, 8, 128
    T = max(lens)
    x = wl.random_kv(41, (B, KVH, T, D), "bf16")
    qb, qv = wl.random_q(42, (B, H, D))
    refs = _oracle_states(x, lens, W, 0)
    cache, table = _new_cache(kvq, B, H, KVH, D, 0, W, W + 1, False, T)
    _write_state(cache, table, refs)
    outs = {}
    for env in (("0", "0"), ("512", "1"), ("512", "0")):
        monkeypatch.setenv("KVQ_SPLIT_LEN", env[0])
        monkeypatch.setenv("KVQ_LONGEST_FIRST", env[1])
        out = cache.decode(bf16_dev(qb), dev_tensor(np.asarray(lens, np.int32)), 0.088, T)
        torch.cuda.synchronize()
        outs[env] = to_host_bits(out)
    assert np.array_equal(outs[("512", "1")], outs[("512", "0")])
    live = np.asarray(lens) > 0
    assert np.all(outs[("0", "0")][~live] == 0)
    ref = orc.attention_decode_recent(qv[live], [r for r, L in zip(refs, lens) if L > 0], 0.088)
    for env, o in outs.items():
        assert_attention_close(o[live], ref, f"splits {env}")


CHUNK_CASES = [
    # D, H, KVH, group, W, ctx_lens, n, paged
    (32, 4, 4, 0, 8, [0, 5, 40], 13, False),
    (64, 8, 2, 0, 16, [3, 100, 0], 37, False),
    (128, 32, 8, 32, 64, [0, 200, 1000], 70, True),
    (128, 16, 8, 0, 128, [10, 300], 5, False),       # chunk shorter than the window
    (128, 32, 8, 0, 128, [0, 700, 2000], 300, False),  # several query blocks, ring inside the chunk
    (64, 16, 4, 32, 32, [1, 90, 500], 100, True),
    (128, 32, 8, 0, 16, [0, 33, 300], 1, False),       # one query per sequence
    (64, 8, 2, 0, 16, [5, 40], 16, False),              # chunk exactly one window long
    (256, 16, 4, 0, 32, [7, 500], 45, False),
    (256, 8, 2, 32, 16, [0, 90], 16, True),
]


@pytest.mark.parametrize("D,H,KVH,group,W,ctx,n,paged", CHUNK_CASES)
def test_chunk_recent(kvq, D, H, KVH, group, W, ctx, n, paged, monkeypatch):
    """Chunked prefill on a hybrid cache: the chunk goes in through
    kvq_append_recent (state checked against the oracle), then
    kvq_attention_chunk_recent against the oracle's causal chunk attention
    over each sequence's get_kv view, with the planner's splits and with
    short forced ones (splits holding INT8 and ring rows, and splits of ring
    rows only)."""
    import torch
    B = len(ctx)
    lens = [c + n for c in ctx]
    T = max(lens)
    log(f"chunk recent: D={D} H={H} KVH={KVH} group={group} W={W} ctx={ctx} n={n} paged={paged}")
    rng = np.random.default_rng(D * 7 + W + n + group + paged)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), "bf16")
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, n, D))
    refs = _oracle_states(x, ctx, W, group)
    cache, table = _new_cache(kvq, B, H, KVH, D, group, W, W + 5, paged, T, rng, lens)
    _write_state(cache, table, refs)
    rows = lambda a: np.ascontiguousarray(np.stack([a[b, :, c:c + n] for b, c in enumerate(ctx)]))
    ctx_dev = dev_tensor(np.asarray(ctx, np.int32))
    cache.append(kv_dev(rows(x["k_raw"])), kv_dev(rows(x["v_raw"])), ctx_dev)
    for b, ref in enumerate(refs):
        ref.append(x["k"][b, :, ctx[b]:lens[b]], x["v"][b, :, ctx[b]:lens[b]])
    _check_state(cache, table, refs, "chunk append")
    scale = 1.0 / np.sqrt(D)
    outs = []
    for split in ("0", "64"):
        monkeypatch.setenv("KVQ_SPLIT_LEN", split)
        out = cache.chunk(bf16_dev(qb), ctx_dev, True, scale, max(ctx))
        torch.cuda.synchronize()
        outs.append(to_host_bits(out))
    kh = np.zeros((B, KVH, T, D))
    vh = np.zeros((B, KVH, T, D))
    for b, ref in enumerate(refs):
        k, v = ref.kv()
        kh[b, :, :lens[b]], vh[b, :, :lens[b]] = k, v
    want = orc.attention_chunk(qv, kh, vh, ctx, True, scale)
    for o, split in zip(outs, ("default", "64")):
        assert np.all(np.isfinite(orc.bf16_bits_to_f32(o)))
        assert_attention_close(o, want, f"chunk recent, splits {split}")
