"""GPU parity of kvq_append (codes and scales bit-exact with the oracle) and
kvq_dequant (bit-exact fp32 and bf16)."""

import numpy as np
import pytest

import oracle as orc
import workloads as wl
from kvq_testlib import bf16_dev, dev_tensor, kv_dev, log, random_block_table, to_host_bits

pytestmark = pytest.mark.gpu


def _contiguous_roundtrip(kvq, k_raw, v_raw, k_vals, v_vals, group, chunks, max_len=None):
    import torch
    B, KVH, T, D = k_vals.shape
    max_len = T if max_len is None else max_len
    cache = kvq.Int8KVCache(B, KVH, KVH, D, max_len=max_len, group32=(group == 32), fill=0)
    pos = 0
    for n in chunks:
        start = dev_tensor(np.full(B, pos, np.int32))
        cache.append(kv_dev(k_raw[:, :, pos:pos + n]), kv_dev(v_raw[:, :, pos:pos + n]), start)
        pos += n
    torch.cuda.synchronize()
    kc, ks, vc, vs = (cache.k_codes.cpu().numpy(), cache.k_scales.cpu().numpy(),
                      cache.v_codes.cpu().numpy(), cache.v_scales.cpu().numpy())
    okc, oks = orc.quantize(k_vals, group)
    ovc, ovs = orc.quantize(v_vals, group)
    assert np.array_equal(kc[:, :, :T], okc), np.argwhere(kc[:, :, :T] != okc)[:5]
    assert np.array_equal(vc[:, :, :T], ovc)
    assert np.array_equal(ks[:, :, :T].view(np.uint32), oks.view(np.uint32))
    assert np.array_equal(vs[:, :, :T].view(np.uint32), ovs.view(np.uint32))
    return cache


def test_tiny_workload_append_bit_exact(kvq):
    log("append: tiny workload fp32 [1,2,256,64] per-token")
    x = wl.tiny_inputs()
    _contiguous_roundtrip(kvq, x["k_raw"], x["v_raw"], x["k"], x["v"], 0, [100, 100, 55, 1])


@pytest.mark.parametrize("D", [32, 64, 96, 128, 160, 256])
@pytest.mark.parametrize("group", [0, 32])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_append_shapes_bit_exact(kvq, D, group, dtype):
    log(f"append: D={D} group={group} dtype={dtype}")
    x = wl.random_kv(1000 + D + group, (3, 2, 37, D), dtype, scale=3.0)
    _contiguous_roundtrip(kvq, x["k_raw"], x["v_raw"], x["k"], x["v"], group, [16, 1, 20], max_len=40)


@pytest.mark.parametrize("group", [0, 32])
def test_exhaustive_bf16_patterns(kvq, group):
    """Every finite bf16 bit pattern as x in rows [x, A, 0, ...] for several
    companions A, both scale modes: codes and scales bit-exact."""
    import torch
    log(f"append: exhaustive bf16 patterns group={group}")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    xs = bits[finite]
    D = 64
    for A in (1.0, 3.0e-3, 250.0, 1.0e-30, 0.0):
        rows = np.zeros((xs.size, D), np.uint16)
        rows[:, 0] = xs
        rows[:, 1] = wl.bf16_bits(np.float32([A]))[0]
        rows[:, 40] = xs[::-1]                 # a second group sees patterns too
        k_raw = rows.reshape(1, 1, xs.size, D)
        vals = wl.bits_to_f32(k_raw)
        cache = kvq.Int8KVCache(1, 1, 1, D, max_len=xs.size, group32=(group == 32), fill=0)
        start = dev_tensor(np.zeros(1, np.int32))
        t = kv_dev(k_raw)
        cache.append(t, t, start)
        torch.cuda.synchronize()
        oc, os_ = orc.quantize(vals, group)
        assert np.array_equal(cache.k_codes.cpu().numpy(), oc), A
        assert np.array_equal(cache.k_scales.cpu().numpy().view(np.uint32), os_.view(np.uint32)), A


def test_special_rows(kvq):
    """All-zero rows, constant rows, denormal rows, exact ties."""
    log("append: special rows")
    D = 64
    rows = np.zeros((6, D), np.float32)
    rows[1] = 5.0                                  # constant: codes 255
    rows[2] = -7.0                                 # constant negative: codes 1
    rows[3, :] = np.float32(1e-40) * np.arange(D)  # denormals
    rows[4, 0] = 63.5                              # s = 0.5: exact ties
    rows[4, 1:9] = [0.25, -0.25, 0.75, -0.75, 1.25, -1.25, 2.25, -2.25]
    rows[5, 0] = 381.0                             # s = 3
    rows[5, 1:] = np.float32((np.arange(D - 1) + 0.5) * 3)
    x = rows.reshape(1, 1, 6, D)
    for group in (0, 32):
        _contiguous_roundtrip(kvq, x, x, x, x, group, [6])


def test_paged_append_bit_exact_and_unmapped_rows_untouched(kvq):
    import torch
    log("append: paged scattered table, ragged chunks")
    rng = np.random.default_rng(5)
    B, KVH, D = 3, 2, 128
    lens = [40, 17, 33]
    table, npages = random_block_table(rng, lens)
    x = wl.random_kv(77, (B, KVH, 40, D), "bf16")
    cache = kvq.Int8KVCache(B, 8, KVH, D, num_pages=npages, block_table=dev_tensor(table), fill=0)
    pos = np.zeros(B, np.int32)
    for n in (5, 11, 1, 23):
        start = dev_tensor(pos.copy())
        cache.append(kv_dev(np.ascontiguousarray(x["k_raw"][:, :, pos[0]:pos[0] + n])),
                     kv_dev(np.ascontiguousarray(x["v_raw"][:, :, pos[0]:pos[0] + n])), start)
        pos += n
    torch.cuda.synchronize()
    arena = cache.k_codes.cpu().numpy()
    okc, oks = orc.quantize(x["k"], 0)
    for b in range(B):
        npg = -(-lens[b] // 16)
        L = min(40, table.shape[1] * 16)
        for t in range(L):
            page = t // 16
            if page >= table.shape[1] or table[b, page] < 0:
                continue
            assert np.array_equal(arena[table[b, page], :, t % 16], okc[b, :, t]), (b, t)
        # pages past the sequence are -1: those positions must not have been written
        assert npg <= table.shape[1]
    used = set(table[table >= 0].tolist())
    for p in range(npages):
        if p not in used:
            assert np.all(arena[p] == 0), p


def test_out_of_capacity_positions_skipped(kvq):
    import torch
    log("append: positions beyond capacity are not written")
    D = 64
    x = wl.random_kv(3, (2, 1, 4, D), "f32")
    cache = kvq.Int8KVCache(2, 1, 1, D, max_len=6, fill=0)
    start = dev_tensor(np.array([4, -2], np.int32))    # rows 6,7 and -2,-1 are outside
    cache.append(kv_dev(x["k_raw"]), kv_dev(x["v_raw"]), start)
    torch.cuda.synchronize()
    kc = cache.k_codes.cpu().numpy()
    okc, _ = orc.quantize(x["k"], 0)
    assert np.array_equal(kc[0, 0, 4:6], okc[0, 0, 0:2])
    assert np.all(kc[0, 0, :4] == 0)
    assert np.array_equal(kc[1, 0, 0:2], okc[1, 0, 2:4])
    assert np.all(kc[1, 0, 2:] == 0)


@pytest.mark.parametrize("group", [0, 32])
@pytest.mark.parametrize("paged", [False, True])
def test_dequant_bit_exact(kvq, group, paged):
    import torch
    log(f"dequant: group={group} paged={paged}")
    rng = np.random.default_rng(9)
    B, KVH, D, T = 2, 2, 128, 45
    lens = np.array([45, 30], np.int32)
    x = wl.random_kv(99, (B, KVH, T, D), "bf16", scale=2.0)
    if paged:
        table, npages = random_block_table(rng, [T, T])
        cache = kvq.Int8KVCache(B, 8, KVH, D, num_pages=npages, block_table=dev_tensor(table),
                                group32=(group == 32), fill=0)
    else:
        cache = kvq.Int8KVCache(B, 8, KVH, D, max_len=48, group32=(group == 32), fill=0)
    cache.append(kv_dev(x["k_raw"]), kv_dev(x["v_raw"]), dev_tensor(np.zeros(B, np.int32)))
    dl = dev_tensor(lens)
    for which, vals in ((0, x["k"]), (1, x["v"])):
        c, s = orc.quantize(vals, group)
        out32 = cache.dequant(which, dl, 46).cpu().numpy()
        out16 = to_host_bits(cache.dequant(which, dl, 46, bf16=True))
        torch.cuda.synchronize()
        ref32 = orc.dequantize_f32(c, s)
        ref16 = orc.dequantize_bf16_bits(c, s)
        for b in range(B):
            L = lens[b]
            assert np.array_equal(out32[b, :, :L].view(np.uint32), ref32[b, :, :L].view(np.uint32))
            assert np.array_equal(out16[b, :, :L], ref16[b, :, :L])
            assert np.all(out32[b, :, L:] == 0) and np.all(out16[b, :, L:] == 0)
