"""GPU checks of kvq_append_decode: it must equal kvq_append (start_pos =
seq_lens - 1) followed by kvq_attention_decode, bit for bit, and its codes
must equal the oracle's."""

import numpy as np
import pytest

import oracle as orc
import workloads as wl
from kvq_testlib import assert_attention_close, bf16_dev, dev_tensor, kv_dev, log, random_block_table, to_host_bits

pytestmark = pytest.mark.gpu

CASES = [
    # D, H, KVH, group, dtype, lens, paged
    (128, 32, 8, 0, "bf16", [1, 2, 64, 65, 511, 512, 513, 2048, 2049, 3000], False),
    (128, 32, 8, 32, "f32", [5, 300, 1024, 1025], False),
    (128, 32, 8, 0, "bf16", [17, 1000, 4096, 16], True),
    (64, 8, 2, 0, "f32", [1, 255, 256, 257], False),
    (64, 8, 2, 32, "bf16", [33, 700], True),
    (32, 4, 4, 0, "bf16", [3, 100], False),
    (256, 16, 4, 0, "bf16", [9, 600, 33, 32], False),
    (256, 8, 4, 32, "f32", [31, 1000], True),
    (128, 64, 8, 0, "bf16", [77, 1500], False),  # two workgroups per KV head
]


def _caches(kvq, B, H, KVH, D, group, T, paged, rng):
    if paged:
        table, npages = random_block_table(rng, [T] * B)
        mk = lambda: kvq.Int8KVCache(B, H, KVH, D, num_pages=npages, block_table=dev_tensor(table),
                                     group32=(group == 32), fill=0)
    else:
        mk = lambda: kvq.Int8KVCache(B, H, KVH, D, max_len=T, group32=(group == 32), fill=0)
    return mk(), mk()


@pytest.mark.parametrize("D,H,KVH,group,dtype,lens,paged", CASES)
def test_fused_equals_append_then_decode(kvq, D, H, KVH, group, dtype, lens, paged):
    import torch
    log(f"fused: D={D} H={H} KVH={KVH} group={group} dtype={dtype} lens={lens} paged={paged}")
    B, T = len(lens), max(lens)
    rng = np.random.default_rng(D + H + group + len(lens))
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), dtype)
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, D))
    a, f = _caches(kvq, B, H, KVH, D, group, T, paged, rng)
    lens_np = np.asarray(lens, np.int32)
    # both caches hold every token except the last of each sequence
    for c in (a, f):
        c.append(kv_dev(x["k_raw"]), kv_dev(x["v_raw"]), dev_tensor(np.zeros(B, np.int32)))
    # the new rows: token L-1 of each sequence, as [B, KVH, 1, D]
    idx = lens_np - 1
    k_new = np.ascontiguousarray(x["k_raw"][np.arange(B), :, idx][:, :, None, :])
    v_new = np.ascontiguousarray(x["v_raw"][np.arange(B), :, idx][:, :, None, :])
    # scramble the rows at L-1 in both caches so the new values must be written
    for c in (a, f):
        junk = wl.random_kv(7, (B, KVH, 1, D), dtype)
        c.append(kv_dev(junk["k_raw"]), kv_dev(junk["v_raw"]), dev_tensor(idx))
    lens_dev = dev_tensor(lens_np)
    q = bf16_dev(qb)
    scale = 1.0 / np.sqrt(D)
    a.append(kv_dev(k_new), kv_dev(v_new), dev_tensor(idx))
    out_a = a.decode(q, lens_dev, scale, T)
    out_f = f.append_decode(kv_dev(k_new), kv_dev(v_new), q, lens_dev, scale, T)
    torch.cuda.synchronize()
    for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
        assert torch.equal(getattr(a, name), getattr(f, name)), name
    ga, gf = to_host_bits(out_a), to_host_bits(out_f)
    assert np.array_equal(ga, gf)
    # and against the oracle
    kc, ks = orc.quantize(x["k"], group)
    vc, vs = orc.quantize(x["v"], group)
    ref = orc.attention_decode(qv, orc.dequantize_exact(kc, ks), orc.dequantize_exact(vc, vs), lens, scale)
    assert_attention_close(gf, ref, "fused")


def test_fused_zero_length(kvq):
    """seq_lens[b] = 0: no row is written and the output is zero."""
    import torch
    log("fused: zero length")
    B, H, KVH, D = 2, 8, 2, 128
    c = kvq.Int8KVCache(B, H, KVH, D, max_len=64, fill=0)
    x = wl.random_kv(3, (B, KVH, 1, D), "bf16")
    qb, _ = wl.random_q(4, (B, H, D))
    out = c.append_decode(kv_dev(x["k_raw"]), kv_dev(x["v_raw"]), bf16_dev(qb), dev_tensor(np.array([0, 5], np.int32)),
                          0.1, 64)
    torch.cuda.synchronize()
    assert np.all(to_host_bits(out)[0] == 0)
    kc = c.k_codes.cpu().numpy()
    assert np.all(kc[0] == 0)
    okc, _ = orc.quantize(x["k"], 0)
    assert np.array_equal(kc[1, :, 4], okc[1, :, 0])
