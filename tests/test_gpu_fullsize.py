"""Parity at the full sizes of the decode workloads, in the launch
configuration the benchmark times (kvq_append_decode after a kvq_append
prefill, hint = the workload's maximum length): codes and scales bit-exact
against the oracle, attention outputs checked on sampled (sequence, head)
pairs that the oracle computes one by one, all outputs finite."""

import numpy as np
import pytest

import oracle as orc
import workloads as wl
from kvq_testlib import assert_attention_close, bf16_dev, dev_tensor, kv_dev, log, to_host_bits

pytestmark = pytest.mark.gpu


def _prefill_contiguous(kvq, w, x, chunk=1024):
    B, KVH, T, D = x["k"].shape
    cache = kvq.Int8KVCache(B, w.num_heads, KVH, D, max_len=w.max_len, group32=(w.group == 32))
    for p0 in range(0, w.ctx, chunk):
        n = min(chunk, w.ctx - p0)
        cache.append(kv_dev(np.ascontiguousarray(x["k_raw"][:, :, p0:p0 + n])),
                     kv_dev(np.ascontiguousarray(x["v_raw"][:, :, p0:p0 + n])),
                     dev_tensor(np.full(B, p0, np.int32)))
    return cache


def _sampled_decode_check(got, x, lens, kc, ks, vc, vs, num_heads, scale, picks, what):
    hpg = num_heads // kc.shape[1]
    ref = np.empty((len(picks), kc.shape[-1]))
    sel = np.empty((len(picks), kc.shape[-1]), np.uint16)
    for j, (b, h) in enumerate(picks):
        g = h // hpg
        L = int(lens[b])
        kh = orc.dequantize_exact(kc[b, g, :L], ks[b, g, :L])
        vh = orc.dequantize_exact(vc[b, g, :L], vs[b, g, :L])
        ref[j] = orc.softmax_attend(x["q"][b, h].astype(np.float64), kh, vh, scale, None)
        sel[j] = got[b, h]
    return assert_attention_close(sel, ref, what)


@pytest.mark.parametrize("name", ["decode_8b", "q8_group32", "decode_d256"])
def test_contiguous_decode_full_size(kvq, name):
    import torch
    w = wl.ALL[name]
    log(f"full size {name}: B={w.batch} H={w.num_heads} KVH={w.num_kv_heads} D={w.head_dim} "
        f"L={w.ctx + w.n_new} group={w.group}")
    x = wl.layer_inputs(w, 0)
    B, KVH, T, D = x["k"].shape
    cache = _prefill_contiguous(kvq, w, x)
    lens = np.full(B, T, np.int32)
    k_new = kv_dev(np.ascontiguousarray(x["k_raw"][:, :, w.ctx:]))
    v_new = kv_dev(np.ascontiguousarray(x["v_raw"][:, :, w.ctx:]))
    out = cache.append_decode(k_new, v_new, bf16_dev(x["q_bits"]), dev_tensor(lens), w.attn_scale, T)
    torch.cuda.synchronize()
    got = to_host_bits(out)
    kc, ks = orc.quantize(x["k"], w.group)
    vc, vs = orc.quantize(x["v"], w.group)
    assert np.array_equal(cache.k_codes.cpu().numpy(), kc), "K codes"
    assert np.array_equal(cache.v_codes.cpu().numpy(), vc), "V codes"
    assert np.array_equal(cache.k_scales.cpu().numpy().view(np.uint32), ks.view(np.uint32)), "K scales"
    assert np.array_equal(cache.v_scales.cpu().numpy().view(np.uint32), vs.view(np.uint32)), "V scales"
    assert np.all(np.isfinite(orc.bf16_bits_to_f32(got)))
    rng = np.random.default_rng(99)
    picks = [(int(rng.integers(B)), int(rng.integers(w.num_heads))) for _ in range(40)] + [(0, 0), (B - 1, w.num_heads - 1)]
    err, rel = _sampled_decode_check(got, x, lens, kc, ks, vc, vs, w.num_heads, w.attn_scale, picks, name)
    log(f"  sampled {len(picks)} rows: max abs err {err:.2e}, rel L2 {rel:.2e}")


def test_paged_decode_full_size(kvq):
    """64 sequences, lengths U[512, 32768], scattered pages: the sampled
    sequences carry the seeded host data; the others device random data (each
    sequence's output depends only on its own rows)."""
    import torch
    w = wl.PAGED
    lens, table, num_pages = wl.paged_layout(w)
    B, H, KVH, D = w.batch, w.num_heads, w.num_kv_heads, w.head_dim
    Lmax = int(lens.max())
    log(f"full size paged: B={B} lengths {int(lens.min())}..{Lmax}, {num_pages} pages")
    dev = torch.device("cuda")
    cache = kvq.Int8KVCache(B, H, KVH, D, num_pages=num_pages, block_table=dev_tensor(table))
    gen = torch.Generator(device=dev)
    gen.manual_seed(12345)
    zero = torch.zeros(B, dtype=torch.int32, device=dev)
    for p0 in range(0, Lmax, 2048):
        n = min(2048, Lmax - p0)
        k = torch.randn((B, KVH, n, D), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn((B, KVH, n, D), generator=gen, device=dev).to(torch.bfloat16)
        cache.append(k, v, zero + p0)
    # sampled sequences: shortest, longest, and three others, written through a
    # one-sequence descriptor over the same arena
    order = np.argsort(lens)
    sampled = sorted({int(order[0]), int(order[-1]), int(order[B // 3]), int(order[B // 2]), int(order[2 * B // 3])})
    xs = {}
    for b in sampled:
        L = int(lens[b])
        xs[b] = wl.sequence_kv(w, b, L)
        row = dev_tensor(np.ascontiguousarray(table[b:b + 1]))
        one = kvq.kvq.make_cache(1, H, KVH, D, cache.k_codes, cache.v_codes, cache.k_scales, cache.v_scales,
                                 layout=kvq.kvq.KVQ_LAYOUT_PAGED, num_pages=num_pages,
                                 max_blocks_per_seq=table.shape[1], block_table=row)
        kvq.kvq.kvq_append(one, kv_dev(xs[b]["k_raw"][None, :, :L - 1]), kv_dev(xs[b]["v_raw"][None, :, :L - 1]),
                           kvq.kvq.KVQ_DT_BF16, L - 1, dev_tensor(np.zeros(1, np.int32)))
        torch.cuda.synchronize()
        del row
    # the step: the last token of every sequence is appended by the attention launch
    k_new = torch.randn((B, KVH, 1, D), generator=gen, device=dev).to(torch.bfloat16)
    v_new = torch.randn((B, KVH, 1, D), generator=gen, device=dev).to(torch.bfloat16)
    for b in sampled:
        L = int(lens[b])
        k_new[b, :, 0] = kv_dev(np.ascontiguousarray(xs[b]["k_raw"][:, L - 1]))
        v_new[b, :, 0] = kv_dev(np.ascontiguousarray(xs[b]["v_raw"][:, L - 1]))
    q_bits, q = wl.paged_q(w)
    out = cache.append_decode(k_new, v_new, bf16_dev(q_bits), dev_tensor(lens), w.attn_scale, Lmax)
    torch.cuda.synchronize()
    got = to_host_bits(out)
    assert np.all(np.isfinite(orc.bf16_bits_to_f32(got)))
    kc_a = cache.k_codes.cpu().numpy()
    ks_a = cache.k_scales.cpu().numpy()
    vc_a = cache.v_codes.cpu().numpy()
    vs_a = cache.v_scales.cpu().numpy()
    hpg = H // KVH
    rng = np.random.default_rng(7)
    refs, sels = [], []
    for b in sampled:
        L = int(lens[b])
        kc, ks = orc.quantize(xs[b]["k"], 0)        # [KVH, L, D]
        vc, vs = orc.quantize(xs[b]["v"], 0)
        gk = orc.paged_gather(kc_a, table, b, L)    # [KVH, L, D]
        assert np.array_equal(gk, kc), f"K codes of sequence {b}"
        assert np.array_equal(orc.paged_gather(vc_a, table, b, L), vc), f"V codes of sequence {b}"
        assert np.array_equal(orc.paged_gather(ks_a, table, b, L).view(np.uint32), ks.view(np.uint32))
        assert np.array_equal(orc.paged_gather(vs_a, table, b, L).view(np.uint32), vs.view(np.uint32))
        for h in sorted({0, H - 1, int(rng.integers(H)), int(rng.integers(H))}):
            g = h // hpg
            refs.append(orc.softmax_attend(q[b, h].astype(np.float64), orc.dequantize_exact(kc[g], ks[g]),
                                           orc.dequantize_exact(vc[g], vs[g]), w.attn_scale, None))
            sels.append(got[b, h])
    err, rel = assert_attention_close(np.stack(sels), np.stack(refs), "paged full size")
    log(f"  sequences {sampled}: {len(refs)} rows, max abs err {err:.2e}, rel L2 {rel:.2e}")
