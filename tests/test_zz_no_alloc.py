"""GPU check of kvq_append_decode_noalloc, the fused decode step whose split
counters and partials live in the library's static per-GPU scratch array:
called through the C ABI, it must give exactly what kvq_append_decode gives
with a caller workspace (same kernels, same plan), on two calls in a row, the
second smaller than the first, and the oracle's result within the bar."""

import numpy as np
import pytest

import oracle as orc
import workloads as wl
from kvq_testlib import assert_attention_close, bf16_dev, dev_tensor, kv_dev, log, to_host_bits

pytestmark = pytest.mark.gpu

CALLS = [
    # B, H, KVH, D, group, dtype, lens: the 8B-shaped decode's shape first, then a smaller one
    (16, 32, 8, 128, 0, "bf16", [4096] * 16),
    (3, 8, 2, 64, 32, "f32", [700, 65, 1]),
]


def _one_call(kvq, B, H, KVH, D, group, dtype, lens, seed):
    import torch
    k = kvq.kvq
    T = max(lens)
    rng = np.random.default_rng(seed)
    x = wl.random_kv(int(rng.integers(1 << 30)), (B, KVH, T, D), dtype)
    qb, qv = wl.random_q(int(rng.integers(1 << 30)), (B, H, D))
    lens_np = np.asarray(lens, np.int32)
    ca = kvq.Int8KVCache(B, H, KVH, D, max_len=T, group32=(group == 32), fill=0)
    cb = kvq.Int8KVCache(B, H, KVH, D, max_len=T, group32=(group == 32), fill=0)
    for c in (ca, cb):  # every token but the last of each sequence
        c.append(kv_dev(x["k_raw"]), kv_dev(x["v_raw"]), dev_tensor(np.zeros(B, np.int32)))
    idx = np.maximum(lens_np - 1, 0)
    k_new = kv_dev(np.ascontiguousarray(x["k_raw"][np.arange(B), :, idx][:, :, None, :]))
    v_new = kv_dev(np.ascontiguousarray(x["v_raw"][np.arange(B), :, idx][:, :, None, :]))
    in_dt = k.KVQ_DT_BF16 if dtype == "bf16" else k.KVQ_DT_F32
    q = bf16_dev(qb)
    lens_dev = dev_tensor(lens_np)
    scale = 1.0 / np.sqrt(D)
    out_a = torch.empty_like(q)
    out_b = torch.full_like(q, float("nan"))
    ws_bytes = k.kvq_workspace_size(ca.desc, T, 1)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    k.kvq_append_decode(ca.desc, k_new, v_new, in_dt, q, lens_dev, scale, out_a, ws, ws_bytes, T)
    k.kvq_append_decode_noalloc(cb.desc, k_new, v_new, in_dt, q, lens_dev, scale, out_b, T)
    torch.cuda.synchronize()
    for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
        assert torch.equal(getattr(ca, name), getattr(cb, name)), name
    ga, gb = to_host_bits(out_a), to_host_bits(out_b)
    assert np.array_equal(ga, gb), "no-alloc output differs from the workspace entry point"
    kc, ks = orc.quantize(x["k"], group)
    vc, vs = orc.quantize(x["v"], group)
    ref = orc.attention_decode(qv, orc.dequantize_exact(kc, ks), orc.dequantize_exact(vc, vs), lens, scale)
    assert_attention_close(gb, ref, "noalloc")


def test_noalloc_equals_workspace_entry_point_two_calls(kvq):
    for i, (B, H, KVH, D, group, dtype, lens) in enumerate(CALLS):
        log(f"noalloc call {i}: B={B} H={H} KVH={KVH} D={D} group={group} dtype={dtype} lens={lens[:4]}")
        _one_call(kvq, B, H, KVH, D, group, dtype, lens, seed=100 + i)
