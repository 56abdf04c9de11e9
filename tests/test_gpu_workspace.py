"""The attention workspace contract: zero-filled once, every call returns it
to zero, so one workspace serves a run of calls of any entry point.

Split partials reach the merging workgroup as their own ready flags (a word
reads zero until its split has written it), so a word left nonzero by any
call would be taken for a finished split by the next.  These tests run
ragged batches with many splits (more than one merge round: over 128 splits
per sequence), the generic kernel's separate merge, the sliding window and
a recent-window chunk followed by decode on the same workspace, and check
both the results (against the fp64 oracle) and that the workspace reads all
zero after each call."""

import numpy as np
import pytest

import oracle as orc
import workloads as wl
from kvq_testlib import assert_attention_close, bf16_dev, dev_tensor, kv_dev, log, to_host_bits

pytestmark = pytest.mark.gpu


def _zero_after(ws, what):
    import torch
    torch.cuda.synchronize()
    nz = int(torch.count_nonzero(ws).item())
    assert nz == 0, f"{what}: {nz} workspace bytes left nonzero"


def _oracle_kv(x, group):
    kc, ks = orc.quantize(x["k"], group)
    vc, vs = orc.quantize(x["v"], group)
    return orc.dequantize_exact(kc, ks), orc.dequantize_exact(vc, vs)


@pytest.mark.parametrize("D,group,split", [(128, 0, "0"), (64, 32, "512"), (96, 0, "64")])
def test_decode_calls_leave_workspace_zero(kvq, monkeypatch, D, group, split):
    """Three decodes on one workspace with different length mixes (the
    splits, and so the merging workgroups, change between calls)."""
    import torch
    monkeypatch.setenv("KVQ_SPLIT_LEN", split)
    B, H, KVH, T = 3, 8, 2, 3000
    log(f"workspace: decode D={D} group={group} split={split}")
    x = wl.random_kv(41 + D + group, (B, KVH, T, D), "bf16")
    cache = kvq.Int8KVCache(B, H, KVH, D, max_len=T, group32=(group == 32), fill=0)
    cache.append(kv_dev(x["k_raw"]), kv_dev(x["v_raw"]), dev_tensor(np.zeros(B, np.int32)))
    kh, vh = _oracle_kv(x, group)
    ws = cache.workspace(T)
    scale = 1.0 / np.sqrt(D)
    for i, lens in enumerate(([3000, 1, 2049], [700, 3000, 1500], [1, 2, 2999])):
        qb, qv = wl.random_q(90 + i, (B, H, D))
        out = cache.decode(bf16_dev(qb), dev_tensor(np.asarray(lens, np.int32)), scale, T, workspace=ws)
        torch.cuda.synchronize()
        assert_attention_close(to_host_bits(out), orc.attention_decode(qv, kh, vh, lens, scale), f"call {i}")
        _zero_after(ws, f"decode call {i}")


def test_more_splits_than_one_merge_round(kvq, monkeypatch):
    """A sequence of 66000 tokens in 512-token splits: 129 partials per head,
    merged in two rounds of the merging workgroup's staging."""
    import torch
    monkeypatch.setenv("KVQ_SPLIT_LEN", "512")
    B, H, KVH, D, T = 1, 4, 1, 64, 66000
    log("workspace: 129 splits")
    x = wl.random_kv(77, (B, KVH, T, D), "bf16")
    cache = kvq.Int8KVCache(B, H, KVH, D, max_len=T, fill=0)
    cache.append(kv_dev(x["k_raw"]), kv_dev(x["v_raw"]), dev_tensor(np.zeros(B, np.int32)))
    kh, vh = _oracle_kv(x, 0)
    ws = cache.workspace(T)
    qb, qv = wl.random_q(78, (B, H, D))
    for lens in ([T], [T - 300]):
        out = cache.decode(bf16_dev(qb), dev_tensor(np.asarray(lens, np.int32)), 0.125, T, workspace=ws)
        torch.cuda.synchronize()
        assert_attention_close(to_host_bits(out), orc.attention_decode(qv, kh, vh, lens, 0.125), f"L={lens[0]}")
        _zero_after(ws, f"129-split decode L={lens[0]}")


def test_sliding_window_calls_leave_workspace_zero(kvq, monkeypatch):
    import torch
    monkeypatch.setenv("KVQ_SPLIT_LEN", "128")
    B, H, KVH, D, T, win = 2, 8, 2, 128, 1500, 700
    log("workspace: sliding window")
    x = wl.random_kv(55, (B, KVH, T, D), "bf16")
    cache = kvq.Int8KVCache(B, H, KVH, D, max_len=T, fill=0)
    cache.append(kv_dev(x["k_raw"]), kv_dev(x["v_raw"]), dev_tensor(np.zeros(B, np.int32)))
    kh, vh = _oracle_kv(x, 0)
    ws = cache.workspace(T, 1, win)
    for i, lens in enumerate(([1500, 650], [900, 1499])):
        qb, qv = wl.random_q(60 + i, (B, H, D))
        out = cache.decode(bf16_dev(qb), dev_tensor(np.asarray(lens, np.int32)), 0.09, T, workspace=ws, window=win)
        torch.cuda.synchronize()
        assert_attention_close(to_host_bits(out), orc.attention_decode(qv, kh, vh, lens, 0.09, window=win),
                               f"window call {i}")
        _zero_after(ws, f"window call {i}")


def test_recent_chunk_then_decode_share_a_workspace(kvq):
    """A recent-window cache: chunked prefill (at head dim 96 through the
    generic kernel, whose split partials use the workspace) and then a fused
    decode step, both on one workspace sized for the larger of the two."""
    import torch
    B, H, KVH, D, W = 2, 8, 2, 96, 16
    L0, n = 200, 24
    T = L0 + n + 1
    log("workspace: recent chunk then decode")
    x = wl.random_kv(31, (B, KVH, T, D), "bf16")
    cache = kvq.Int8KVCache(B, H, KVH, D, max_len=T, recent_window=W, fill=0)
    nb = max(kvq.kvq.kvq_workspace_size_chunk_recent(cache.desc, cache.recent, L0 + n, n),
             kvq.kvq.kvq_workspace_size_recent(cache.desc, cache.recent, T))
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    refs = [orc.RecentWindowCache(KVH, D, W) for _ in range(B)]
    part = lambda a, lo, hi: np.ascontiguousarray(a[:, :, lo:hi])
    cache.append(kv_dev(part(x["k_raw"], 0, L0)), kv_dev(part(x["v_raw"], 0, L0)), dev_tensor(np.zeros(B, np.int32)))
    ctx = np.full(B, L0, np.int32)
    cache.append(kv_dev(part(x["k_raw"], L0, L0 + n)), kv_dev(part(x["v_raw"], L0, L0 + n)), dev_tensor(ctx))
    for b in range(B):
        refs[b].append(x["k"][b, :, :L0], x["v"][b, :, :L0])
        refs[b].append(x["k"][b, :, L0:L0 + n], x["v"][b, :, L0:L0 + n])
    qb, qv = wl.random_q(32, (B, H, n, D))
    scale = 1.0 / np.sqrt(D)
    out = cache.chunk(bf16_dev(qb), dev_tensor(ctx), True, scale, L0, workspace=ws)
    torch.cuda.synchronize()
    kh = np.zeros((B, KVH, T, D))
    vh = np.zeros((B, KVH, T, D))
    for b, r in enumerate(refs):
        kh[b, :, :L0 + n], vh[b, :, :L0 + n] = r.kv()
    assert_attention_close(to_host_bits(out), orc.attention_chunk(qv, kh, vh, ctx, True, scale), "recent chunk")
    _zero_after(ws, "recent chunk")
    # one fused decode step on the same workspace
    lens = np.full(B, T, np.int32)
    for b in range(B):
        refs[b].append(x["k"][b, :, T - 1:T], x["v"][b, :, T - 1:T])
    qd, qdv = wl.random_q(33, (B, H, D))
    out = cache.append_decode(kv_dev(part(x["k_raw"], T - 1, T)), kv_dev(part(x["v_raw"], T - 1, T)), bf16_dev(qd),
                              dev_tensor(lens), scale, T, workspace=ws)
    torch.cuda.synchronize()
    assert_attention_close(to_host_bits(out), orc.attention_decode_recent(qdv, refs, scale), "recent decode")
    _zero_after(ws, "recent decode")
