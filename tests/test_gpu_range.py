"""GPU parity at the edges of the kernels' f16 range, against the fp64 oracle.

The chunk kernel runs both products on f16 MFMA and the decode kernel takes
f16 dot products, with queries scaled by powers of two into f16 range and the
V scales carried in the weights' exponents.  These cases stress exactly that:
  * query heads of one chunk workgroup (the 4 query heads of a KV head) whose
    magnitudes are 2^20 and 2^30 apart; only the smallest head's scores are
    of order one (the others' queries are orthogonal to the keys), so a
    shared power of two that pushed the small head into f16 subnormals would
    flatten its softmax;
  * V rows of absmax about 1e-6 next to rows of about 1e4: attention spread
    over both, and attention concentrated on the tiny rows; with group-32
    scales the 32-element groups inside a row also differ by 1e4.
Each runs through chunked prefill and decode, per-token and group-32 scales.

The bar is reading 9's with its absolute term scaled to what enters each
output element: |gpu - oracle| <= 1e-2 * S + 2^-8 * |oracle|, where S is the
oracle's attention over |V-hat| (the attention-weighted magnitude of the
values; about 0.8 for unit-normal values).  Attention is linear in V, so
values scaled by c scale both the result and every rounding in it by c; a
fixed 1e-2 would ask for 20-bit weights when V is 1e4 and test nothing when V
is 1e-6.  Below fp32's normal range (2^-126) nothing is resolved: an output
made only of weights that small (e^-90 leakage) may come out as 0.  Relative
L2 stays at 5e-3.
"""

import numpy as np
import pytest

import oracle as orc
import workloads as wl
from kvq_testlib import REL_L2, RTOL, bf16_dev, dev_tensor, kv_dev, log, to_host_bits

pytestmark = pytest.mark.gpu

B, H, KVH, D = 2, 8, 2, 128
TINY = 2.0 ** -126  # below fp32's normal range results are not resolved (weights flush there)
CTX, N = [150, 37], 48


def _assert_scaled(gpu_bits, ref, scale_ref, what):
    g = orc.bf16_bits_to_f32(gpu_bits).astype(np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref)
    bound = 1e-2 * scale_ref + RTOL * np.abs(ref) + TINY
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), (f"{what}: |gpu-oracle| {err[worst]:.3e} > {bound[worst]:.3e} "
                                  f"(S {scale_ref[worst]:.3e}, ref {ref[worst]:.3e}) at {worst}")
    rel = np.linalg.norm(g - ref) / np.linalg.norm(ref)
    assert rel <= REL_L2, f"{what}: relative L2 {rel:.3e} > {REL_L2}"


def _run(kvq, x, qb_c, qv_c, qb_d, qv_d, group, what):
    import torch
    T = max(CTX) + N
    scale = 1.0 / np.sqrt(D)
    cache = kvq.Int8KVCache(B, H, KVH, D, max_len=T, group32=(group == 32), fill=0)
    cache.append(kv_dev(x["k"]), kv_dev(x["v"]), dev_tensor(np.zeros(B, np.int32)))
    kc, ks = orc.quantize(x["k"], group)
    vc, vs = orc.quantize(x["v"], group)
    kh, vh = orc.dequantize_exact(kc, ks), orc.dequantize_exact(vc, vs)
    # chunked prefill: queries at ctx + i, causal
    out = cache.chunk(bf16_dev(qb_c), dev_tensor(np.asarray(CTX, np.int32)), True, scale, max(CTX))
    torch.cuda.synchronize()
    ref = orc.attention_chunk(qv_c, kh, vh, CTX, True, scale)
    mag = orc.attention_chunk(qv_c, kh, np.abs(vh), CTX, True, scale)
    _assert_scaled(to_host_bits(out), ref, mag, f"{what} chunk")
    # decode over ctx + n tokens
    lens = np.asarray(CTX, np.int32) + N
    out = cache.decode(bf16_dev(qb_d), dev_tensor(lens), scale, int(lens.max()))
    torch.cuda.synchronize()
    ref = orc.attention_decode(qv_d, kh, vh, lens, scale)
    mag = orc.attention_decode(qv_d, kh, np.abs(vh), lens, scale)
    _assert_scaled(to_host_bits(out), ref, mag, f"{what} decode")


def _bf16(x):
    bits = wl.bf16_bits(x)
    return bits, wl.bits_to_f32(bits)


def _q_spread(e: int, seed: int, shape):
    """Queries of every KV group: head 0 is 2^e N(0,1) on dims 0..63, head 1
    is 2^-e N(0,1) on dims 64..127, heads 2 and 3 are N(0,1) on dims 0..63
    (other dims zero)."""
    rng = np.random.default_rng(seed)
    q = wl.normal(rng, shape)
    lo = np.arange(D) < D // 2
    heads = np.arange(H) % 4
    f = np.where(heads == 0, 2.0 ** e, np.where(heads == 1, 2.0 ** -e, 1.0)).astype(np.float32)
    mask = np.where(heads[:, None] == 1, ~lo[None, :], lo[None, :]).astype(np.float32)  # [H, D]
    hshape = (1, H) + (1,) * (len(shape) - 3) + (D,)
    q = q * f.reshape((1, H) + (1,) * (len(shape) - 2)) * mask.reshape(hshape)
    return _bf16(q)


@pytest.mark.parametrize("group", [0, 32])
@pytest.mark.parametrize("e", [20, 30])
def test_query_heads_far_apart(kvq, group, e):
    """Keys are zero on dims 0..63 and 2^e N(0,1) on dims 64..127: heads 0,
    2, 3 score 0 on every key, head 1 (2^-e) scores of order one."""
    log(f"range: query heads 2^+-{e}, group={group}")
    T = max(CTX) + N
    x = wl.random_kv(100 + e + group, (B, KVH, T, D), "f32")
    k = x["k"] * np.float32(2.0 ** e)
    k[..., : D // 2] = 0.0
    x = {"k": k.astype(np.float32), "v": x["v"]}
    qb_c, qv_c = _q_spread(e, 7 + e, (B, H, N, D))
    qb_d, qv_d = _q_spread(e, 8 + e, (B, H, D))
    _run(kvq, x, qb_c, qv_c, qb_d, qv_d, group, f"heads 2^+-{e}")


@pytest.mark.parametrize("group", [0, 32])
@pytest.mark.parametrize("focus", ["spread", "tiny"])
def test_value_rows_of_very_different_size(kvq, group, focus):
    """V rows of absmax about 1e4 (even tokens) and 1e-6 (odd tokens).
    spread: unit-normal keys and queries.  tiny: every query is +u and the
    keys are +4u on odd tokens and -4u on even ones (u a unit-normal
    direction), so the 1e-6 rows take nearly all the weight.  With group-32
    scales the odd 32-element groups of every row are also 1e-4 the size of
    the even ones."""
    log(f"range: V rows 1e-6 / 1e4, group={group}, focus={focus}")
    T = max(CTX) + N
    x = wl.random_kv(300 + group, (B, KVH, T, D), "f32")
    odd = (np.arange(T) % 2 == 1)[None, None, :, None]
    v = x["v"] * np.where(odd, 1e-6 / 4, 1e4 / 4).astype(np.float32)
    if group == 32:
        # odd groups of each row 1e-4 the size of its even groups (each
        # group's ratio to the row's largest enters an f16 weight; ratios
        # below about 2^-20 leave those weights in f16 subnormals)
        g_small = ((np.arange(D) // 32) % 2 == 1)[None, None, None, :]
        v = np.where(g_small, v * np.float32(1e-4), v).astype(np.float32)
    k = x["k"]
    if focus == "tiny":
        rng = np.random.default_rng(5 + group)
        u = wl.normal(rng, (D,))
        k = np.where(odd, 4.0 * u, -4.0 * u).astype(np.float32) * np.ones_like(k)
        qb_c, qv_c = _bf16(np.broadcast_to(u, (B, H, N, D)).astype(np.float32))
        qb_d, qv_d = _bf16(np.broadcast_to(u, (B, H, D)).astype(np.float32))
    else:
        qb_c, qv_c = wl.random_q(11, (B, H, N, D))
        qb_d, qv_d = wl.random_q(12, (B, H, D))
    x = {"k": k.astype(np.float32), "v": v.astype(np.float32)}
    _run(kvq, x, qb_c, qv_c, qb_d, qv_d, group, f"V 1e-6/1e4 {focus}")


@pytest.mark.parametrize("group", [0, 32])
def test_ring_rows_of_very_different_size(kvq, group):
    """Chunked prefill over a hybrid cache stages its ring rows (bf16) in the
    MFMA tiles as f16 with one power of two per row.  Ring rows alternate
    between V absmax about 1e-6 and 1e4, with unit-normal keys spreading
    attention over both; each row keeps its own power of two, so neither
    kind loses its bits.  Against the oracle's get_kv view, with the scaled bar."""
    import torch
    W, L0, n = 32, 150, 40
    T = L0 + n
    log(f"range: ring rows 1e-6 / 1e4, group={group}")
    x = wl.random_kv(400 + group, (B, KVH, T, D), "f32")
    odd = (np.arange(T) % 2 == 1)[None, None, :, None]
    mag = np.where(odd, 1e-6 / 4, 1e4 / 4).astype(np.float32)
    x = {"k": x["k"], "v": (x["v"] * mag).astype(np.float32)}
    cache = kvq.Int8KVCache(B, H, KVH, D, max_len=T, group32=(group == 32), fill=0, recent_window=W)
    cache.append(kv_dev(np.ascontiguousarray(x["k"][:, :, :L0])), kv_dev(np.ascontiguousarray(x["v"][:, :, :L0])),
                 dev_tensor(np.zeros(B, np.int32)))
    cache.append(kv_dev(np.ascontiguousarray(x["k"][:, :, L0:])), kv_dev(np.ascontiguousarray(x["v"][:, :, L0:])),
                 dev_tensor(np.full(B, L0, np.int32)))
    refs = []
    for b in range(B):
        r = orc.RecentWindowCache(KVH, D, W, group)
        r.append(x["k"][b, :, :L0], x["v"][b, :, :L0])
        r.append(x["k"][b, :, L0:], x["v"][b, :, L0:])
        refs.append(r)
    qb, qv = wl.random_q(13, (B, H, n, D))
    scale = 1.0 / np.sqrt(D)
    ctx = [L0] * B
    out = cache.chunk(bf16_dev(qb), dev_tensor(np.asarray(ctx, np.int32)), True, scale, L0)
    torch.cuda.synchronize()
    kh = np.stack([r.kv()[0] for r in refs])
    vh = np.stack([r.kv()[1] for r in refs])
    ref = orc.attention_chunk(qv, kh, vh, ctx, True, scale)
    mag_ref = orc.attention_chunk(qv, kh, np.abs(vh), ctx, True, scale)
    _assert_scaled(to_host_bits(out), ref, mag_ref, f"ring rows 1e-6/1e4 group={group}")
