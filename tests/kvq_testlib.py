"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
library through its C ABI, and compare with the oracle at the stated bar."""

from __future__ import annotations

import sys

import numpy as np

import oracle as orc

# Attention tolerance (bf16 output): per element 1e-2 beyond bf16's own
# half-ulp rounding (2^-8 relative covers it), and relative L2 5e-3.
ATOL = 1e-2
RTOL = 2.0 ** -8
REL_L2 = 5e-3


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def dev_tensor(a: np.ndarray, dtype=None):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def bf16_dev(bits: np.ndarray):
    torch = torch_mod()
    return dev_tensor(bits.view(np.int16)).view(torch.bfloat16)


def kv_dev(raw: np.ndarray):
    """Device tensor for appended rows: fp32 array, or bf16 bit patterns."""
    torch = torch_mod()
    if raw.dtype == np.uint16:
        return dev_tensor(raw.view(np.int16)).view(torch.bfloat16)
    return dev_tensor(raw.astype(np.float32))


def to_host_bits(t) -> np.ndarray:
    torch = torch_mod()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_attention_close(gpu_bits: np.ndarray, ref: np.ndarray, what: str = ""):
    g = orc.bf16_bits_to_f32(gpu_bits).astype(np.float64)
    ref = np.asarray(ref, np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref)
    bound = ATOL + RTOL * np.abs(ref)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), f"{what}: |gpu-oracle| {err[worst]:.3e} > {bound[worst]:.3e} at {worst}"
    den = np.linalg.norm(ref)
    rel = np.linalg.norm(g - ref) / den if den > 0 else np.linalg.norm(g - ref)
    assert rel <= REL_L2, f"{what}: relative L2 {rel:.3e} > {REL_L2}"
    return float(np.max(err)), float(rel)


def oracle_cache_contiguous(k: np.ndarray, v: np.ndarray, group: int):
    """Oracle codes/scales of full K/V tensors [B, KVH, T, D] (fp32 values)."""
    kc, ks = orc.quantize(k, group)
    vc, vs = orc.quantize(v, group)
    return kc, ks, vc, vs


def random_block_table(rng: np.random.Generator, lens, page_size: int = 16, extra_pages: int = 3):
    """Scattered page assignment: a random permutation of all needed pages
    (plus unused spares), -1 padding past each sequence."""
    npg = [-(-int(L) // page_size) for L in lens]
    total = sum(npg) + extra_pages
    perm = rng.permutation(total).astype(np.int32)
    maxb = max(max(npg), 1)
    table = np.full((len(lens), maxb), -1, np.int32)
    off = 0
    for b, n in enumerate(npg):
        table[b, :n] = perm[off:off + n]
        off += n
    return table, total
