"""Torch-owned storage for one layer's INT8 KV cache, driven through libkvq.

PyTorch only allocates device memory and provides the stream; every step of
quantization, append, attention and dequantization runs in libkvq's kernels.
"""

from __future__ import annotations

import torch

from . import kvq as _k


def rolling_block_table(batch: int, max_len: int, window: int, chunk: int = 1):
    """Block table of a sliding-window layer's rolling store: a paged cache
    in which each sequence owns P = ceil((window + chunk - 1) / 16) pages and
    its logical page j is its physical page j mod P.  The row of position p
    then takes the slot of position p - 16 P, which no query of that append
    or any later one sees, so the store holds 16 P rows per sequence however
    long it grows (combs-models' sliding layers keep only the last w - 1).
    ``chunk`` is the most rows one append adds before attention; the
    attention calls take the window as usual.  Returns (int32 table
    [batch, ceil(max_len / 16)] on the host, pages)."""
    if window < 1 or chunk < 1 or max_len < 1:
        raise ValueError("window, chunk and max_len must be at least 1")
    per = -(-(window + chunk - 1) // 16)
    blocks = -(-max_len // 16)
    j = torch.arange(blocks, dtype=torch.int32)
    table = torch.stack([b * per + j % per for b in range(batch)])
    return table, batch * per


class Int8KVCache:
    """One layer's cache: u8 codes + fp32 scales, contiguous or paged.

    Contiguous: codes ``[B, KVH, max_len, D]``, scales ``[B, KVH, max_len, G]``.
    Paged: arena codes ``[P, KVH, 16, D]``, scales ``[P, KVH, 16, G]``, with a
    caller-provided int32 ``block_table [B, max_blocks_per_seq]``.
    ``fp8="e4m3"`` or ``"e5m2"`` stores FP8 codes instead, with no scales
    (``k_scales`` / ``v_scales`` are then None).  ``block_scales="head"`` or
    ``"channel"`` (with a recent window of at least 15) takes one scale per
    16-row block and KV head, or per block, KV head and element index:
    per-head scales are stored on every row (G = 1); per-channel scales are
    ``[B, KVH, max_len / 16, D]`` (paged: ``[P, KVH, D]``).
    """

    def __init__(self, batch: int, num_heads: int, num_kv_heads: int, head_dim: int, *,
                 max_len: int = 0, group32: bool = False, num_pages: int = 0,
                 block_table: torch.Tensor | None = None, device="cuda", fill: int | None = None,
                 recent_window: int = 0, recent_capacity: int | None = None, scale_bf16: bool = False,
                 fp8: str | None = None, block_scales: str | None = None):
        self.batch, self.num_heads, self.num_kv_heads, self.head_dim = batch, num_heads, num_kv_heads, head_dim
        self.groups = head_dim // 32 if group32 else 1
        self.paged = block_table is not None
        if self.paged:
            rows = (num_pages, num_kv_heads, 16)
            self.block_table = block_table.to(device=device, dtype=torch.int32).contiguous()
            self.max_blocks = self.block_table.shape[1]
            self.capacity = self.max_blocks * 16
        else:
            rows = (batch, num_kv_heads, max_len)
            self.block_table = None
            self.max_blocks = 0
            self.capacity = max_len
        shape_c = rows + (head_dim,)
        shape_s = rows + (self.groups,)
        if block_scales not in (None, "head", "channel"):
            raise ValueError("block_scales must be None, 'head' or 'channel'")
        if block_scales and (group32 or scale_bf16 or fp8):
            raise ValueError("block scales are fp32 INT8 scales of their own layout")
        if block_scales == "channel":
            shape_s = (num_pages, num_kv_heads, head_dim) if self.paged else (batch, num_kv_heads, max_len // 16, head_dim)
        if fill is None:
            self.k_codes = torch.empty(shape_c, dtype=torch.uint8, device=device)
            self.v_codes = torch.empty(shape_c, dtype=torch.uint8, device=device)
        else:
            self.k_codes = torch.full(shape_c, fill, dtype=torch.uint8, device=device)
            self.v_codes = torch.full(shape_c, fill, dtype=torch.uint8, device=device)
        if scale_bf16 and group32:
            raise ValueError("bf16-stored scales are per-token only")
        if fp8 not in (None, "e4m3", "e5m2"):
            raise ValueError("fp8 must be None, 'e4m3' or 'e5m2'")
        if fp8 and (scale_bf16 or group32):
            raise ValueError("FP8 codes carry no scales")
        self.fp8 = fp8
        if fp8:
            self.k_scales = self.v_scales = None
            mode = _k.KVQ_CODES_FP8_E4M3 if fp8 == "e4m3" else _k.KVQ_CODES_FP8_E5M2
        else:
            sdt = torch.bfloat16 if scale_bf16 else torch.float32
            self.k_scales = torch.zeros(shape_s, dtype=sdt, device=device)
            self.v_scales = torch.zeros(shape_s, dtype=sdt, device=device)
            mode = (_k.KVQ_SCALE_GROUP32 if group32 else
                    _k.KVQ_SCALE_PER_TOKEN_BF16 if scale_bf16 else
                    _k.KVQ_SCALE_BLOCK_HEAD if block_scales == "head" else
                    _k.KVQ_SCALE_BLOCK_CHANNEL if block_scales == "channel" else _k.KVQ_SCALE_PER_TOKEN)
        self.block_scales = block_scales
        self.desc = _k.make_cache(
            batch, num_heads, num_kv_heads, head_dim, self.k_codes, self.v_codes, self.k_scales,
            self.v_scales,
            layout=_k.KVQ_LAYOUT_PAGED if self.paged else _k.KVQ_LAYOUT_CONTIGUOUS,
            scale_mode=mode,
            max_len=0 if self.paged else max_len, num_pages=num_pages,
            max_blocks_per_seq=self.max_blocks, block_table=self.block_table)
        # recent-window hybrid: the last W positions of each sequence stay bf16
        # in a ring of R > W slots per (sequence, KV head)
        self.recent = None
        if recent_window > 0:
            cap = recent_capacity or recent_window + 1
            ring = (batch, num_kv_heads, cap, head_dim)
            self.k_recent = torch.zeros(ring, dtype=torch.bfloat16, device=device)
            self.v_recent = torch.zeros(ring, dtype=torch.bfloat16, device=device)
            self.recent = _k.make_recent(recent_window, cap, self.k_recent, self.v_recent)

    # -- entry points -----------------------------------------------------------
    def append(self, k_new: torch.Tensor, v_new: torch.Tensor, start_pos: torch.Tensor, stream=None):
        """k_new/v_new: [B, KVH, n, D] fp32 or bf16 on the device; start_pos int32 [B]."""
        dt = _k.KVQ_DT_BF16 if k_new.dtype == torch.bfloat16 else _k.KVQ_DT_F32
        if k_new.dtype not in (torch.float32, torch.bfloat16) or v_new.dtype != k_new.dtype:
            raise TypeError("k_new and v_new must both be float32 or both bfloat16")
        if not (k_new.is_contiguous() and v_new.is_contiguous()):
            raise ValueError("k_new and v_new must be contiguous")
        if self.recent is not None:
            _k.kvq_append_recent(self.desc, self.recent, k_new, v_new, dt, k_new.shape[2], start_pos, stream)
        else:
            _k.kvq_append(self.desc, k_new, v_new, dt, k_new.shape[2], start_pos, stream)

    def workspace(self, max_seq_len: int, n_query: int = 1, window: int = 0) -> torch.Tensor:
        """Zero-filled scratch for the attention calls (it must be zero before
        the first call; every call leaves it zero again)."""
        if window > 0:
            n = _k.kvq_workspace_size_window(self.desc, max_seq_len, n_query, window)
        elif self.recent is not None and n_query == 1:
            n = _k.kvq_workspace_size_recent(self.desc, self.recent, max_seq_len)
        elif self.recent is not None:  # a chunk of n_query queries
            n = _k.kvq_workspace_size_chunk_recent(self.desc, self.recent, max_seq_len, n_query)
        else:
            n = _k.kvq_workspace_size(self.desc, max_seq_len, n_query)
        return torch.zeros(max(n, 1), dtype=torch.uint8, device=self.k_codes.device)

    def decode(self, q: torch.Tensor, seq_lens: torch.Tensor, attn_scale: float, max_seq_len_hint: int,
               out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None,
               window: int = 0):
        """q: bf16 [B, H, D]; returns bf16 [B, H, D].  window > 0: sliding window."""
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            workspace = self.workspace(max_seq_len_hint, 1, window)
        if window > 0:
            if self.recent is not None:
                raise NotImplementedError("a sliding window over a recent-window cache is not provided")
            _k.kvq_attention_decode_window(self.desc, q, seq_lens, attn_scale, window, out, workspace,
                                           workspace.numel(), max_seq_len_hint, stream)
        elif self.recent is not None:
            _k.kvq_attention_decode_recent(self.desc, self.recent, q, seq_lens, attn_scale, out, workspace,
                                           workspace.numel(), max_seq_len_hint, stream)
        else:
            _k.kvq_attention_decode(self.desc, q, seq_lens, attn_scale, out, workspace, workspace.numel(),
                                    max_seq_len_hint, stream)
        return out

    def append_decode(self, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor, seq_lens: torch.Tensor,
                      attn_scale: float, max_seq_len_hint: int, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, stream=None, window: int = 0):
        """Append one K/V row per sequence at seq_lens - 1 and decode, in one launch."""
        if k_new.dtype not in (torch.float32, torch.bfloat16) or v_new.dtype != k_new.dtype:
            raise TypeError("k_new and v_new must both be float32 or both bfloat16")
        if not (k_new.is_contiguous() and v_new.is_contiguous()):
            raise ValueError("k_new and v_new must be contiguous")
        dt = _k.KVQ_DT_BF16 if k_new.dtype == torch.bfloat16 else _k.KVQ_DT_F32
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            workspace = self.workspace(max_seq_len_hint, 1, window)
        if window > 0:
            if self.recent is not None:
                raise NotImplementedError("a sliding window over a recent-window cache is not provided")
            _k.kvq_append_decode_window(self.desc, k_new, v_new, dt, q, seq_lens, attn_scale, window, out, workspace,
                                        workspace.numel(), max_seq_len_hint, stream)
        elif self.recent is not None:
            _k.kvq_append_decode_recent(self.desc, self.recent, k_new, v_new, dt, q, seq_lens, attn_scale, out,
                                        workspace, workspace.numel(), max_seq_len_hint, stream)
        else:
            _k.kvq_append_decode(self.desc, k_new, v_new, dt, q, seq_lens, attn_scale, out, workspace,
                                 workspace.numel(), max_seq_len_hint, stream)
        return out

    def chunk(self, q: torch.Tensor, ctx_lens: torch.Tensor, causal: bool, attn_scale: float,
              max_ctx_len_hint: int, out: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None, stream=None, window: int = 0):
        """q: bf16 [B, H, n, D]; returns bf16 [B, H, n, D].  window > 0:
        sliding window (implies causal)."""
        n = q.shape[2]
        if out is None:
            out = torch.empty_like(q)
        if self.recent is not None:
            if window > 0:
                raise NotImplementedError("a sliding window over a recent-window cache is not provided")
            if not causal:
                raise ValueError("chunked attention over a recent-window cache is causal")
            if workspace is None:
                nb = _k.kvq_workspace_size_chunk_recent(self.desc, self.recent, max_ctx_len_hint + n, n)
                workspace = torch.zeros(max(nb, 1), dtype=torch.uint8, device=self.k_codes.device)
            _k.kvq_attention_chunk_recent(self.desc, self.recent, q, n, ctx_lens, attn_scale, out, workspace,
                                          workspace.numel(), max_ctx_len_hint, stream)
            return out
        if workspace is None:
            workspace = self.workspace(max_ctx_len_hint + n, n, window)
        if window > 0:
            _k.kvq_attention_chunk_window(self.desc, q, n, ctx_lens, attn_scale, window, out, workspace,
                                          workspace.numel(), max_ctx_len_hint, stream)
        else:
            _k.kvq_attention_chunk(self.desc, q, n, ctx_lens, causal, attn_scale, out, workspace,
                                   workspace.numel(), max_ctx_len_hint, stream)
        return out

    def dequant(self, which: int, seq_lens: torch.Tensor, out_len: int, bf16: bool = False, stream=None):
        dt = torch.bfloat16 if bf16 else torch.float32
        out = torch.empty((self.batch, self.num_kv_heads, out_len, self.head_dim), dtype=dt,
                          device=self.k_codes.device)
        dt_code = _k.KVQ_DT_BF16 if bf16 else _k.KVQ_DT_F32
        if self.recent is not None:
            _k.kvq_dequant_recent(self.desc, self.recent, which, seq_lens, dt_code, out, out_len, stream)
        else:
            _k.kvq_dequant(self.desc, which, seq_lens, dt_code, out, out_len, stream)
        return out

    def nbytes(self) -> int:
        return _k.kvq_cache_bytes(self.desc)
