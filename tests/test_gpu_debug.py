"""The KVQ_DEBUG build of the C ABI layer: before each attention launch it
checks, on the host, the device-side values the kernels otherwise take on
trust (lengths within their bound, every page a call reads mapped to an arena
page) and refuses the call with KVQ_ERR_OUT_OF_RANGE.  Valid calls give the
release build's output bit for bit (the same kernels).  A refused call
launches nothing, so no case here reaches the device with a bad page id.
"""

import ctypes
import os

import pytest
import torch

import int8_quantized_kv_amd as kvq
from int8_quantized_kv_amd import kvq as _k

pytestmark = pytest.mark.gpu

DBG = os.path.join(os.path.dirname(os.path.abspath(kvq.__file__)), "_dbg", "libkvq.so")
B, H, KVH, D, P, MB = 2, 8, 2, 128, 16, 6   # batch, heads, KV heads, head dim, arena pages, table row


@pytest.fixture(scope="module")
def dbg():
    if not os.path.exists(DBG):
        pytest.skip("debug library not built (python int8_quantized_kv_amd/build.py --debug)")
    return _k.load_library(DBG)


def paged_cache(table):
    bt = torch.tensor(table, dtype=torch.int32)
    c = kvq.Int8KVCache(B, H, KVH, D, num_pages=P, block_table=bt, fill=0)
    g = torch.Generator(device="cuda").manual_seed(11)
    c.k_codes.random_(0, 256, generator=g)
    c.v_codes.random_(0, 256, generator=g)
    c.k_scales.uniform_(0.001, 0.01, generator=g)
    c.v_scales.uniform_(0.001, 0.01, generator=g)
    return c


def good_table():
    return [[3, 7, 1, 12, -1, -1], [0, 9, 4, 15, 2, -1]]


def decode_debug(lib, c, q, lens, hint, window=0):
    out = torch.zeros_like(q)
    ws = c.workspace(hint, 1, window)
    stream = torch.cuda.current_stream().cuda_stream
    if window > 0:
        st = lib.kvq_attention_decode_window(ctypes.byref(c.desc), q.data_ptr(), lens.data_ptr(), 0.088, window,
                                             out.data_ptr(), ws.data_ptr(), ws.numel(), hint, stream)
    else:
        st = lib.kvq_attention_decode(ctypes.byref(c.desc), q.data_ptr(), lens.data_ptr(), 0.088, out.data_ptr(),
                                      ws.data_ptr(), ws.numel(), hint, stream)
    torch.cuda.synchronize()
    return st, lib.kvq_last_error().decode(), out


def inputs(lens):
    g = torch.Generator(device="cuda").manual_seed(5)
    q = torch.randn(B, H, D, device="cuda", generator=g).to(torch.bfloat16)
    return q, torch.tensor(lens, dtype=torch.int32, device="cuda")


def test_valid_calls_match_the_release_build(dbg):
    c = paged_cache(good_table())
    q, lens = inputs([61, 80])
    st, msg, out = decode_debug(dbg, c, q, lens, 80)
    assert st == _k.KVQ_OK, msg
    ref = c.decode(q, lens, 0.088, 80)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    # a sliding window reads only the pages it sees: an unmapped page below it is fine
    t = good_table()
    t[1][0] = -1
    c2 = paged_cache(t)
    st, msg, out = decode_debug(dbg, c2, q, lens, 80, window=40)
    assert st == _k.KVQ_OK, msg
    ref = c2.decode(q, lens, 0.088, 80, window=40)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("bad_id", [16, 99, -1])
def test_page_outside_the_arena_is_refused(dbg, bad_id):
    t = good_table()
    t[1][2] = bad_id                     # positions 32..47 of sequence 1
    c = paged_cache(t)
    q, lens = inputs([61, 80])
    st, msg, _ = decode_debug(dbg, c, q, lens, 80)
    assert st == _k.KVQ_ERR_OUT_OF_RANGE and f"page {bad_id}" in msg and "sequence 1" in msg, (st, msg)
    # a shorter sequence 1 does not read that page
    q, lens = inputs([61, 32])
    st, msg, _ = decode_debug(dbg, c, q, lens, 80)
    assert st == _k.KVQ_OK, msg


def test_length_past_the_hint_is_refused(dbg):
    c = paged_cache(good_table())
    q, lens = inputs([81, 10])
    st, msg, _ = decode_debug(dbg, c, q, lens, 80)
    assert st == _k.KVQ_ERR_OUT_OF_RANGE and "sequence 0" in msg and "length 81" in msg, (st, msg)
    q, lens = inputs([-3, 10])
    st, msg, _ = decode_debug(dbg, c, q, lens, 80)
    assert st == _k.KVQ_ERR_OUT_OF_RANGE and "sequence 0" in msg, (st, msg)


def test_window_page_inside_the_window_is_refused(dbg):
    t = good_table()
    t[1][3] = -1                          # positions 48..63, inside the window of the last 40 of 80
    c = paged_cache(t)
    q, lens = inputs([61, 80])
    st, msg, _ = decode_debug(dbg, c, q, lens, 80, window=40)
    assert st == _k.KVQ_ERR_OUT_OF_RANGE and "page -1" in msg, (st, msg)


def test_chunk_reads_through_its_new_rows(dbg):
    # a chunk of n = 8 queries after a context of 60: positions 0..67 are read,
    # so sequence 0's fifth page (positions 64..79) must be mapped
    c = paged_cache(good_table())
    n, hint = 8, 70
    g = torch.Generator(device="cuda").manual_seed(6)
    q = torch.randn(B, H, n, D, device="cuda", generator=g).to(torch.bfloat16)
    out = torch.zeros_like(q)
    ctx = torch.tensor([60, 40], dtype=torch.int32, device="cuda")
    ws = c.workspace(hint + n, n)
    st = dbg.kvq_attention_chunk(ctypes.byref(c.desc), q.data_ptr(), n, ctx.data_ptr(), 1, 0.088, out.data_ptr(),
                                 ws.data_ptr(), ws.numel(), hint, torch.cuda.current_stream().cuda_stream)
    msg = dbg.kvq_last_error().decode()
    assert st == _k.KVQ_ERR_OUT_OF_RANGE and "sequence 0" in msg and "page -1" in msg, (st, msg)
