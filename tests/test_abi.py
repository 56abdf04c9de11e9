"""C-ABI checks that need no GPU: exported symbols, struct layout, sizing and
every host-checkable error path (each returns before any HIP call)."""

import ctypes
import os
import re
import subprocess

import pytest

import oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

kvq = pytest.importorskip("int8_quantized_kv_amd.kvq")

FAKE = 0x10000  # never dereferenced: every case below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(kvq.EXPORTED)
    lib = kvq.library()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", kvq.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (kvq_[a-z_]+)", out))
    assert exported == set(names), exported ^ set(names)


@pytest.mark.parametrize("struct", ["kvq_cache", "kvq_recent"])
def test_struct_layout_matches_header(tmp_path, struct):
    """sizeof/offsetof of each descriptor from the C compiler equal the ctypes mirror."""
    mirror = getattr(kvq, struct)
    fields = [f for f, _ in mirror._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "kvq.h"\nint main(void){\n'
                   f'  printf("%zu\\n", sizeof({struct}));\n' +
                   "".join(f'  printf("%zu\\n", offsetof({struct}, {f}));\n' for f in fields) +
                   "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(mirror)
    for f, off in zip(fields, vals[1:]):
        assert getattr(mirror, f).offset == off, f


def _desc(**kw):
    base = dict(batch=2, num_heads=8, num_kv_heads=2, head_dim=128, max_len=64)
    base.update(kw)
    layout = base.pop("layout", kvq.KVQ_LAYOUT_CONTIGUOUS)
    scale = base.pop("scale_mode", kvq.KVQ_SCALE_PER_TOKEN)
    ptrs = base.pop("ptrs", (FAKE, FAKE, FAKE, FAKE))
    return kvq.make_cache(base.pop("batch"), base.pop("num_heads"), base.pop("num_kv_heads"),
                          base.pop("head_dim"), *ptrs, layout=layout, scale_mode=scale, **base)


def test_cache_bytes_pins_the_q8_sizing():
    """realizar kv_cache_q8_init.rs sizing: 32 layers x 8 KV heads x 128 dim x
    4096 positions with group-32 fp32 scales; batch 8 gives the printed
    "2.15 GB" of codes and 8.59 GB fp32-equivalent."""
    d = _desc(batch=8, num_heads=32, num_kv_heads=8, head_dim=128, max_len=4096,
              scale_mode=kvq.KVQ_SCALE_GROUP32)
    per_layer = kvq.kvq_cache_bytes(d)
    assert per_layer * 32 == orc.cache_bytes(8, 4096, 128, 32, batch=8, layers=32) == 2_415_919_104
    codes = 8 * 8 * 4096 * 128 * 2 * 32
    assert codes == orc.codes_bytes(8, 4096, 128, batch=8, layers=32) == 2_147_483_648
    assert per_layer * 32 - codes == 268_435_456
    d1 = _desc(batch=1, num_heads=32, num_kv_heads=8, head_dim=128, max_len=4096,
               scale_mode=kvq.KVQ_SCALE_GROUP32)
    assert kvq.kvq_cache_bytes(d1) * 32 == 301_989_888
    # per-token, paged
    dp = _desc(batch=4, num_heads=32, num_kv_heads=8, head_dim=128, max_len=0, layout=kvq.KVQ_LAYOUT_PAGED,
               num_pages=100, max_blocks_per_seq=10, block_table=FAKE)
    assert kvq.kvq_cache_bytes(dp) == 2 * 100 * 8 * 16 * (128 + 4)


def test_workspace_size_positive_and_monotone():
    d = _desc(batch=16, num_heads=32, num_kv_heads=8, head_dim=128, max_len=4096)
    a = kvq.kvq_workspace_size(d, 512, 1)
    b = kvq.kvq_workspace_size(d, 4096, 1)
    assert 0 < a <= b
    # at least one split's partials: (m, l) and D outputs per (sequence, head)
    assert b >= 16 * 32 * (128 + 2) * 4


def _status(fn, *args):
    lib = kvq.library()
    st = getattr(lib, fn)(*args)
    return st, kvq.kvq_last_error()


INVALID_DESCRIPTORS = [
    ("heads_not_multiple", dict(num_heads=6, num_kv_heads=4)),
    ("head_dim_not_32", dict(head_dim=48)),
    ("head_dim_too_big", dict(head_dim=288)),
    ("zero_batch", dict(batch=0)),
    ("bad_scale_mode", dict(scale_mode=7)),
    ("bad_layout", dict(layout=5)),
    ("contiguous_no_len", dict(max_len=0)),
    ("paged_page_size", dict(layout=kvq.KVQ_LAYOUT_PAGED, page_size=8, num_pages=4, max_blocks_per_seq=2,
                             block_table=FAKE)),
    ("paged_no_table", dict(layout=kvq.KVQ_LAYOUT_PAGED, num_pages=4, max_blocks_per_seq=2)),
    ("null_codes", dict(ptrs=(0, FAKE, FAKE, FAKE))),
    ("null_scales", dict(ptrs=(FAKE, FAKE, FAKE, 0))),
    # kernels read the aligned 32-bit word that holds a scale
    ("misaligned_scales", dict(scale_mode=kvq.KVQ_SCALE_PER_TOKEN_BF16, ptrs=(FAKE, FAKE, FAKE + 2, FAKE))),
]
# errors in device pointers only: the sizing calls, which read the geometry
# alone, accept these descriptors
POINTER_ONLY = {"paged_no_table", "null_codes", "null_scales", "misaligned_scales"}


@pytest.mark.parametrize("name,kw", INVALID_DESCRIPTORS, ids=[n for n, _ in INVALID_DESCRIPTORS])
def test_invalid_descriptor_rejected_everywhere(name, kw):
    d = ctypes.byref(_desc(**kw))
    calls = [
        ("kvq_append", (d, FAKE, FAKE, 0, 1, FAKE, None)),
        ("kvq_attention_decode", (d, FAKE, FAKE, 0.1, FAKE, FAKE, 1 << 30, 8, None)),
        ("kvq_attention_chunk", (d, FAKE, 4, FAKE, 1, 0.1, FAKE, FAKE, 1 << 30, 8, None)),
        ("kvq_dequant", (d, 0, FAKE, 0, FAKE, 8, None)),
    ]
    for fn, args in calls:
        st, msg = _status(fn, *args)
        assert st == kvq.KVQ_ERR_INVALID_ARG, (fn, st, msg)
        assert msg
    if name in POINTER_ONLY:
        assert kvq.library().kvq_cache_bytes(d) > 0
        assert kvq.library().kvq_workspace_size(d, 16, 1) > 0
    else:
        assert kvq.library().kvq_cache_bytes(d) == 0
        assert kvq.library().kvq_workspace_size(d, 16, 1) == 0


def test_null_descriptor():
    st, msg = _status("kvq_append", None, FAKE, FAKE, 0, 1, FAKE, None)
    assert st == kvq.KVQ_ERR_INVALID_ARG and "NULL" in msg


def test_append_argument_errors():
    d = ctypes.byref(_desc())
    assert _status("kvq_append", d, FAKE, FAKE, 0, 0, FAKE, None)[0] == kvq.KVQ_ERR_INVALID_ARG
    assert _status("kvq_append", d, FAKE, FAKE, 0, -3, FAKE, None)[0] == kvq.KVQ_ERR_INVALID_ARG
    assert _status("kvq_append", d, None, FAKE, 0, 1, FAKE, None)[0] == kvq.KVQ_ERR_INVALID_ARG
    assert _status("kvq_append", d, FAKE, FAKE, 0, 1, None, None)[0] == kvq.KVQ_ERR_INVALID_ARG
    assert _status("kvq_append", d, FAKE, FAKE, 9, 1, FAKE, None)[0] == kvq.KVQ_ERR_INVALID_ARG
    st, msg = _status("kvq_append", d, FAKE, FAKE, 0, 65, FAKE, None)
    assert st == kvq.KVQ_ERR_OUT_OF_RANGE and "capacity" in msg


def test_decode_argument_errors():
    d = ctypes.byref(_desc())
    ws = kvq.kvq_workspace_size(_desc(), 64, 1)
    assert _status("kvq_attention_decode", d, None, FAKE, 0.1, FAKE, FAKE, ws, 64, None)[0] == kvq.KVQ_ERR_INVALID_ARG
    assert _status("kvq_attention_decode", d, FAKE, FAKE, float("nan"), FAKE, FAKE, ws, 64, None)[0] == \
        kvq.KVQ_ERR_INVALID_ARG
    assert _status("kvq_attention_decode", d, FAKE, FAKE, 0.1, FAKE, FAKE, ws, 65, None)[0] == kvq.KVQ_ERR_OUT_OF_RANGE
    assert _status("kvq_attention_decode", d, FAKE, FAKE, 0.1, FAKE, FAKE, ws, 0, None)[0] == kvq.KVQ_ERR_OUT_OF_RANGE
    st, msg = _status("kvq_attention_decode", d, FAKE, FAKE, 0.1, FAKE, FAKE, ws - 1, 64, None)
    assert st == kvq.KVQ_ERR_WORKSPACE and "workspace" in msg
    assert _status("kvq_attention_decode", d, FAKE, FAKE, 0.1, FAKE, None, ws, 64, None)[0] == kvq.KVQ_ERR_WORKSPACE
    # head dims whose lane count is not a power of two run on the generic
    # kernel: sized like the others, refused only for a short workspace
    for d in (96, 160, 192, 224):
        dd = _desc(head_dim=d)
        need = kvq.kvq_workspace_size(dd, 64, 1)
        assert need > 0
        st, msg = _status("kvq_attention_decode", ctypes.byref(dd), FAKE, FAKE, 0.1, FAKE, FAKE, need - 1, 64, None)
        assert st == kvq.KVQ_ERR_WORKSPACE and f"the {need} bytes needed" in msg


def test_chunk_and_dequant_argument_errors():
    d = ctypes.byref(_desc())
    assert _status("kvq_attention_chunk", d, FAKE, 0, FAKE, 1, 0.1, FAKE, FAKE, 1 << 30, 8, None)[0] == \
        kvq.KVQ_ERR_INVALID_ARG
    assert _status("kvq_attention_chunk", d, FAKE, 8, FAKE, 1, 0.1, FAKE, FAKE, 1 << 30, 60, None)[0] == \
        kvq.KVQ_ERR_OUT_OF_RANGE
    assert _status("kvq_attention_chunk", d, None, 8, FAKE, 1, 0.1, FAKE, FAKE, 1 << 30, 8, None)[0] == \
        kvq.KVQ_ERR_INVALID_ARG
    assert _status("kvq_attention_chunk", d, FAKE, 8, FAKE, 1, float("nan"), FAKE, FAKE, 1 << 30, 8, None)[0] == \
        kvq.KVQ_ERR_INVALID_ARG
    # head sizes without an MFMA chunk kernel take chunks on the generic kernel
    d96 = _desc(head_dim=96)
    need = kvq.kvq_workspace_size(d96, 8 + 8, 8)
    assert need > 0
    st, msg = _status("kvq_attention_chunk", ctypes.byref(d96), FAKE, 8, FAKE, 1, 0.1, FAKE, FAKE, need - 1, 8, None)
    assert st == kvq.KVQ_ERR_WORKSPACE and f"the {need} bytes needed" in msg
    assert _status("kvq_dequant", d, 2, FAKE, 0, FAKE, 8, None)[0] == kvq.KVQ_ERR_INVALID_ARG
    assert _status("kvq_dequant", d, 0, FAKE, 3, FAKE, 8, None)[0] == kvq.KVQ_ERR_INVALID_ARG
    assert _status("kvq_dequant", d, 0, FAKE, 0, FAKE, 65, None)[0] == kvq.KVQ_ERR_OUT_OF_RANGE
    assert _status("kvq_dequant", d, 0, None, 0, FAKE, 8, None)[0] == kvq.KVQ_ERR_INVALID_ARG


def test_python_binding_raises():
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_append(_desc(head_dim=48), FAKE, FAKE, 0, 1, FAKE, stream=0)
    assert e.value.status == kvq.KVQ_ERR_INVALID_ARG


def _recent(window=4, capacity=5, k=FAKE, v=FAKE):
    return kvq.make_recent(window, capacity, k, v)


def test_recent_argument_errors():
    """A recent-window descriptor is checked before anything is enqueued."""
    d = ctypes.byref(_desc())
    ws = kvq.kvq_workspace_size_recent(_desc(), _recent(), 64)
    assert ws > kvq.kvq_workspace_size(_desc(), 64, 1) - 1
    for bad, word in ((None, "NULL"), (_recent(window=0), "window"), (_recent(capacity=4), "capacity"),
                      (_recent(k=None), "ring"), (_recent(v=None), "ring")):
        r = None if bad is None else ctypes.byref(bad)
        for name, args in (("kvq_append_recent", (FAKE, FAKE, 0, 1, FAKE, None)),
                           ("kvq_attention_decode_recent", (FAKE, FAKE, 0.1, FAKE, FAKE, 1 << 30, 64, None)),
                           ("kvq_append_decode_recent", (FAKE, FAKE, 0, FAKE, FAKE, 0.1, FAKE, FAKE, 1 << 30, 64,
                                                         None)),
                           ("kvq_dequant_recent", (0, FAKE, 0, FAKE, 8, None)),
                           ("kvq_attention_chunk_recent", (FAKE, 8, FAKE, 0.1, FAKE, FAKE, 1 << 30, 8, None))):
            st, msg = _status(name, d, r, *args)
            assert st == kvq.KVQ_ERR_INVALID_ARG and word in msg, (name, msg)
    r = ctypes.byref(_recent())
    assert _status("kvq_attention_decode_recent", d, r, FAKE, FAKE, 0.1, FAKE, FAKE, ws - 1, 64, None)[0] == \
        kvq.KVQ_ERR_WORKSPACE
    # head dim 96 runs on the generic kernel: sized like the others (the
    # calls are refused for a workspace one byte short, before any launch)
    d96 = _desc(head_dim=96)
    need = kvq.kvq_workspace_size_recent(d96, _recent(), 64)
    st, msg = _status("kvq_attention_decode_recent", ctypes.byref(d96), r, FAKE, FAKE, 0.1, FAKE, FAKE, need - 1, 64,
                      None)
    assert st == kvq.KVQ_ERR_WORKSPACE and f"the {need} bytes needed" in msg
    need = kvq.kvq_workspace_size_chunk_recent(d96, _recent(), 16, 8)
    st, msg = _status("kvq_attention_chunk_recent", ctypes.byref(d96), r, FAKE, 8, FAKE, 0.1, FAKE, FAKE, need - 1, 8,
                      None)
    assert st == kvq.KVQ_ERR_WORKSPACE and f"the {need} bytes needed" in msg
    assert _status("kvq_append_recent", d, r, FAKE, FAKE, 0, 65, FAKE, None)[0] == kvq.KVQ_ERR_OUT_OF_RANGE


def test_chunk_recent_workspace():
    """Chunks over a hybrid cache: at head dims 64 and 128 one MFMA launch
    with no workspace; elsewhere (and with per-channel block scales) one
    decode per (sequence, query), whose workspace holds partials for
    batch * n rows, any n including 1.  The descriptor is checked first."""
    r = _recent(window=16, capacity=17)
    for d in (64, 128):
        assert kvq.kvq_workspace_size_chunk_recent(_desc(head_dim=d), r, 64, 8) == 0
    for d in (32, 96, 256):
        one = kvq.kvq_workspace_size_chunk_recent(_desc(head_dim=d), r, 64, 1)
        eight = kvq.kvq_workspace_size_chunk_recent(_desc(head_dim=d), r, 64, 8)
        assert 0 < one < eight
    chan = _desc(scale_mode=kvq.KVQ_SCALE_BLOCK_CHANNEL, max_len=64)
    assert kvq.kvq_workspace_size_chunk_recent(chan, r, 64, 8) > 0
    with pytest.raises(kvq.KvqError, match="window"):
        kvq.kvq_workspace_size_chunk_recent(_desc(), _recent(window=0), 64, 8)
    with pytest.raises(kvq.KvqError, match="positive"):
        kvq.kvq_workspace_size_chunk_recent(_desc(), r, 64, 0)


def test_recent_workspace_is_the_int8_parts():
    """The ring adds no split of its own (the last INT8 split's workgroup
    attends to it): the workspace is that of the INT8 part, hint - W."""
    with_ring = kvq.kvq_workspace_size_recent(_desc(max_len=4096), _recent(window=128, capacity=129), 4096)
    assert with_ring > 0 and with_ring == kvq.kvq_workspace_size(_desc(max_len=4096), 4096 - 128, 1)


def test_window_argument_errors():
    """window < 1 is rejected by every sliding-window entry point."""
    d = ctypes.byref(_desc())
    for w in (0, -4):
        assert _status("kvq_attention_decode_window", d, FAKE, FAKE, 0.1, w, FAKE, FAKE, 1 << 30, 64, None)[0] == \
            kvq.KVQ_ERR_INVALID_ARG
        assert _status("kvq_append_decode_window", d, FAKE, FAKE, 0, FAKE, FAKE, 0.1, w, FAKE, FAKE, 1 << 30, 64,
                       None)[0] == kvq.KVQ_ERR_INVALID_ARG
        assert _status("kvq_attention_chunk_window", d, FAKE, 8, FAKE, 0.1, w, FAKE, FAKE, 1 << 30, 8, None)[0] == \
            kvq.KVQ_ERR_INVALID_ARG
        assert kvq.library().kvq_workspace_size_window(d, 64, 1, w) == 0
    # a window shorter than the hint plans fewer splits
    big = _desc(max_len=32768)
    assert 0 < kvq.kvq_workspace_size_window(big, 32768, 1, 256) < kvq.kvq_workspace_size(big, 32768, 1)


def test_bf16_scale_mode_sizing():
    """bf16-stored per-token scales take 2 bytes per row."""
    d = _desc(scale_mode=kvq.KVQ_SCALE_PER_TOKEN_BF16, max_len=4096)
    assert kvq.kvq_cache_bytes(d) == 2 * 2 * 2 * 4096 * (128 + 2)
    assert kvq.kvq_cache_bytes(_desc(max_len=4096)) == 2 * 2 * 2 * 4096 * (128 + 4)
    assert _status("kvq_cache_bytes", ctypes.byref(_desc(scale_mode=-1)))[0] == 0


def test_fp8_descriptors_need_no_scales():
    """FP8 codes (llama-gguf kv_quantized.rs): scale pointers may be NULL and
    the cache holds the code bytes alone (the page's memory_usage counts
    scales for Int8 only); a recent window is reported as unsupported
    before anything is launched."""
    for mode in (kvq.KVQ_CODES_FP8_E4M3, kvq.KVQ_CODES_FP8_E5M2):
        d = _desc(scale_mode=mode, max_len=4096, ptrs=(FAKE, FAKE, 0, 0))
        assert kvq.kvq_cache_bytes(d) == 2 * 2 * 2 * 4096 * 128
        assert kvq.kvq_cache_bytes(d) == orc.codes_bytes(2, 4096, 128, batch=2)
        r = kvq.make_recent(4, 5, FAKE, FAKE)
        st, msg = _status("kvq_append_recent", ctypes.byref(d), ctypes.byref(r), FAKE, FAKE, 0, 1, FAKE, None)
        assert st == kvq.KVQ_ERR_UNSUPPORTED, msg
    assert _status("kvq_cache_bytes", ctypes.byref(_desc(scale_mode=7)))[0] == 0


def test_sizing_before_allocation():
    """A descriptor with no device pointers yet sizes the cache it describes
    (the same figures as with pointers) and its decode workspace."""
    for mode in (kvq.KVQ_SCALE_PER_TOKEN, kvq.KVQ_SCALE_GROUP32, kvq.KVQ_CODES_FP8_E4M3):
        bare = _desc(scale_mode=mode, max_len=512, ptrs=(0, 0, 0, 0))
        full = _desc(scale_mode=mode, max_len=512)
        assert kvq.kvq_cache_bytes(bare) == kvq.kvq_cache_bytes(full) > 0
        assert kvq.library().kvq_workspace_size(ctypes.byref(bare), 512, 1) == \
            kvq.library().kvq_workspace_size(ctypes.byref(full), 512, 1) > 0
    paged = _desc(layout=kvq.KVQ_LAYOUT_PAGED, num_pages=10, max_blocks_per_seq=4, ptrs=(0, 0, 0, 0))
    assert kvq.kvq_cache_bytes(paged) == 2 * 10 * 2 * 16 * (128 + 4)
    # the entry points that touch memory still require the pointers
    st, msg = _status("kvq_append", ctypes.byref(paged), FAKE, FAKE, 0, 1, FAKE, None)
    assert st == kvq.KVQ_ERR_INVALID_ARG and "block_table" in msg


def test_noalloc_host_errors():
    """kvq_append_decode_noalloc checks its arguments and the scratch size on
    the host, before any launch."""
    d = ctypes.byref(_desc())
    F = ctypes.c_float
    assert _status("kvq_append_decode_noalloc", d, None, FAKE, 1, FAKE, FAKE, F(0.1), FAKE, 64, None)[0] == \
        kvq.KVQ_ERR_INVALID_ARG
    assert _status("kvq_append_decode_noalloc", d, FAKE, FAKE, 7, FAKE, FAKE, F(0.1), FAKE, 64, None)[0] == \
        kvq.KVQ_ERR_INVALID_ARG
    assert _status("kvq_append_decode_noalloc", d, FAKE, FAKE, 1, FAKE, FAKE, F(0.1), FAKE, 65, None)[0] == \
        kvq.KVQ_ERR_OUT_OF_RANGE
    # 512 sequences x 64 heads x 2 splits x 130 floats of partials: above the 8 MiB array
    big = ctypes.byref(kvq.make_cache(512, 64, 8, 128, FAKE, FAKE, FAKE, FAKE, max_len=4096))
    st, msg = _status("kvq_append_decode_noalloc", big, FAKE, FAKE, 1, FAKE, FAKE, F(0.1), FAKE, 4096, None)
    assert st == kvq.KVQ_ERR_WORKSPACE and "maximum" in msg


@pytest.mark.parametrize("head_dim", [32, 96])
def test_one_query_chunk_workspace_is_enough(head_dim):
    """kvq_workspace_size(cache, hint + 1, 1) covers a one-query chunk at head
    dims that run chunks on the generic kernel (whose splits are shorter than
    decode's): one byte less is refused as exactly that many bytes short."""
    c = kvq.make_cache(4, 32, 8, head_dim, FAKE, FAKE, FAKE, FAKE, max_len=8192)
    ws = kvq.kvq_workspace_size(c, 4096 + 1, 1)
    st, msg = _status("kvq_attention_chunk", ctypes.byref(c), FAKE, 1, FAKE, 1, ctypes.c_float(0.1), FAKE, FAKE,
                      ws - 1, 4096, None)
    assert st == kvq.KVQ_ERR_WORKSPACE and f"the {ws} bytes needed" in msg


def test_block_scale_descriptors():
    """Per-head and per-channel block scales (abaddon QuantGranularity over
    16-row blocks): the byte count (per head: one fp32 scale per row; per
    channel: head_dim scales per 16 rows), max_len a multiple of 16, a window
    of at least 15, and the entry points without a recent window refusing
    the modes before anything is launched."""
    head = _desc(scale_mode=kvq.KVQ_SCALE_BLOCK_HEAD, max_len=4096)
    chan = _desc(scale_mode=kvq.KVQ_SCALE_BLOCK_CHANNEL, max_len=4096)
    rows = 2 * 2 * 4096
    assert kvq.kvq_cache_bytes(head) == 2 * rows * (128 + 4)
    assert kvq.kvq_cache_bytes(chan) == 2 * (rows * 128 + (rows // 16) * 128 * 4)
    for mode in (kvq.KVQ_SCALE_BLOCK_HEAD, kvq.KVQ_SCALE_BLOCK_CHANNEL):
        bad = _desc(scale_mode=mode, max_len=100)
        with pytest.raises(kvq.KvqError, match="16"):
            kvq.kvq_cache_bytes(bad)
        d = _desc(scale_mode=mode, max_len=4096)
        st, msg = _status("kvq_append", ctypes.byref(d), FAKE, FAKE, 0, 1, FAKE, None)
        assert st == kvq.KVQ_ERR_UNSUPPORTED and "recent" in msg, msg
        st, msg = _status("kvq_attention_decode", ctypes.byref(d), FAKE, FAKE, ctypes.c_float(0.1), FAKE, FAKE,
                          ctypes.c_size_t(1 << 20), 64, None)
        assert st == kvq.KVQ_ERR_UNSUPPORTED, msg
        st, msg = _status("kvq_attention_chunk", ctypes.byref(d), FAKE, 4, FAKE, 1, ctypes.c_float(0.1), FAKE,
                          FAKE, ctypes.c_size_t(1 << 20), 64, None)
        assert st == kvq.KVQ_ERR_UNSUPPORTED, msg
        st, msg = _status("kvq_append_decode_noalloc", ctypes.byref(d), FAKE, FAKE, 0, FAKE, FAKE,
                          ctypes.c_float(0.1), FAKE, 64, None)
        assert st == kvq.KVQ_ERR_UNSUPPORTED, msg
        with pytest.raises(kvq.KvqError, match="recent"):
            kvq.kvq_workspace_size(d, 64, 1)
        short = kvq.make_recent(14, 20, FAKE, FAKE)
        st, msg = _status("kvq_append_recent", ctypes.byref(d), ctypes.byref(short), FAKE, FAKE, 0, 1, FAKE, None)
        assert st == kvq.KVQ_ERR_INVALID_ARG and "15" in msg, msg
        ok = kvq.make_recent(15, 16, FAKE, FAKE)
        assert kvq.kvq_workspace_size_recent(d, ok, 4096) > 0
        # per-head blocks chunk on the MFMA kernel (no workspace), per-channel on the generic one
        got = kvq.kvq_workspace_size_chunk_recent(d, ok, 4096, 64)
        assert got == 0 if mode == kvq.KVQ_SCALE_BLOCK_HEAD else got > 0


def test_stream_read_flag_errors():
    # bits 0 (interleave) and 1 (non-temporal) are the only flags; the rest is
    # refused before anything reaches the device
    for flags in (4, 8, -1):
        st, msg = _status("kvq_stream_read", FAKE, 1 << 20, FAKE, 256, 8, 2, flags, None)
        assert st == kvq.KVQ_ERR_INVALID_ARG and "interleave" in msg, (flags, st, msg)
    assert _status("kvq_stream_read", FAKE, 1 << 20, FAKE, 256, 8, 3, 1, None)[0] == kvq.KVQ_ERR_INVALID_ARG


def _plan_bytes(batch, heads, groups, splits, head_dim):
    """Workspace of a decode plan: the splits' ticket counters (one per
    (sequence, head group), 256-byte aligned), then (m, l) and D outputs per
    (sequence, head, split)."""
    def up(x):
        return (x + 255) // 256 * 256
    partials = batch * heads * splits
    return up(groups * 4) + up(partials * 2 * 4) + partials * head_dim * 4


def test_split_planner_rules():
    # one round: the 8B-shaped decode, four heads per workgroup, two splits of
    # 2048 tokens (128 head groups x 2 = 256 workgroups)
    d = _desc(batch=16, num_heads=32, num_kv_heads=8, head_dim=128, max_len=4096)
    assert kvq.kvq_workspace_size(d, 4096, 1) == _plan_bytes(16, 32, 128, 2, 128)
    # several rounds: about two rounds of the longest length, at most 32768
    # tokens a split -- the paged workload's 64 sequences up to 31912 tokens
    # take one split each (512 workgroups), a uniform 16 x 32768 batch four
    # splits of 8192
    dp = _desc(batch=64, num_heads=32, num_kv_heads=8, head_dim=128, max_len=0, layout=kvq.KVQ_LAYOUT_PAGED,
               num_pages=70000, max_blocks_per_seq=2048, block_table=FAKE)
    assert kvq.kvq_workspace_size(dp, 31912, 1) == _plan_bytes(64, 32, 512, 1, 128)
    dl = _desc(batch=16, num_heads=32, num_kv_heads=8, head_dim=128, max_len=32768)
    assert kvq.kvq_workspace_size(dl, 32768, 1) == _plan_bytes(16, 32, 128, 4, 128)
    # a one-round plan that would leave half the compute units idle halves the
    # heads per workgroup when the KV heads are a multiple of 8: the sliding
    # decode (16 x 8 KV heads, 1024-token window) runs 256 workgroups of two
    # heads, one split each
    dw = _desc(batch=16, num_heads=32, num_kv_heads=8, head_dim=128, max_len=8192)
    assert kvq.kvq_workspace_size_window(dw, 8192, 1, 1024) == _plan_bytes(16, 32, 256, 1, 128)
    # ... but not with 2 KV heads (the tiny decode keeps four heads, one split)
    dt = _desc(batch=1, num_heads=8, num_kv_heads=2, head_dim=64, max_len=256)
    assert kvq.kvq_workspace_size(dt, 256, 1) == _plan_bytes(1, 8, 2, 1, 64)
