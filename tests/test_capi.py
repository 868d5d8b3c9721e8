"""The C-ABI library: it loads, exports every function include/pa.h declares,
and rejects bad arguments before launching anything (no GPU needed: every
call here fails its host-side checks)."""

import ctypes
import os
import re

import pytest

import paged_kv_cache_382_amd as pa
from paged_kv_cache_382_amd import probe as pa_probe

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "pa.h")
PROBE_HEADER = os.path.join(os.path.dirname(HEADER), "pa_probe.h")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("pa_store_kvcache", "pa_decode", "pa_copy_blocks",
                     "pa_decode_workspace_bytes", "pa_alloc_create", "pa_alloc_append_slot",
                     "pa_alloc_fork", "pa_alloc_free_seq", "pa_alloc_export"):
        assert required in names


def test_library_exports_every_declared_symbol():
    handle = ctypes.CDLL(pa.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(handle, n)]
    assert missing == []
    assert set(declared_functions()) == set(pa.SIGNATURES)


def test_probe_library_exports_its_header_and_stays_out_of_the_path():
    """The measurement probes are a library of their own (include/pa_probe.h);
    the attention library exports neither."""
    probe_names = declared_functions(PROBE_HEADER)
    assert probe_names == ["pa_mfma_probe", "pa_range_probe", "pa_read_probe"]
    handle = ctypes.CDLL(pa_probe.PROBE_LIB_PATH)
    assert all(hasattr(handle, n) for n in probe_names)
    assert set(probe_names) == set(pa_probe.SIGNATURES)
    attention = ctypes.CDLL(pa.LIB_PATH)
    assert not any(hasattr(attention, n) for n in probe_names)


@pytest.mark.parametrize("buf,nbytes,sink,code", [
    (0x1000, 24, 0x2000, "SHAPE"),                 # not a multiple of 16
    (None, 32, 0x2000, "NULL"),
    (0x1000, 32, None, "NULL"),
    (0x1008, 32, 0x2000, "ALIGN"),
    (0x1000, 32, 0x2002, "ALIGN"),
])
def test_read_probe_rejects_bad_arguments(buf, nbytes, sink, code):
    assert pa_probe.lib().pa_read_probe(buf, nbytes, sink, None) == NAMES[code]


def test_read_probe_of_nothing_launches_nothing():
    assert pa_probe.lib().pa_read_probe(None, 0, None, None) == 0


@pytest.mark.parametrize("sink,workgroups,iters,code", [
    (0x2000, -1, 8, "SHAPE"),
    (0x2000, 65537, 8, "SHAPE"),
    (0x2000, 4, 0, "SHAPE"),
    (0x2000, 4, 65537, "SHAPE"),
    (None, 4, 8, "NULL"),
    (0x2002, 4, 8, "ALIGN"),
])
def test_mfma_probe_rejects_bad_arguments(sink, workgroups, iters, code):
    assert pa_probe.lib().pa_mfma_probe(sink, workgroups, iters, 1.0, None) == NAMES[code]


def test_mfma_probe_of_no_workgroups_launches_nothing():
    assert pa_probe.lib().pa_mfma_probe(None, 0, 8, 1.0, None) == 0


def _offsets(*vals):
    return (ctypes.c_uint32 * len(vals))(*vals)


@pytest.mark.parametrize("buf,alloc,rng,soff,offs,n,out,code", [
    (0x1000, 4096, 4096, 0, (0,), 0, 0x2000, "SHAPE"),          # no lanes
    (0x1000, 4096, 4096, 0, (0,) * 65, 65, 0x2000, "SHAPE"),    # more than 64 lanes
    (None, 4096, 4096, 0, (0,), 1, 0x2000, "NULL"),
    (0x1000, 4096, 4096, 0, None, 1, 0x2000, "NULL"),
    (0x1000, 4096, 4096, 0, (0,), 1, None, "NULL"),
    (0x1008, 4096, 4096, 0, (0,), 1, 0x2000, "ALIGN"),          # buf not 16-byte aligned
    (0x1000, 4096, 4096, 2, (0,), 1, 0x2000, "ALIGN"),          # soffset not a multiple of 4
    (0x1000, 4096, 4096, 0, (6,), 1, 0x2000, "ALIGN"),          # voffset not a multiple of 4
    (0x1000, 4096, 4097, 0, (0,), 1, 0x2000, "RANGE"),          # range past the allocation
    (0x1000, 4096, 4096, 0, (4084,), 1, 0x2000, "RANGE"),       # a load could leave the allocation
    (0x1000, 4096, 4096, 16, (4072,), 1, 0x2000, "RANGE"),      # ... once soffset is added
])
def test_range_probe_rejects_bad_arguments(buf, alloc, rng, soff, offs, n, out, code):
    arr = _offsets(*offs) if offs is not None else None
    assert pa_probe.lib().pa_range_probe(buf, alloc, rng, soff, arr, n, out, None) == NAMES[code]


def _desc(nb=64, bs=16, hkv=4, d=64):
    return pa.CacheDesc(nb, bs, hkv, d)


def call_decode(desc=None, **kw):
    args = dict(q=0x1000, k=0x2000, v=0x3000, tables=0x4000, M=4, lens=0x5000, B=4, hq=4,
                max_ctx=33, scale=0.125, out=0x6000, split=0, ws=None, ws_bytes=0)
    args.update(kw)
    d = desc if desc is not None else _desc()
    return pa.lib().pa_decode(args["q"], args["k"], args["v"], ctypes.byref(d) if d else None,
                              args["tables"], args["M"], args["lens"], args["B"], args["hq"],
                              args["max_ctx"], args["scale"], args["out"], args["split"],
                              args["ws"], args["ws_bytes"], None)


NAMES = {v: k for k, v in pa.STATUS.items()}


@pytest.mark.parametrize("kw,desc,code", [
    (dict(q=None), None, "NULL"),
    (dict(out=None), None, "NULL"),
    (dict(q=0x1008), None, "ALIGN"),
    (dict(hq=6), None, "SHAPE"),                   # 6 % 4 != 0
    (dict(B=-1), None, "SHAPE"),
    (dict(M=0), None, "SHAPE"),
    (dict(), _desc(d=96), "UNSUPPORTED"),
    (dict(), _desc(bs=4), "UNSUPPORTED"),
    (dict(hq=12, split=16), None, "WORKSPACE"),    # group 3 is supported: it gets to the workspace check
    (dict(split=-2), None, "RANGE"),
    (dict(split=-1, B=65, ws=0x7000, ws_bytes=1 << 30), None, "RANGE"),   # whole pairs: <= 64 seqs
    (dict(split=(1 << 20) + 1), None, "RANGE"),
    (dict(split=16), None, "WORKSPACE"),
    (dict(split=16, ws=0x7000, ws_bytes=10), None, "WORKSPACE"),
    (dict(split=16, ws=0x7010, ws_bytes=1 << 20), None, "ALIGN"),
    (dict(), _desc(nb=0), "SHAPE"),
])
def test_decode_rejects_bad_arguments(kw, desc, code):
    assert call_decode(desc, **kw) == NAMES[code]
    assert pa.lib().pa_last_error().decode()


def test_decode_null_descriptor():
    assert pa.lib().pa_decode(0x1000, 0x2000, 0x3000, None, 0x4000, 4, 0x5000, 4, 4, 33, 0.1,
                              0x6000, 0, None, 0, None) == NAMES["NULL"]


def test_decode_zero_sequences_is_a_no_op():
    assert call_decode(B=0, q=None, out=None) == 0


def test_store_rejects_bad_arguments():
    d = _desc()
    f = pa.lib().pa_store_kvcache
    assert f(None, 0x2000, 0x3000, 4, 0x4000, 0x5000, ctypes.byref(d), None) == NAMES["NULL"]
    assert f(0x1004, 0x2000, 0x3000, 4, 0x4000, 0x5000, ctypes.byref(d), None) == NAMES["ALIGN"]
    assert f(0x1000, 0x2000, 0x3000, -1, 0x4000, 0x5000, ctypes.byref(d), None) == NAMES["SHAPE"]
    assert f(0x1000, 0x2000, 0x3000, 0, 0x4000, 0x5000, ctypes.byref(d), None) == 0
    bad = _desc(d=12)
    assert f(0x1000, 0x2000, 0x3000, 4, 0x4000, 0x5000, ctypes.byref(bad), None) == NAMES["UNSUPPORTED"]


def test_copy_blocks_rejects_bad_arguments():
    d = _desc()
    f = pa.lib().pa_copy_blocks
    assert f(None, 0x2000, ctypes.byref(d), 0x3000, 1, None) == NAMES["NULL"]
    assert f(0x1000, 0x2000, ctypes.byref(d), 0x3000, -1, None) == NAMES["SHAPE"]
    assert f(0x1000, 0x2000, ctypes.byref(d), None, 0, None) == 0


def test_workspace_and_split_queries():
    d = _desc(nb=8192, bs=16, hkv=8, d=128)
    assert pa.pa_decode_num_splits(d, 32, 512) == 512
    # head-group order (4 query heads a KV head on the matrix cores, 8 KV heads):
    # (4 x 512 splits + 4 sequences x 8 KV heads) slots x 4 heads x (2 + 128) floats
    assert pa.pa_decode_workspace_bytes(d, 4, 32, 512) == (4 * 512 + 32) * 4 * (2 + 128) * 4
    n = pa.pa_decode_num_splits(d, 32, 0)
    assert n > 0
    assert pa.pa_decode_workspace_bytes(d, 4, 32, 0) == (4 * n + 32) * 4 * (2 + 128) * 4
    # plain order: 2 KV heads (not a multiple of 4), or one query head a KV head
    d2 = _desc(nb=8192, bs=16, hkv=2, d=128)
    assert pa.pa_decode_workspace_bytes(d2, 4, 8, 512) == (512 + 8) * 4 * (2 + 128) * 4
    assert pa.pa_decode_workspace_bytes(d, 4, 8, 512) == 512 * 1 * (2 + 128) * 4 + 32 * 1 * (2 + 128) * 4
    # blocks of 8 tokens run on the vector kernel: plain order
    d3 = _desc(nb=8192, bs=8, hkv=8, d=128)
    assert pa.pa_decode_workspace_bytes(d3, 4, 32, 512) == (512 + 32) * 4 * (2 + 128) * 4
    assert pa.pa_decode_workspace_bytes(d, 4, 33, 0) == 0             # invalid -> 0
    assert pa.pa_decode_num_splits(d, 32, -3) == 0


def call_prefill(desc=None, **kw):
    args = dict(q=0x1000, k=0x2000, v=0x3000, tables=0x4000, M=4, lens=0x5000, starts=0x5800, B=2,
                T=8, hq=4, max_q=4, max_ctx=64, scale=0.125, out=0x6000)
    args.update(kw)
    d = desc if desc is not None else _desc()
    return pa.lib().pa_prefill(args["q"], args["k"], args["v"], ctypes.byref(d) if d else None,
                               args["tables"], args["M"], args["lens"], args["starts"], args["B"],
                               args["T"], args["hq"], args["max_q"], args["max_ctx"], args["scale"],
                               args["out"], None)


@pytest.mark.parametrize("kw,desc,code", [
    (dict(q=None), None, "NULL"),
    (dict(starts=None), None, "NULL"),
    (dict(out=0x6008), None, "ALIGN"),
    (dict(hq=6), None, "SHAPE"),
    (dict(T=-1), None, "SHAPE"),
    (dict(max_q=-1), None, "SHAPE"),
    (dict(M=0), None, "SHAPE"),
    (dict(scale=0.0), None, "RANGE"),
    (dict(scale=-0.5), None, "RANGE"),
    (dict(scale=float("nan")), None, "RANGE"),
    (dict(), _desc(d=96), "UNSUPPORTED"),
    (dict(), _desc(nb=0), "SHAPE"),
])
def test_prefill_rejects_bad_arguments(kw, desc, code):
    assert call_prefill(desc, **kw) == NAMES[code]
    assert pa.lib().pa_last_error().decode()


def test_prefill_empty_batch_is_a_no_op():
    assert call_prefill(B=0, q=None, out=None) == 0
    assert call_prefill(T=0, q=None, out=None) == 0


def test_prefill_rejects_block_sizes_that_are_not_powers_of_two():
    assert call_prefill(_desc(bs=12)) == NAMES["UNSUPPORTED"]
    assert call_prefill(_desc(bs=24)) == NAMES["UNSUPPORTED"]


def test_host_memory_exhaustion_is_a_status_not_an_abort(tmp_path):
    """Under a 1 GiB address-space cap, an allocator for 400 million blocks
    cannot be built: the call returns PA_ERR_HOST with a message instead of
    letting std::bad_alloc cross the C ABI (which would abort the process)."""
    import subprocess
    import sys
    script = tmp_path / "oom.py"
    script.write_text(
        "import ctypes, resource, sys\n"
        "resource.setrlimit(resource.RLIMIT_AS, (1 << 30, resource.RLIM_INFINITY))\n"
        "lib = ctypes.CDLL(sys.argv[1])\n"
        "lib.pa_last_error.restype = ctypes.c_char_p\n"
        "h = ctypes.c_void_p()\n"
        "rc = lib.pa_alloc_create(400_000_000, 4, 8, None, ctypes.byref(h))\n"
        "print(rc, lib.pa_last_error().decode())\n")
    res = subprocess.run([sys.executable, str(script), pa.LIB_PATH], capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 0, res.stderr[-2000:]
    rc, msg = res.stdout.strip().split(" ", 1)
    assert int(rc) == NAMES["HOST"]
    assert "out of host memory" in msg


@pytest.mark.parametrize("layout", [2, -1])
def test_unknown_cache_layout_is_rejected_before_any_launch(layout):
    d = pa.CacheDesc(64, 16, 4, 64, layout)
    assert call_decode(d) == NAMES["UNSUPPORTED"]
    assert call_prefill(d) == NAMES["UNSUPPORTED"]
    f = pa.lib().pa_store_kvcache
    assert f(0x1000, 0x2000, 0x3000, 4, 0x4000, 0x5000, ctypes.byref(d), None) == NAMES["UNSUPPORTED"]
    assert pa.lib().pa_copy_blocks(0x1000, 0x2000, ctypes.byref(d), 0x3000, 1, None) == NAMES["UNSUPPORTED"]
    assert "layout" in pa.lib().pa_last_error().decode()


def test_cache_desc_reads_the_shape_in_the_named_layout():
    class T:
        shape = (64, 4, 16, 128)       # head-major: [NB][Hkv][BS][D]
    d = pa.cache_desc(T, "head")
    assert (d.num_blocks, d.block_size, d.num_kv_heads, d.head_dim, d.layout) == (64, 16, 4, 128, 1)
    d = pa.cache_desc(T)               # slot-major reading of the same shape
    assert (d.num_blocks, d.block_size, d.num_kv_heads, d.head_dim, d.layout) == (64, 4, 16, 128, 0)
    with pytest.raises(ValueError):
        pa.cache_desc(T, "column")


def call_noalloc(desc=None, **kw):
    args = dict(q=0x1000, k=0x2000, v=0x3000, tables=0x4000, M=4, lens=0x5000, B=4, hq=4,
                max_ctx=33, scale=0.125, out=0x6000, split=0)
    args.update(kw)
    d = desc if desc is not None else _desc()
    return pa.lib().pa_decode_noalloc(args["q"], args["k"], args["v"], ctypes.byref(d) if d else None,
                                      args["tables"], args["M"], args["lens"], args["B"], args["hq"],
                                      args["max_ctx"], args["scale"], args["out"], args["split"], None)


@pytest.mark.parametrize("kw,desc,code", [
    (dict(q=None), None, "NULL"),
    (dict(q=0x1008), None, "ALIGN"),
    (dict(hq=6), None, "SHAPE"),
    (dict(), _desc(d=96), "UNSUPPORTED"),
    (dict(split=-2), None, "RANGE"),
    # 60000 splits of a 32-head group need more than the 8 MiB scratch
    (dict(hq=128, split=60000, max_ctx=1 << 20, M=1 << 16), None, "WORKSPACE"),
])
def test_noalloc_rejects_bad_arguments_before_any_device_call(kw, desc, code):
    """Every check (the scratch size included) runs before the scratch's
    device address is looked up, so it also works with no GPU present."""
    assert call_noalloc(desc, **kw) == NAMES[code]
    assert pa.lib().pa_last_error().decode()
