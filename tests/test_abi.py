"""Host-only checks of the C ABI: the library loads, exports every function the header
declares, the descriptor layout matches the C compiler's, and invalid arguments are
rejected before anything is enqueued (no GPU is touched)."""
import ctypes as C
import os
import re
import subprocess
import tempfile

import pytest

from decode_attention_kvq_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from decode_attention_kvq_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(r"\bT %s$" % n, out, re.M), n


def test_descriptor_layout_matches_c():
    src = r"""
    #include <stddef.h>
    #include <stdio.h>
    #include "kvq.h"
    int main(void) {
      printf("%zu %zu %zu %zu %zu\n", sizeof(kvq_cache_desc), offsetof(kvq_cache_desc, p_lo),
             offsetof(kvq_cache_desc, num_pages), offsetof(kvq_cache_desc, k_pages),
             offsetof(kvq_cache_desc, v_pages));
      return 0;
    }"""
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "l.c")
        exe = os.path.join(d, "l")
        open(c, "w").write(src)
        subprocess.check_call(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), c, "-o", exe])
        got = subprocess.check_output([exe]).decode().split()
    D = _lib.KvqCacheDesc
    assert [int(x) for x in got] == [C.sizeof(D), D.p_lo.offset, D.num_pages.offset,
                                      D.k_pages.offset, D.v_pages.offset]


def _desc(**kw):
    d = dict(num_kv_heads=8, head_dim=128, page_size=64, bits_k=2, bits_v=2, quant_k=0, quant_v=0,
             p_lo=0.01, p_hi=0.99, alpha_k=2.83, alpha_v=2.83, num_pages=4, k_pages=0x1000,
             v_pages=0x2000)
    d.update(kw)
    return _lib.KvqCacheDesc(**d)


def test_block_bytes_and_status_strings(lib):
    assert lib.kvq_block_bytes(2) == 2304 and lib.kvq_block_bytes(4) == 4352
    assert lib.kvq_block_bytes(3) == 3328 and lib.kvq_block_bytes(5) == 0
    assert lib.kvq_status_string(-3) == b"workspace too small"


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), -2), (dict(page_size=32), -2), (dict(bits_k=5), -2), (dict(bits_v=8), -2),
    (dict(num_kv_heads=0), -1), (dict(p_lo=0.5, p_hi=0.4), -1), (dict(p_hi=1.5), -1),
    (dict(quant_k=1, alpha_k=0.0), -1), (dict(quant_v=7), -1), (dict(k_pages=0), -1),
])
def test_append_rejects_bad_descriptor(lib, kw, status):
    d = _desc(**kw)
    p = C.c_void_p(0x10)
    rc = lib.kvq_quantize_append(C.byref(d), p, p, 1, 5, p, None, 1, None)
    assert rc == status, lib.kvq_last_error()
    assert lib.kvq_last_error()


def test_append_argument_checks(lib):
    d = _desc()
    p = C.c_void_p(0x10)
    assert lib.kvq_quantize_append(C.byref(d), p, p, 1, -1, p, None, 1, None) == -1
    assert lib.kvq_quantize_append(C.byref(d), None, p, 1, 5, p, None, 1, None) == -1
    assert lib.kvq_quantize_append(C.byref(d), p, p, 9, 5, p, None, 1, None) == -1
    assert lib.kvq_quantize_append(C.byref(d), p, p, 1, 5, p, p, 0, None) == -2   # T dtype mismatch
    assert lib.kvq_quantize_append(C.byref(d), p, p, 1, 0, p, None, 1, None) == 0  # nothing to do
    assert lib.kvq_quantize_append(None, p, p, 1, 5, p, None, 1, None) == -1


def test_decode_argument_checks(lib):
    d = _desc()
    p = C.c_void_p(0x10)
    call = lambda **kw: lib.kvq_decode_attn(
        C.byref(kw.get("d", d)), kw.get("q", p), kw.get("qd", 1), kw.get("B", 2), kw.get("Hq", 32),
        None, kw.get("bt", p), kw.get("mp", 4), kw.get("sl", p), kw.get("msl", 256),
        kw.get("scale", 0.088), kw.get("out", p), kw.get("ws", None), kw.get("wsb", 0), None)
    assert call(Hq=30) == -1                    # not a multiple of the KV heads
    assert call(Hq=8 * 17) == -2                # more than 16 query heads per KV head
    assert call(mp=3) == -1                     # block table too short for max_seq_len
    assert call(B=-1) == -1
    assert call(B=0) == 0
    assert call(q=None) == -1
    assert call(qd=5) == -1
    assert call(scale=float("inf")) == -1
    # one long sequence is split over several workgroups: partial results need a workspace
    need = lib.kvq_decode_workspace_bytes(C.byref(d), 1, 32, 16384)
    assert need >= 32 * 2 * 130 * 4
    assert call(B=1, mp=256, msl=16384) == -3  # workspace missing
    assert call(B=1, mp=256, msl=16384, ws=p, wsb=need - 1) == -3
    assert lib.kvq_decode_workspace_bytes(C.byref(d), 0, 32, 0) == 0
    # many sequences fill the GPU without splitting: no workspace
    assert lib.kvq_decode_workspace_bytes(C.byref(d), 64, 32, 16384) == 0
    assert lib.kvq_decode_workspace_bytes(C.byref(d), 1, 32, 0) == 0
    # the step's append runs in the decode's own launch: its workspace is the decode's, split
    # or not
    for (b, hq, msl) in ((1, 32, 16384), (1, 64, 16384), (16, 64, 131072), (3, 8, 5000),
                         (64, 32, 16384), (3, 8, 100), (600, 8, 200000)):
        assert lib.kvq_decode_step_workspace_bytes(C.byref(d), b, hq, msl) == \
            lib.kvq_decode_workspace_bytes(C.byref(d), b, hq, msl)
    assert lib.kvq_decode_workspace_bytes(C.byref(d), 1, 32, 16384) > 0          # split
    assert lib.kvq_decode_step_workspace_bytes(C.byref(d), 0, 32, 16) == 0
    assert lib.kvq_decode_step_workspace_bytes(C.byref(d), 1, 31, 16) == 0      # not a multiple of the KV heads
    assert lib.kvq_decode_step_workspace_bytes(None, 1, 32, 16) == 0
    d0 = _desc(num_pages=0)
    assert call(d=d0) == -1                                                   # empty pool


def test_dequant_argument_checks(lib):
    d = _desc()
    p = C.c_void_p(0x10)
    assert lib.kvq_dequant(C.byref(d), 2, p, 5, p, None) == -1
    assert lib.kvq_dequant(C.byref(d), 0, None, 5, p, None) == -1
    assert lib.kvq_dequant(C.byref(d), 0, p, 0, p, None) == 0


def test_decode_step_argument_checks(lib):
    d = _desc()
    p = C.c_void_p(0x10)

    def call(**kw):
        return lib.kvq_decode_step(
            C.byref(kw.get("d", d)), kw.get("q", p), kw.get("k", p), kw.get("v", p), kw.get("dt", 1),
            kw.get("B", 2), kw.get("Hq", 32), kw.get("slots", p), kw.get("t", None), kw.get("tdt", 1), None,
            kw.get("bt", p), kw.get("mp", 4), kw.get("sl", p), kw.get("msl", 256), kw.get("scale", 0.088),
            kw.get("out", p), kw.get("ws", None), kw.get("wsb", 0), None)
    assert call(Hq=30) == -1                    # decode checks apply
    assert call(mp=3) == -1
    assert call(B=0) == 0
    assert call(k=None) == -1                   # the new tokens are required
    assert call(slots=None) == -1
    assert call(t=p, tdt=0) == -2               # transform dtype differs from the inputs
    assert call(d=_desc(p_lo=0.7, p_hi=0.2)) == -1
    assert call(d=_desc(quant_k=1, alpha_k=-1.0)) == -1
    assert call(B=1, mp=256, msl=16384) == -3   # split launch without a workspace


def test_window_descriptor_layout_matches_c():
    src = r"""
    #include <stddef.h>
    #include <stdio.h>
    #include "kvq.h"
    int main(void) {
      printf("%zu %zu %zu %zu %zu %d\n", sizeof(kvq_window_desc), offsetof(kvq_window_desc, num_rows),
             offsetof(kvq_window_desc, dtype), offsetof(kvq_window_desc, k_win),
             offsetof(kvq_window_desc, v_win), (int)KVQ_WINDOW_MAX_SLOTS);
      return 0;
    }"""
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "w.c")
        exe = os.path.join(d, "w")
        open(c, "w").write(src)
        subprocess.check_call(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), c, "-o", exe])
        got = subprocess.check_output([exe]).decode().split()
    W = _lib.KvqWindowDesc
    assert [int(x) for x in got] == [C.sizeof(W), W.num_rows.offset, W.dtype.offset, W.k_win.offset,
                                      W.v_win.offset, 65535]


def _win(**kw):
    w = dict(sink=4, keep=16, flush=16, num_rows=2, dtype=1, k_win=0x3000, v_win=0x4000)
    w.update(kw)
    return _lib.KvqWindowDesc(**w)


def test_window_sizes(lib):
    d = _desc()
    assert lib.kvq_window_bytes(C.byref(d), C.byref(_win())) == 2 * 36 * 8 * 128 * 2
    assert lib.kvq_window_bytes(C.byref(d), C.byref(_win(dtype=0))) == 2 * 36 * 8 * 128 * 4
    assert lib.kvq_window_bytes(C.byref(d), C.byref(_win(flush=0))) == 0
    # windowed decodes always merge through the workspace, even unsplit
    assert lib.kvq_decode_workspace_bytes(C.byref(d), 64, 32, 256) == 0
    assert lib.kvq_window_workspace_bytes(C.byref(d), C.byref(_win()), 64, 32, 256) >= 64 * 32 * 130 * 4


def test_window_argument_checks(lib):
    d = _desc()
    p = C.c_void_p(0x10)

    def attn(**kw):
        return lib.kvq_window_decode_attn(
            C.byref(kw.get("d", d)), C.byref(kw.get("w", _win())), kw.get("q", p), kw.get("B", 2),
            kw.get("Hq", 32), None, kw.get("bt", p), kw.get("mp", 4), kw.get("sl", p), None,
            kw.get("msl", 256), 0.088, kw.get("out", p), kw.get("ws", p), kw.get("wsb", 0), None)

    def step(**kw):
        return lib.kvq_window_decode_step(
            C.byref(kw.get("d", d)), C.byref(kw.get("w", _win())), p, kw.get("k", p), kw.get("v", p),
            kw.get("B", 2), 32, None, None, p, 4, p, None, 256, 0.088, p, p, kw.get("wsb", 1 << 20), None)

    def prefill(**kw):
        return lib.kvq_window_prefill(
            C.byref(kw.get("d", d)), C.byref(kw.get("w", _win())), kw.get("k", p), p, kw.get("B", 2),
            kw.get("cu", p), kw.get("n", 100), kw.get("bt", p), kw.get("mp", 4), None, None, None)

    assert attn(w=_win(flush=0)) == -1
    assert attn(w=_win(sink=-1)) == -1
    assert attn(w=_win(sink=40000, keep=30000)) == -2
    # a window row of 2^32 or more elements is refused (32-bit offsets inside a row)
    assert attn(d=_desc(num_kv_heads=16384), Hq=16384, w=_win(sink=1000, keep=1000, flush=100)) == -2
    assert attn(d=_desc(num_kv_heads=16384), Hq=16384, w=_win(sink=1000, keep=1000, flush=47)) == -3
    assert attn(w=_win(dtype=7)) == -1
    assert attn(w=_win(k_win=None)) == -1
    assert attn(w=_win(num_rows=0)) == -1
    assert attn(Hq=30) == -1
    assert attn(mp=3) == -1
    assert attn() == -3                          # always needs a workspace
    assert attn(B=0) == 0
    assert step(k=None) == -1
    assert step(d=_desc(p_lo=0.7, p_hi=0.2)) == -1
    assert step(wsb=0) == -3
    assert step(B=0) == 0
    assert prefill(cu=None) == -1
    assert prefill(mp=0) == -1
    assert prefill(w=_win(flush=0)) == -1
    assert prefill(n=0) == 0
    assert prefill(B=0) == 0


def test_noalloc_rejects_sizes_beyond_its_scratch(lib):
    """Sizes whose partial outputs exceed the allocation-free decode's array are refused on
    the host, before any device call (null pointers are never touched)."""
    d = _lib.KvqCacheDesc(8, 128, 64, 2, 2, 0, 0, 0.01, 0.99, 2.83, 2.83, 2048, None, None)
    need = lib.kvq_decode_workspace_bytes(C.byref(d), 65535, 128, 131072)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    st = lib.kvq_decode_attn_noalloc(C.byref(d), None, 1, 65535, 128, None, None, 2048, None, 131072,
                                     0.088, None, None)
    assert st == -3, st
    assert b"allocation-free" in lib.kvq_last_error()
