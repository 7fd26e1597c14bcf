"""The C ABI library loads, exports what include/attn_sink.h declares, and rejects bad arguments on
the host (every check runs before any HIP call, so none of this needs a GPU)."""
import ctypes
import os
import re

import pytest

import attention_learnable_sinks_attn_amd as asa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_sink.h")

needs_lib = pytest.mark.skipif(not os.path.exists(asa.library_path()),
                               reason="libattn_sink.so not built (python -m attention_learnable_sinks_attn_amd.build)")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_sink_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("attn_sink_fwd", "attn_sink_bwd", "attn_sink_bwd_workspace_bytes", "attn_sink_strerror"):
        assert n in names


@needs_lib
def test_library_exports_every_declared_symbol():
    lib = asa.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name


@needs_lib
def test_strerror_and_kernel_names():
    lib = asa.load_library()
    for code in asa.ERROR_CODES:
        assert lib.attn_sink_strerror(code)
    assert lib.attn_sink_strerror(12345) == b"unknown error code"
    n = lib.attn_sink_bwd_num_kernels()
    assert n >= 1
    assert all(lib.attn_sink_bwd_kernel_name(i) for i in range(n))
    assert lib.attn_sink_bwd_kernel_name(n) is None


def shape(T=128, B=1, maxlen=128, hq=8, hkv=2, d=64, scale=0.0, dtype=0):
    return asa.Shape(T, B, maxlen, hq, hkv, d, scale, dtype)


# Fake, 256-byte aligned "device" addresses: validation must fail before anything dereferences them.
P = 0x10000
PM = 0x10008  # 8-byte aligned only


def fwd(lib, s, q=P, k=P, v=P, sinks=P, causal=1, window=0, cu=P, out=P, lse=P):
    return lib.attn_sink_fwd(q, k, v, sinks, causal, window, cu, ctypes.byref(s) if s is not None else None, out, lse,
                              None)


def bwd(lib, s, ws=P, ws_bytes=None, causal=1, window=0, **ptrs):
    p = dict(q=P, k=P, v=P, sinks=P, out=P, lse=P, dout=P, cu=P, dq=P, dk=P, dv=P, ds=P)
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = lib.attn_sink_bwd_workspace_bytes(ctypes.byref(s)) if s is not None else 0
    return lib.attn_sink_bwd(p["q"], p["k"], p["v"], p["sinks"], p["out"], p["lse"], p["dout"], causal, window, p["cu"],
                             ctypes.byref(s) if s is not None else None, ws, ws_bytes, p["dq"], p["dk"], p["dv"],
                             p["ds"], None)


@needs_lib
def test_forward_argument_errors():
    lib = asa.load_library()
    assert fwd(lib, None) == -1
    assert fwd(lib, shape(), q=None) == -1
    assert fwd(lib, shape(), sinks=None) == -1
    assert fwd(lib, shape(), cu=None) == -1
    assert fwd(lib, shape(), lse=None) == -1
    assert fwd(lib, shape(T=-1)) == -2
    assert fwd(lib, shape(B=0)) == -2
    assert fwd(lib, shape(hq=6, hkv=4)) == -2
    assert fwd(lib, shape(hkv=0)) == -2
    assert fwd(lib, shape(maxlen=-1)) == -2
    assert fwd(lib, shape(maxlen=129)) == -2
    assert fwd(lib, shape(d=96)) == -3   # head_dim 64 and 128 only
    assert fwd(lib, shape(d=32)) == -3
    assert fwd(lib, shape(dtype=2)) == -3  # bf16 (1) is a valid forward output dtype
    assert fwd(lib, shape(), q=PM) == -7
    assert fwd(lib, shape(), out=PM) == -7


@needs_lib
def test_backward_argument_errors():
    lib = asa.load_library()
    assert bwd(lib, None) == -1
    assert bwd(lib, shape(), dout=None) == -1
    assert bwd(lib, shape(), ds=None) == -1
    assert bwd(lib, shape(), dq=None) == -1
    assert bwd(lib, shape(hq=5, hkv=2)) == -2
    assert bwd(lib, shape(d=32)) == -3
    assert bwd(lib, shape(dtype=1)) == -3  # the backward reads the fp32 forward output
    s = shape()
    need = lib.attn_sink_bwd_workspace_bytes(ctypes.byref(s))
    assert bwd(lib, s, ws=None) == -5
    assert bwd(lib, s, ws_bytes=need - 1) == -5
    assert bwd(lib, s, dk=PM) == -7


@needs_lib
def test_workspace_size_formula():
    lib = asa.load_library()
    s = shape(T=4096, maxlen=4096, hq=64, hkv=8)
    need = lib.attn_sink_bwd_workspace_bytes(ctypes.byref(s))
    # -LSE/scale and -D_i for every (head, row), one dSink partial per (head, 32-row block slot), and
    # fp32 dK/dV partials for the two query-head halves of each KV group; each region 256-byte aligned
    assert need == 2 * 64 * 4096 * 4 + 64 * (4096 // 32 + 1 + 1) * 4 + 2 * 2 * 4096 * 8 * 64 * 4
    assert need % 256 == 0
    assert lib.attn_sink_bwd_workspace_bytes(None) == 0
    assert lib.attn_sink_bwd_workspace_bytes(ctypes.byref(shape(d=16))) == 0


@needs_lib
def test_timed_entry_point_checks_event_count():
    lib = asa.load_library()
    s = shape()
    need = lib.attn_sink_bwd_workspace_bytes(ctypes.byref(s))
    n = lib.attn_sink_bwd_num_kernels()
    evs = (ctypes.c_void_p * n)(*([P] * n))  # one too few
    rc = lib.attn_sink_bwd_timed(P, P, P, P, P, P, P, 1, 0, P, ctypes.byref(s), P, need, P, P, P, P, None, evs, n)
    assert rc == -2


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(asa, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(asa, "_lib", None)
    with pytest.raises(ImportError):
        asa.load_library()


def dshape(tq=8, tk=300, B=2, max_q=4, max_k=200, hq=8, hkv=1, d=64, scale=0.0, dtype=0):
    return asa.DecodeShape(tq, tk, B, max_q, max_k, hq, hkv, d, scale, dtype)


def decode(lib, s, ws=P, ws_bytes=None, window=0, **ptrs):
    p = dict(q=P, k=P, v=P, sinks=P, cuq=P, cuk=P, out=P, lse=P)
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = lib.attn_sink_decode_workspace_bytes(ctypes.byref(s)) if s is not None else 0
    return lib.attn_sink_decode_fwd(p["q"], p["k"], p["v"], p["sinks"], window, p["cuq"], p["cuk"],
                                    ctypes.byref(s) if s is not None else None, ws, ws_bytes, p["out"], p["lse"], None)


@needs_lib
def test_decode_argument_errors():
    lib = asa.load_library()
    assert decode(lib, None) == -1
    assert decode(lib, dshape(), q=None) == -1
    assert decode(lib, dshape(), k=None) == -1
    assert decode(lib, dshape(), sinks=None) == -1
    assert decode(lib, dshape(), cuk=None) == -1
    assert decode(lib, dshape(), lse=None) == -1
    assert decode(lib, dshape(tq=-1)) == -2
    assert decode(lib, dshape(B=0)) == -2
    assert decode(lib, dshape(hq=6, hkv=4)) == -2
    assert decode(lib, dshape(max_q=9)) == -2    # above total_q
    assert decode(lib, dshape(max_k=301)) == -2  # above total_k
    assert decode(lib, dshape(max_q=0)) == -2    # new tokens but max_q = 0
    assert decode(lib, dshape(d=96)) == -3
    assert decode(lib, dshape(dtype=2)) == -3
    # at most 1024 (new token, query head) pairs per KV head
    assert decode(lib, dshape(tq=300, max_q=129, hq=8, hkv=1)) == -3
    assert decode(lib, dshape(tq=300, max_q=129, hq=64, hkv=8)) == -3
    assert decode(lib, dshape(tq=300, max_q=33, hq=32, hkv=1)) == -3
    assert decode(lib, dshape(), window=-1) == -4
    s = dshape()
    need = lib.attn_sink_decode_workspace_bytes(ctypes.byref(s))
    assert decode(lib, s, ws=None) == -5
    assert decode(lib, s, ws_bytes=need - 1) == -5
    assert decode(lib, s, ws=PM) == -5
    assert decode(lib, s, k=PM) == -7
    assert decode(lib, s, out=PM) == -7
    # nothing to compute: succeeds without touching memory (no HIP call is made)
    assert decode(lib, dshape(tq=0, max_q=0), q=None, out=None, lse=None) == 0


@needs_lib
def test_decode_workspace_formula():
    lib = asa.load_library()
    # 8 sequences x 8 KV heads = 64 (sequence, KV head) pairs; the key axis is split so that about
    # 4096 waves run: 32768 keys = 512 tiles of 64 -> chunks of 8 tiles -> 64 chunks per pair. Each
    # chunk keeps a 32 x 64 fp32 partial output and a running max and sum per column.
    s = dshape(tq=8, tk=200000, B=8, max_q=1, max_k=32768, hq=64, hkv=8)
    need = lib.attn_sink_decode_workspace_bytes(ctypes.byref(s))
    assert need == 64 * 64 * 32 * 64 * 4 + 64 * 64 * 2 * 32 * 4
    assert lib.attn_sink_decode_workspace_bytes(None) == 0
    assert lib.attn_sink_decode_workspace_bytes(ctypes.byref(dshape(tq=300, max_q=129))) == 0
    # 40 columns per KV head: two groups of 32, each with its own partials
    s2 = dshape(tq=8, tk=200000, B=8, max_q=5, max_k=32768, hq=64, hkv=8)
    need2 = lib.attn_sink_decode_workspace_bytes(ctypes.byref(s2))
    # 128 (sequence, KV head, column group) triples -> 4096 / 128 = 32 chunks of 16 tiles
    assert need2 == 128 * 32 * 32 * 64 * 4 + 128 * 32 * 2 * 32 * 4


@needs_lib
def test_decode_timed_entry_point_checks_event_count():
    lib = asa.load_library()
    s = dshape()
    need = lib.attn_sink_decode_workspace_bytes(ctypes.byref(s))
    n = lib.attn_sink_decode_num_kernels()
    assert [lib.attn_sink_decode_kernel_name(i) for i in range(n)] == [b"attn_sink_decode_partial_kernel",
                                                                      b"attn_sink_decode_combine_kernel"]
    assert lib.attn_sink_decode_kernel_name(n) is None
    evs = (ctypes.c_void_p * n)(*([P] * n))  # one too few
    rc = lib.attn_sink_decode_fwd_timed(P, P, P, P, 0, P, P, ctypes.byref(s), P, need, P, P, None, evs, n)
    assert rc == -2


@needs_lib
def test_workspace_without_head_halves():
    lib = asa.load_library()
    # 32768 tokens: 512 key blocks x 8 KV heads = 4096 dK/dV workgroups without splitting the query
    # heads, so the pass writes dK/dV itself and needs no partial sums
    s = shape(T=32768, maxlen=32768, hq=64, hkv=8)
    need = lib.attn_sink_bwd_workspace_bytes(ctypes.byref(s))
    assert need == 2 * 64 * 32768 * 4 + 64 * (32768 // 32 + 1 + 1) * 4
    # an odd group never splits
    s = shape(T=4096, maxlen=4096, hq=24, hkv=8)
    dsink = 24 * (4096 // 32 + 2) * 4
    assert lib.attn_sink_bwd_workspace_bytes(ctypes.byref(s)) == 2 * 24 * 4096 * 4 + (dsink + 255) // 256 * 256


C_CALLER = r"""
#include <stdio.h>
#include "attn_sink.h"
int main(void) {
  const int32_t cu[3] = {0, 3000, 4096};
  attn_sink_shape s = {.total_tokens = 4096, .num_seqs = 2, .max_seqlen = 3000, .num_heads_q = 64,
                       .num_heads_kv = 8, .head_dim = 64, .softmax_scale = 0.0f, .out_dtype = ATTN_SINK_F32};
  printf("%d %d %zu %d %s\n", attn_sink_check_cu_seqlens(cu, 2, 4096, 3000),
         attn_sink_check_cu_seqlens(cu, 2, 4096, 2999), attn_sink_bwd_workspace_bytes(&s),
         attn_sink_bwd_num_kernels(), attn_sink_strerror(ATTN_SINK_ERR_BAD_SEQLENS));
  return 0;
}
"""


def _compiler(name):
    import shutil
    path = shutil.which(name)
    if path is None:
        pytest.skip(f"{name} not found")
    return path


@pytest.mark.parametrize("cc,std,suffix", [("gcc", "-std=c99", ".c"), ("g++", "-std=c++17", ".cpp")])
def test_header_compiles_alone(tmp_path, cc, std, suffix):
    # plain C and C++ callers need no HIP headers
    src = tmp_path / ("use" + suffix)
    src.write_text('#include "attn_sink.h"\nint f(void) { return ATTN_SINK_OK + (int)sizeof(attn_sink_shape); }\n')
    import subprocess
    r = subprocess.run([_compiler(cc), std, "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-I",
                        os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


@needs_lib
def test_c_program_links_and_calls_host_entry_points(tmp_path):
    import subprocess
    src = tmp_path / "caller.c"
    src.write_text(C_CALLER)
    exe = tmp_path / "caller"
    libdir = os.path.dirname(asa.library_path())
    r = subprocess.run([_compiler("gcc"), "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        str(src), "-o", str(exe), f"-L{libdir}", "-l:libattn_sink.so", f"-Wl,-rpath,{libdir}"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    fields = r.stdout.split(" ", 4)
    lib = asa.load_library()
    s = asa.Shape(4096, 2, 3000, 64, 8, 64, 0.0, 0)
    assert int(fields[0]) == 0 and int(fields[1]) == -8
    assert int(fields[2]) == lib.attn_sink_bwd_workspace_bytes(ctypes.byref(s))
    assert int(fields[3]) == lib.attn_sink_bwd_num_kernels()
    assert fields[4].startswith("cu_seqlens")
