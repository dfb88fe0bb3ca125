"""The C-ABI library: it loads, exports every declared entry point, and its
host-side argument checks return error codes before any HIP call (so these
run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")

try:
    import speculative_decoding_verification_04_amd as sv
    LIB = sv.library()
except RuntimeError as exc:  # not built
    LIB = None
    _why = str(exc)

needs_lib = pytest.mark.skipif(LIB is None, reason="libspecverify.so not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_steps():
    names = _declared()
    for n in ["spec_verify_greedy", "spec_verify_sample", "spec_commit_realign_kv",
              "spec_group_same_length", "spec_strerror", "spec_verify_greedy_workspace_bytes",
              "spec_verify_sample_workspace_bytes"]:
        assert n in names


@needs_lib
def test_every_declared_symbol_is_exported():
    for name in _declared():
        assert hasattr(LIB, name), name
    from speculative_decoding_verification_04_amd._lib import PROTOTYPES
    assert sorted(PROTOTYPES) == _declared()


@needs_lib
def test_strerror():
    assert sv.spec_strerror(0) == "ok"
    assert "invalid" in sv.spec_strerror(-1)
    assert "workspace" in sv.spec_strerror(-2)
    assert sv.spec_strerror(12345) == "unknown error"


@needs_lib
def test_workspace_queries():
    a = sv.spec_verify_greedy_workspace_bytes(32, 8, 128256, sv.SPEC_BF16)
    assert a > 32 * 9 * 8 and a % 256 == 0
    assert sv.spec_verify_greedy_workspace_bytes(0, 8, 100, sv.SPEC_BF16) == 0
    assert sv.spec_verify_greedy_workspace_bytes(1, 200, 100, sv.SPEC_BF16) == 0
    b = sv.spec_verify_sample_workspace_bytes(8, 4, 151936)
    assert b > 8 * 8 and b % 256 == 0
    assert sv.spec_verify_sample_workspace_bytes(8, 4, 1 << 30) == 0   # too many chunks
    c = sv.spec_process_workspace_bytes(72, 151936)
    assert c >= 72 * 16 and c % 256 == 0 and sv.spec_process_workspace_bytes(0, 100) == 0
    assert sv.spec_process_workspace_bytes(4, 0) == 0 and sv.spec_process_workspace_bytes(4, sv.SPEC_PROC_MAX_V + 1) == 0
    d = sv.spec_verify_sample_logits_workspace_bytes(8, 4, 151936)
    assert d > b and d % 256 == 0
    assert sv.spec_verify_sample_logits_workspace_bytes(8, 4, sv.SPEC_PROC_MAX_V + 1) == 0


# fake, never-dereferenced device addresses: validation fails before any use
A, B_, C_, D_, E_, F_, G_, H_ = (ctypes.c_void_p(0x10000 * (i + 1)) for i in range(8))
WS = ctypes.c_void_p(0x7000000)
N = None


@needs_lib
@pytest.mark.parametrize("args,code", [
    ((N, 1, 2, 4, 100, B_, -1, N, C_, D_, E_, N, N, WS, 1 << 20, N), sv.SPEC_EINVAL),      # NULL logits
    ((A, 1, 0, 4, 100, B_, -1, N, C_, D_, E_, N, N, WS, 1 << 20, N), sv.SPEC_EINVAL),      # B < 1
    ((A, 1, 2, 0, 100, B_, -1, N, C_, D_, E_, N, N, WS, 1 << 20, N), sv.SPEC_EINVAL),      # k < 1
    ((A, 1, 2, 4, 0, B_, -1, N, C_, D_, E_, N, N, WS, 1 << 20, N), sv.SPEC_EINVAL),        # V < 1
    ((A, 7, 2, 4, 100, B_, -1, N, C_, D_, E_, N, N, WS, 1 << 20, N), sv.SPEC_EINVAL),      # dtype
    ((A, 1, 2, 200, 100, B_, -1, N, C_, D_, E_, N, N, WS, 1 << 20, N), sv.SPEC_ECAPACITY),  # k > max
    ((ctypes.c_void_p(0x10001), 1, 2, 4, 100, B_, -1, N, C_, D_, E_, N, N, WS, 1 << 20, N), sv.SPEC_EINVAL),
    ((A, 1, 2, 4, 100, B_, -1, N, C_, D_, E_, N, N, WS, 8, N), sv.SPEC_EWORKSPACE),        # ws too small
    ((A, 1, 2, 4, 100, B_, -1, N, C_, D_, E_, N, N, ctypes.c_void_p(0x7000008), 1 << 20, N), sv.SPEC_EWORKSPACE),
    ((A, 1, 2, 4, 100, B_, -1, N, C_, C_, E_, N, N, WS, 1 << 20, N), sv.SPEC_EINVAL),      # outputs alias
    ((A, 1, 2, 4, 100, B_, -1, N, ctypes.c_void_p(0x10000 + 64), D_, E_, N, N, WS, 1 << 20, N), sv.SPEC_EINVAL),
])
def test_greedy_argument_errors(args, code):
    assert LIB.spec_verify_greedy(*args) == code


@needs_lib
@pytest.mark.parametrize("args,code", [
    ((N, B_, C_, D_, 2, 4, 100, -1, N, E_, F_, G_, N, N, N, WS, 1 << 20, N), sv.SPEC_EINVAL),
    ((A, B_, C_, D_, 2, 4, 1 << 30, -1, N, E_, F_, G_, N, N, N, WS, 1 << 40, N), sv.SPEC_ECAPACITY),
    ((A, B_, C_, D_, 2, 4, 100, -1, N, E_, F_, G_, N, N, N, WS, 16, N), sv.SPEC_EWORKSPACE),
    ((A, B_, C_, D_, 2, 4, 100, -1, N, E_, E_, G_, N, N, N, WS, 1 << 20, N), sv.SPEC_EINVAL),
])
def test_sample_argument_errors(args, code):
    assert LIB.spec_verify_sample(*args) == code


PROC_OK = (A, 1, 4, 1000, 0.7, 50, 0.9, B_, C_, D_, E_, WS, 1 << 20, N)


def _proc(**kw):
    names = ["logits", "dt", "R", "V", "T", "top_k", "top_p", "probs", "row_max", "row_thr",
             "row_mass", "ws", "ws_bytes", "stream"]
    a = dict(zip(names, PROC_OK))
    a.update(kw)
    return tuple(a[n] for n in names)


@needs_lib
@pytest.mark.parametrize("args,code", [
    (_proc(logits=N), sv.SPEC_EINVAL),
    (_proc(R=0), sv.SPEC_EINVAL),
    (_proc(V=0), sv.SPEC_EINVAL),
    (_proc(V=sv.SPEC_PROC_MAX_V + 1), sv.SPEC_EINVAL),
    (_proc(T=0.0), sv.SPEC_EINVAL),
    (_proc(T=-1.0), sv.SPEC_EINVAL),
    (_proc(T=float("inf")), sv.SPEC_EINVAL),
    (_proc(T=float("nan")), sv.SPEC_EINVAL),
    (_proc(top_k=-1), sv.SPEC_EINVAL),
    (_proc(top_p=0.0), sv.SPEC_EINVAL),
    (_proc(top_p=1.5), sv.SPEC_EINVAL),
    (_proc(dt=5), sv.SPEC_EINVAL),
    (_proc(logits=ctypes.c_void_p(0x10001)), sv.SPEC_EINVAL),        # misaligned bf16
    (_proc(ws_bytes=8), sv.SPEC_EWORKSPACE),
    (_proc(probs=ctypes.c_void_p(0x10000 + 64)), sv.SPEC_EINVAL),    # probs overlap logits
    (_proc(row_max=C_, row_thr=C_), sv.SPEC_EINVAL),                  # outputs alias
])
def test_process_argument_errors(args, code):
    assert LIB.spec_process_logits(*args) == code


VSL_OK = (A, B_, 1, 2, 4, 1000, 0.7, 0, 1.0, C_, D_, -1, N, E_, F_, G_, N, N, N, WS, 1 << 24, N)


def _vsl(**kw):
    names = ["zp", "zq", "dt", "B", "k", "V", "T", "top_k", "top_p", "draft", "u", "eos", "rem",
             "acc", "emit", "toks", "offs", "mass", "status", "ws", "ws_bytes", "stream"]
    a = dict(zip(names, VSL_OK))
    a.update(kw)
    return tuple(a[n] for n in names)


@needs_lib
@pytest.mark.parametrize("args,code", [
    (_vsl(zp=N), sv.SPEC_EINVAL),
    (_vsl(zq=N), sv.SPEC_EINVAL),
    (_vsl(B=0), sv.SPEC_EINVAL),
    (_vsl(k=0), sv.SPEC_EINVAL),
    (_vsl(k=200), sv.SPEC_ECAPACITY),
    (_vsl(T=0.0), sv.SPEC_EINVAL),
    (_vsl(top_p=0.0), sv.SPEC_EINVAL),
    (_vsl(V=sv.SPEC_PROC_MAX_V + 1), sv.SPEC_EINVAL),
    (_vsl(ws_bytes=64), sv.SPEC_EWORKSPACE),
    (_vsl(emit=E_), sv.SPEC_EINVAL),                                 # outputs alias
])
def test_sample_logits_argument_errors(args, code):
    assert LIB.spec_verify_sample_logits(*args) == code


@needs_lib
@pytest.mark.parametrize("args,code", [
    ((N, 1, 2, 2, 2, 16, 8, 3, A, B_, C_, D_, E_, F_, G_, N, N, N), sv.SPEC_EINVAL),
    ((H_, 1, 0, 2, 2, 16, 8, 3, A, B_, C_, D_, E_, F_, G_, N, N, N), sv.SPEC_EINVAL),       # L < 1
    ((H_, 1, 2, 2, 2, 16, 8, 0, A, B_, C_, D_, E_, F_, G_, N, N, N), sv.SPEC_EINVAL),       # k < 1
    ((ctypes.c_void_p(0x80001), 1, 2, 2, 2, 16, 8, 3, A, B_, C_, D_, E_, F_, G_, N, N, N), sv.SPEC_EINVAL),
    ((H_, 1, 2, 2, 2, 16, 8, 3, A, B_, C_, A, E_, F_, G_, N, N, N), sv.SPEC_EINVAL),         # E' aliases E
    ((H_, 1, 2, 2, 2, 16, 8, 3, A, B_, C_, D_, B_, F_, G_, N, N, N), sv.SPEC_EINVAL),        # n' aliases n
])
def test_commit_argument_errors(args, code):
    assert LIB.spec_commit_realign_kv(*args) == code


@needs_lib
@pytest.mark.parametrize("args,code", [
    ((N, 1, 2, 2, 2, 16, 8, 3, A, B_, C_, D_, E_, N, N, N, N, N), sv.SPEC_EINVAL),        # NULL kv
    ((H_, 1, 2, 2, 2, 16, 8, 0, A, B_, C_, D_, E_, N, N, N, N, N), sv.SPEC_EINVAL),       # k < 1
    ((H_, 1, 2, 2, 2, 16, 8, 3, A, B_, C_, N, E_, N, N, N, N, N), sv.SPEC_EINVAL),        # NULL E'
    ((H_, 1, 2, 2, 2, 16, 8, 3, A, B_, C_, D_, B_, N, N, N, N, N), sv.SPEC_EINVAL),       # n' aliases n
    ((H_, 9, 2, 2, 2, 16, 8, 3, A, B_, C_, D_, E_, N, N, N, N, N), sv.SPEC_EINVAL),       # dtype
])
def test_resync_argument_errors(args, code):
    assert LIB.spec_resync_draft_kv(*args) == code


@needs_lib
@pytest.mark.parametrize("args,code", [
    ((4, 3, 16, 8, N, B_, C_, D_, E_, F_, G_, N, N), sv.SPEC_EINVAL),          # NULL n
    ((0, 3, 16, 8, A, B_, C_, D_, E_, F_, G_, N, N), sv.SPEC_EINVAL),          # B < 1
    ((4, 0, 16, 8, A, B_, C_, D_, E_, F_, G_, N, N), sv.SPEC_EINVAL),          # k < 1
    ((4, 3, 0, 8, A, B_, C_, D_, E_, F_, G_, N, N), sv.SPEC_EINVAL),           # page < 1
    ((4, 3, 16, 0, A, B_, C_, D_, E_, F_, G_, N, N), sv.SPEC_EINVAL),          # max_pages < 1
    ((4, 3, 16, 8, A, B_, C_, D_, D_, F_, G_, N, N), sv.SPEC_EINVAL),          # outputs alias
    ((4, 3, 16, 8, A, B_, C_, A, E_, F_, G_, N, N), sv.SPEC_EINVAL),           # output aliases input
    ((1 << 20, 3, 16, 1 << 12, A, B_, C_, D_, E_, F_, G_, N, N), sv.SPEC_EINVAL),  # table too large
])
def test_paged_argument_errors(args, code):
    assert LIB.spec_commit_paged(*args) == code


@needs_lib
@pytest.mark.parametrize("args,code", [
    ((N, 1, 2, 4, 100, B_, C_, D_, -1, N, E_, F_, G_, H_, N, N, WS, 1 << 20, N), sv.SPEC_EINVAL),      # NULL logits
    ((A, 1, 2, 0, 100, B_, C_, D_, -1, N, E_, F_, G_, H_, N, N, WS, 1 << 20, N), sv.SPEC_EINVAL),      # N < 1
    ((A, 1, 2, 300, 100, B_, C_, D_, -1, N, E_, F_, G_, H_, N, N, WS, 1 << 20, N), sv.SPEC_ECAPACITY),  # N > max
    ((A, 1, 2, 4, 100, B_, N, D_, -1, N, E_, F_, G_, H_, N, N, WS, 1 << 20, N), sv.SPEC_EINVAL),       # NULL links
    ((A, 1, 2, 4, 100, B_, C_, D_, -1, N, E_, F_, G_, H_, N, N, WS, 8, N), sv.SPEC_EWORKSPACE),
    ((A, 1, 2, 4, 100, B_, C_, D_, -1, N, E_, E_, G_, H_, N, N, WS, 1 << 20, N), sv.SPEC_EINVAL),      # alias
])
def test_tree_argument_errors(args, code):
    assert LIB.spec_verify_tree(*args) == code


@needs_lib
@pytest.mark.parametrize("args,code", [
    ((N, 1, 2, 2, 2, 16, 8, 4, A, B_, C_, N, N), sv.SPEC_EINVAL),
    ((H_, 1, 2, 2, 2, 16, 8, 0, A, B_, C_, N, N), sv.SPEC_EINVAL),
    ((H_, 1, 2, 2, 2, 16, 8, 300, A, B_, C_, N, N), sv.SPEC_ECAPACITY),
    ((H_, 1, 2, 2, 2, 16, 8, 4, A, N, C_, N, N), sv.SPEC_EINVAL),
    ((ctypes.c_void_p(0x80001), 1, 2, 2, 2, 16, 8, 4, A, B_, C_, N, N), sv.SPEC_EINVAL),
])
def test_compact_argument_errors(args, code):
    assert LIB.spec_compact_tree_kv(*args) == code


I_, J_, K_ = (ctypes.c_void_p(0x10000 * (i + 9)) for i in range(3))


def _tree_sample_args(**kw):
    a = dict(p=A, q=B_, draft=C_, fc=D_, ns=E_, u=F_, B=2, N=4, V=100, eos=-1, rem=N, acc=G_, emit=H_,
             toks=I_, path=J_, offs=K_, mass=N, st=N, ws=N, ws_bytes=0, stream=N)
    a.update(kw)
    return tuple(a.values())


@needs_lib
@pytest.mark.parametrize("args,code", [
    (_tree_sample_args(p=N), sv.SPEC_EINVAL),                       # NULL p
    (_tree_sample_args(path=N), sv.SPEC_EINVAL),                    # NULL path
    (_tree_sample_args(B=0), sv.SPEC_EINVAL),
    (_tree_sample_args(N=0), sv.SPEC_EINVAL),
    (_tree_sample_args(V=0), sv.SPEC_EINVAL),
    (_tree_sample_args(N=300), sv.SPEC_ECAPACITY),                 # N > SPEC_TREE_MAX_N
    (_tree_sample_args(V=(1 << 22) + 1), sv.SPEC_ECAPACITY),       # more chunks than one workgroup holds
    (_tree_sample_args(q=ctypes.c_void_p(0x20002)), sv.SPEC_EINVAL),   # misaligned q
    (_tree_sample_args(toks=G_), sv.SPEC_EINVAL),                  # outputs alias
    (_tree_sample_args(path=C_), sv.SPEC_EINVAL),                  # output over an input
    # several chunks (V = 20000): the workspace is used, and checked
    (_tree_sample_args(V=20000, ws=WS, ws_bytes=8), sv.SPEC_EWORKSPACE),     # workspace below the query
    (_tree_sample_args(V=20000, ws=ctypes.c_void_p(0x7000008), ws_bytes=1 << 20), sv.SPEC_EWORKSPACE),
])
def test_tree_sample_argument_errors(args, code):
    assert LIB.spec_verify_tree_sample(*args) == code


@needs_lib
def test_tree_sample_workspace_query():
    small = sv.spec_verify_tree_sample_workspace_bytes(8, 16, 151936)
    assert small >= 8 * 16 * 38 * 8 and small % 256 == 0            # slots for every pass of every chunk
    assert sv.spec_verify_tree_sample_workspace_bytes(200, 16, 151936) == 0   # large batch: one workgroup each
    assert sv.spec_verify_tree_sample_workspace_bytes(8, 300, 1000) == 0       # N beyond the maximum
    assert sv.spec_verify_tree_sample_workspace_bytes(64, 256, 1 << 22) == 0   # slots beyond 64 MB


@needs_lib
@pytest.mark.parametrize("args,code", [
    ((N, 10, 8, 2, B_, C_, D_, E_, F_, N), sv.SPEC_EINVAL),
    ((A, -1, 8, 2, B_, C_, D_, E_, F_, N), sv.SPEC_EINVAL),
    ((A, 10, 0, 2, B_, C_, D_, E_, F_, N), sv.SPEC_EINVAL),
    ((A, 10, 8, 0, B_, C_, D_, E_, F_, N), sv.SPEC_EINVAL),
    ((A, 5000, 8, 2, B_, C_, D_, E_, F_, N), sv.SPEC_ECAPACITY),
    ((A, 10, 8, 2, B_, B_, D_, E_, F_, N), sv.SPEC_EINVAL),
])
def test_group_argument_errors(args, code):
    assert LIB.spec_group_same_length(*args) == code


@needs_lib
def test_one_hip_runtime_in_the_process():
    """The library and torch share one HIP runtime (same device memory, same streams)."""
    import torch  # noqa: F401
    maps = open("/proc/self/maps").read().splitlines()
    hip = {line.split()[-1] for line in maps if "libamdhip64" in line}
    assert len(hip) == 1, hip
    assert any("libspecverify.so" in line for line in maps)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from speculative_decoding_verification_04_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load()


def test_header_is_plain_c(tmp_path):
    """The boundary is plain C: the header compiles as C99 on its own (no HIP,
    no torch types), and a C program can take the address of every entry
    point (linked against the library when it is built)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    names = _declared()
    src = tmp_path / "use.c"
    src.write_text('#include "spec_verify.h"\n#include <stdio.h>\n'
                   "typedef void (*any_fn)(void);\n"
                   "int main(void) {\n  any_fn fns[] = {\n"
                   + "".join(f"    (any_fn)&{n},\n" for n in names)
                   + "  };\n  printf(\"%d\\n\", (int)(sizeof fns / sizeof fns[0]));\n  return 0;\n}\n")
    inc = os.path.join(ROOT, "include")
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-pedantic", "-fsyntax-only", "-I", inc, str(src)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    if LIB is None:
        return
    libdir = os.path.join(ROOT, "speculative_decoding_verification_04_amd")
    exe = tmp_path / "use"
    r = subprocess.run([cc, "-std=c99", "-I", inc, str(src), "-L", libdir, "-lspecverify",
                        f"-Wl,-rpath,{libdir}", "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and int(r.stdout) == len(names)
