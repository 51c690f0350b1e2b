"""The C ABI library (CPU only: loading, exported symbols, argument checks).

Argument validation runs before any HIP call, so invalid requests can be
made here without a GPU; nothing in this file launches a kernel.
"""

import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    from io_aware_tiled_05_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libfa.so is not built (run __graft_entry__.build())")
    return _lib.load()


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "fa_bwd", "fa_bwd_blocksparse", "fa_bwd_dropout", "fa_bwd_noalloc", "fa_bwd_stage",
        "fa_bwd_strided", "fa_bwd_workspace_size", "fa_fwd_strided",
        "fa_decode", "fa_decode_workspace_size", "fa_fwd", "fa_fwd_blocksparse",
        "fa_fwd_dropout", "fa_status_string"])


def test_library_exports_every_declared_symbol(lib):
    from io_aware_tiled_05_amd import _lib
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, name


def test_library_has_no_undefined_kernel_stubs(lib):
    # every kernel the launchers can select must have its host launch stub
    # in the library; a missing one only fails when the library is opened on
    # a machine with a GPU
    import shutil
    import subprocess
    from io_aware_tiled_05_amd import _lib
    nm = shutil.which("nm") or shutil.which("llvm-nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--undefined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    stubs = [line for line in out.splitlines() if "__device_stub__" in line]
    assert stubs == [], stubs


def test_status_strings(lib):
    assert lib.fa_status_string(0) == b"ok"
    assert lib.fa_status_string(-1) == b"invalid argument"
    assert lib.fa_status_string(-2) == b"unsupported configuration"
    assert lib.fa_status_string(-3) == b"HIP launch error"
    assert b"fixed scratch buffer" in lib.fa_status_string(-4)
    assert lib.fa_status_string(7) == b"unknown status"


def ws_formula(B, H, N, d):
    # per query row: D, shift and their scaled negations (4 floats) and the
    # fp16 copies of its q, k and dO rows (6 d bytes); per (b, h): four
    # maxima and four partial maxima from each of at most 128 D-pass
    # workgroups; 256-byte alignment of nine regions
    return 16 * B * H * N + 6 * B * H * N * d + 16 * B * H + 16 * 128 * B * H


def test_workspace_is_linear_in_N(lib):
    for B, H, N, d in [(1, 16, 16384, 64), (2, 3, 1000, 128), (1, 1, 1, 64)]:
        got = lib.fa_bwd_workspace_size(B, H, N, d)
        assert ws_formula(B, H, N, d) <= got < ws_formula(B, H, N, d) + 9 * 256
        assert got % 256 == 0
    a, b = lib.fa_bwd_workspace_size(1, 16, 8192, 64), lib.fa_bwd_workspace_size(1, 16, 16384, 64)
    assert abs(b - 2 * a) <= 16 * 128 * 16 + 9 * 256
    assert lib.fa_bwd_workspace_size(2, 2, 256, 64) == WS
    assert lib.fa_bwd_workspace_size(0, 1, 1, 64) == 0


# Fake, never-dereferenced, 16-byte aligned "device" addresses: validation
# rejects every call below before anything touches them.
P = 0x100000
WS = 418048  # fa_bwd_workspace_size(2, 2, 256, 64), checked below
F16, BF16, F32 = 1, 2, 0


def fwd(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=128, d=64, scale=0.125, causal=0,
             key_len=None, dtype=BF16)
    a.update(kw)
    return lib.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                      a["d"], a["scale"], a["causal"], a["key_len"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(lse=None), -1),
    (dict(q=P + 8), -1),                          # misaligned
    (dict(B=0), -1), (dict(N=0), -1), (dict(H=-1), -1),
    (dict(d=48), -2), (dict(d=160), -2), (dict(d=16), -2),
    (dict(scale=float("nan")), -1), (dict(scale=float("inf")), -1), (dict(scale=0.0), -1),
    (dict(causal=2), -1), (dict(dtype=7), -1),
    (dict(B=1 << 16, H=1 << 16, N=1), -1),        # B*H too large
    (dict(N=1 << 20, H=64, d=64), -1),            # tensor exceeds 2^31 elements
])
def test_fwd_validation(lib, kw, status):
    assert fwd(lib, **kw) == status


def bwd(lib, blocksparse=False, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, dO=P, dq=P, dk=P, dv=P, B=2, H=2, N=256, d=64,
             scale=0.125, causal=0, key_len=None, ws=P, ws_bytes=WS, dtype=BF16,
             bm=P, bs=128)
    a.update(kw)
    if blocksparse:
        return lib.fa_bwd_blocksparse(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dO"],
                                      a["dq"], a["dk"], a["dv"], a["B"], a["H"], a["N"],
                                      a["d"], a["scale"], a["bm"], a["bs"], a["ws"],
                                      a["ws_bytes"], a["dtype"], None)
    return lib.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dO"], a["dq"], a["dk"],
                      a["dv"], a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"],
                      a["key_len"], a["ws"], a["ws_bytes"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dO=None), -1), (dict(dk=None), -1), (dict(ws=None), -1),
    (dict(ws_bytes=WS - 1), -1),                  # workspace too small
    (dict(d=80), -2),
    (dict(scale=-1.0), -1), (dict(N=0), -1),
])
def test_bwd_validation(lib, kw, status):
    assert bwd(lib, **kw) == status


def noalloc(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, dO=P, dq=P, dk=P, dv=P, B=2, H=2, N=256, d=64,
             scale=0.125, causal=0, key_len=None, dtype=BF16)
    a.update(kw)
    return lib.fa_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dO"], a["dq"],
                              a["dk"], a["dv"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                              a["causal"], a["key_len"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dO=None), -1), (dict(dv=None), -1), (dict(lse=None), -1), (dict(dq=P + 4), -1),
    (dict(d=80), -2), (dict(scale=-1.0), -1), (dict(N=0), -1), (dict(causal=3), -1),
    (dict(dtype=9), -1),
    # fa_bwd_workspace_size(1, 16, 16384, 128) = 196 MiB > the 128 MiB array
    (dict(B=1, H=16, N=16384, d=128), -4),
    (dict(B=4, H=16, N=16384, d=64), -4),
])
def test_bwd_noalloc_validation(lib, kw, status):
    # every case is rejected before any HIP call
    assert noalloc(lib, **kw) == status


def test_noalloc_scratch_limit_matches_header(lib):
    from io_aware_tiled_05_amd import _lib
    src = open(HEADER).read()
    assert "#define FA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)" in src
    assert _lib.FA_NOALLOC_SCRATCH_BYTES == 128 << 20
    # the bench workload's backward fits it, twice its size does not
    assert lib.fa_bwd_workspace_size(1, 16, 16384, 64) <= 128 << 20
    assert lib.fa_bwd_workspace_size(2, 16, 16384, 64) > 128 << 20


def strided_layout(d=64, **over):
    from io_aware_tiled_05_amd._lib import FaLayout, FaStrides
    N, H = 256, 2
    packed = dict(batch=H * N * d, head=N * d, row=d)
    lay = FaLayout(*(FaStrides(**packed) for _ in range(8)))
    for name, st in over.items():
        setattr(lay, name, FaStrides(*st))
    return lay


def fwd_strided(lib, lay=None, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, H=2, N=256, d=64, scale=0.125, causal=0,
             key_len=None, bm=None, bs=128, p=0.0, dtype=BF16)
    a.update(kw)
    return lib.fa_fwd_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                              a["d"], a["scale"], a["causal"], a["key_len"], a["bm"], a["bs"],
                              a["p"], 1, 0, lay, a["dtype"], None)


def bwd_strided(lib, lay=None, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, dO=P, dq=P, dk=P, dv=P, B=2, H=2, N=256, d=64,
             scale=0.125, causal=0, key_len=None, bm=None, bs=128, p=0.0, ws=P, ws_bytes=WS,
             dtype=BF16)
    a.update(kw)
    return lib.fa_bwd_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dO"], a["dq"],
                              a["dk"], a["dv"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                              a["causal"], a["key_len"], a["bm"], a["bs"], a["p"], 1, 0, lay,
                              a["ws"], a["ws_bytes"], a["dtype"], None)


# (layout overrides, other args, forward status, backward status); "ok" means
# the layout passed validation, shown by the unsupported head dimension 80
# (checked after the strides) failing next, so that no case reaches a HIP
# call
STRIDED_CASES = [
    (dict(q=(256 * 64, 64, 4)), {}, -1, -1),              # row stride not a multiple of 8
    (dict(k=(2 * 256 * 64, 64, 2 * 64)), {}, "ok", "ok"),  # [B][N][H][d] views are fine
    (dict(o=(256 * 64, 64, 32)), {}, -1, "ok"),           # output rows overlap (o is read
                                                           # only by the backward)
    (dict(v=(-64, 64, 64)), {}, -1, -1),                  # negative stride
    (dict(q=(0, 0, 1 << 24)), {}, -1, -1),                # row stride too large
    (dict(q=(256 * 16, 16, 16)), dict(dtype=F32), "ok", "ok"),  # fp32: multiples of 4
    (dict(q=(256 * 64, 64, 68)), {}, -1, -1),             # 16-bit: multiples of 8
    ({}, dict(bm=P, causal=1), -1, -1), ({}, dict(bm=P, p=0.1), -1, -1),
    ({}, dict(bm=P, bs=64), -2, -2), ({}, dict(p=1.5), -1, -1),
    ({}, dict(p=0.1, dtype=F32), -2, -2), ({}, dict(bm=P, dtype=F32), -2, -2),
]


@pytest.mark.parametrize("over,kw,fst,bst", STRIDED_CASES)
def test_strided_validation(lib, over, kw, fst, bst):
    for call, want in ((fwd_strided, fst), (bwd_strided, bst)):
        if want == "ok":
            assert call(lib, strided_layout(d=80, **over), d=80, **kw) == -2
        else:
            assert call(lib, strided_layout(**over), **kw) == want


def test_strided_output_strides_checked_in_backward(lib):
    # dq/dk/dv rows must not overlap either (dO, an input, may)
    for name in ("dq", "dk", "dv"):
        assert bwd_strided(lib, strided_layout(**{name: (256 * 64, 64, 8)})) == -1


@pytest.mark.parametrize("kw,status", [
    (dict(bm=None), -1), (dict(bs=64), -2), (dict(bs=0), -1), (dict(dtype=F32), -2),
    (dict(ws_bytes=0), -1),
])
def test_blocksparse_validation(lib, kw, status):
    assert bwd(lib, blocksparse=True, **kw) == status
    fkw = {k: v for k, v in kw.items() if k in ("bm", "bs", "dtype")}
    if fkw:
        a = dict(bm=P, bs=128, dtype=BF16)
        a.update(fkw)
        st = lib.fa_fwd_blocksparse(P, P, P, P, P, 1, 1, 256, 64, 0.125, a["bm"], a["bs"],
                                    a["dtype"], None)
        assert st == status


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from io_aware_tiled_05_amd import _lib
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load()


def stage(lib, st, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, dO=P, dq=P, dk=P, dv=P, B=2, H=2, N=256, d=64,
             scale=0.125, causal=0, key_len=None, bm=None, bs=128, ws=P, ws_bytes=WS,
             dtype=BF16)
    a.update(kw)
    return lib.fa_bwd_stage(st, a["q"], a["k"], a["v"], a["o"], a["lse"], a["dO"], a["dq"],
                            a["dk"], a["dv"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                            a["causal"], a["key_len"], a["bm"], a["bs"], a["ws"], a["ws_bytes"],
                            a["dtype"], None)


@pytest.mark.parametrize("st,kw,status", [
    (0, {}, -1), (5, {}, -1), (-1, {}, -1), (4, dict(d=80), -2), (4, dict(ws=None), -1),
    (1, dict(ws=None), -1), (2, dict(d=80), -2), (3, dict(dtype=F32, bm=P), -2),
    (2, dict(bm=P, causal=1), -1), (2, dict(bm=P, key_len=P), -1), (3, dict(bm=P, bs=64), -2),
    (1, dict(ws_bytes=8), -1),
])
def test_bwd_stage_validation(lib, st, kw, status):
    assert stage(lib, st, **kw) == status


def test_decode_workspace(lib):
    # one partial (d + 2 floats) per (b, h, query, key chunk); chunks of
    # 256 .. 1024 keys, halved while the launch has under 1024 workgroups
    assert lib.fa_decode_workspace_size(1, 16, 1, 16384, 64) == 16 * 64 * 66 * 4  # 256-key chunks
    assert lib.fa_decode_workspace_size(8, 32, 1, 65536, 128) == 256 * 64 * 130 * 4  # 1024
    assert lib.fa_decode_workspace_size(1, 1, 1, 1, 64) == 66 * 4
    assert lib.fa_decode_workspace_size(0, 1, 1, 1, 64) == 0
    assert lib.fa_decode_workspace_size(1, 1, 1, 0, 64) == 0


def decode(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, Nq=1, Nk=1000, d=64, scale=0.125,
             key_len=None, ws=P, ws_bytes=1 << 20, dtype=BF16)
    a.update(kw)
    return lib.fa_decode(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                         a["Nk"], a["d"], a["scale"], a["key_len"], a["ws"], a["ws_bytes"],
                         a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(lse=None), -1), (dict(ws=None), -1), (dict(k=P + 4), -1),
    (dict(Nq=0), -1), (dict(Nk=0), -1), (dict(B=0), -1), (dict(d=112), -2),
    (dict(scale=0.0), -1), (dict(dtype=9), -1), (dict(ws_bytes=16), -1),
    (dict(Nk=1 << 25, H=1, d=128), -1),           # k exceeds 2^31 elements
])
def test_decode_validation(lib, kw, status):
    assert decode(lib, **kw) == status


def fwd_drop(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=128, d=64, scale=0.125, causal=0,
             key_len=None, p=0.1, seed=1, offset=0, dtype=BF16)
    a.update(kw)
    return lib.fa_fwd_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                              a["d"], a["scale"], a["causal"], a["key_len"], a["p"], a["seed"],
                              a["offset"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(p=-0.1), -1), (dict(p=1.0), -1), (dict(p=float("nan")), -1), (dict(q=None), -1),
    (dict(dtype=F32), -2), (dict(d=256), -2),
])
def test_dropout_validation(lib, kw, status):
    assert fwd_drop(lib, **kw) == status
    b = dict(p=0.1, dtype=BF16, d=64)
    b.update({k: v for k, v in kw.items() if k in ("p", "dtype", "d")})
    st = lib.fa_bwd_dropout(P, P, P, P, P, P, P, P, P, 2, 2, 256, b["d"], 0.125, 0, None, b["p"],
                            1, 0, P, WS, b["dtype"], None)
    if "q" not in kw:
        assert st == status
