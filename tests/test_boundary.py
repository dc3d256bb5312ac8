"""The C ABI without a GPU: the library loads, exports what the header
declares, and every argument check returns its status before any HIP call
(attn_fwd_validate / attn_fwd_select_path are pure host logic)."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mi355_attn.h")

FP32, BF16, FP16 = 0, 1, 2
OK, INVALID, UNSUPPORTED, MISALIGNED, HIPERR = 0, 1, 2, 3, 4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*((?:attn|axial)_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(
        ["attn_fwd", "attn_fwd_validate", "attn_fwd_path", "attn_fwd_select_path",
         "attn_status_string", "attn_bwd", "attn_bwd_validate", "axial_pass",
         "axial_pass_validate", "axial_block", "attn_fwd_dv", "attn_fwd_dv_validate",
         "axial_pass_split", "attn_bwd_noalloc", "attn_fwd_fp8", "attn_fwd_fp8_validate",
         "attn_bwd_ws", "attn_bwd_work_bytes", "attn_bwd_work_error_offset"])


def test_library_exports_every_declared_symbol(hip_lib):
    lib = hip_lib.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", hip_lib.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)$", out, re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    assert set(hip_lib.EXPORTS) == set(declared_functions())


def test_header_constants_match_binding(hip_lib):
    text = open(HEADER).read()
    for name, val in re.findall(r"#define\s+(MI355_(?:ATTN|AXIAL)_\w+)\s+(\d+)", text):
        assert getattr(hip_lib, name) == int(val), name


# Stand-in addresses: never dereferenced (validation makes no HIP call).
A = 1 << 20
SZ = 1 << 34  # far apart, so none of the buffers below overlap


def ptrs():
    return A, A + SZ, A + 2 * SZ, A + 3 * SZ, A + 4 * SZ


def val(hip_lib, *, q=None, k=None, v=None, o=None, lse=None, B=2, H=3, M=100,
        N=70, D=64, scale=0.125, causal=0, dtype=BF16):
    p = ptrs()
    q = p[0] if q is None else q
    k = p[1] if k is None else k
    v = p[2] if v is None else v
    o = p[3] if o is None else o
    lse = p[4] if lse is None else lse
    return hip_lib.attn_fwd_validate(q, k, v, o, lse, B, H, M, N, D, scale, causal, dtype)


def test_valid_arguments(hip_lib):
    for dtype in (FP32, BF16, FP16):
        for D in (16, 32, 64, 128):
            for causal in (0, 1):
                assert val(hip_lib, D=D, dtype=dtype, causal=causal) == OK


def test_invalid_arguments(hip_lib):
    assert val(hip_lib, q=0) == INVALID
    assert val(hip_lib, k=0) == INVALID
    assert val(hip_lib, v=0) == INVALID
    assert val(hip_lib, o=0) == INVALID
    assert val(hip_lib, lse=0) == INVALID
    assert val(hip_lib, B=-1) == INVALID
    assert val(hip_lib, H=-1) == INVALID
    assert val(hip_lib, M=-1) == INVALID
    assert val(hip_lib, N=0) == INVALID
    assert val(hip_lib, N=-5) == INVALID
    assert val(hip_lib, D=0) == INVALID
    assert val(hip_lib, causal=2) == INVALID
    assert val(hip_lib, causal=-1) == INVALID
    assert val(hip_lib, dtype=3) == INVALID
    assert val(hip_lib, dtype=-1) == INVALID
    assert val(hip_lib, scale=float("inf")) == INVALID
    assert val(hip_lib, scale=float("nan")) == INVALID


def test_unsupported(hip_lib):
    for D in (1, 8, 48, 96, 256):
        assert val(hip_lib, D=D) == UNSUPPORTED
    assert val(hip_lib, M=1 << 40) == UNSUPPORTED           # M*D beyond 32-bit
    assert val(hip_lib, B=1 << 40, H=1 << 40) == UNSUPPORTED  # B*H overflows


def test_misaligned(hip_lib):
    p = ptrs()
    assert val(hip_lib, q=p[0] + 8) == MISALIGNED
    assert val(hip_lib, k=p[1] + 2) == MISALIGNED
    assert val(hip_lib, v=p[2] + 4) == MISALIGNED
    assert val(hip_lib, o=p[3] + 8) == MISALIGNED
    assert val(hip_lib, lse=p[4] + 2) == MISALIGNED
    assert val(hip_lib, lse=p[4] + 4) == OK  # fp32 alignment is enough for L


def test_overlaps(hip_lib):
    p = ptrs()
    assert val(hip_lib, o=p[0]) == INVALID            # o on q
    assert val(hip_lib, o=p[1] + 256) == INVALID      # o inside k
    assert val(hip_lib, lse=p[2] + 64) == INVALID     # lse inside v
    assert val(hip_lib, lse=p[3] + 1024) == INVALID   # lse inside o
    assert val(hip_lib, k=p[0], v=p[0]) == OK         # inputs may alias
    # o ends exactly where lse starts: adjacent, not overlapping
    o_bytes = 2 * 3 * 100 * 64 * 2
    assert val(hip_lib, lse=p[3] + o_bytes) == OK
    assert val(hip_lib, lse=p[3] + o_bytes - 4) == INVALID


def test_empty_problems_are_ok(hip_lib):
    assert val(hip_lib, B=0, q=0, k=0, v=0, o=0, lse=0) == OK
    assert val(hip_lib, H=0, q=0, k=0, v=0, o=0, lse=0) == OK
    assert val(hip_lib, M=0, N=0, q=0, k=0, v=0, o=0, lse=0) == OK
    # empty but with a bad flag is still rejected
    assert val(hip_lib, M=0, causal=3) == INVALID


def test_select_path(hip_lib):
    f = hip_lib.attn_fwd_select_path
    SMALL, MAIN = hip_lib.MI355_ATTN_PATH_SMALL, hip_lib.MI355_ATTN_PATH_MAIN
    assert f(128, 4, 32, 32, 16, 0, FP32) == SMALL   # axial pass
    assert f(1, 1, 64, 64, 32, 1, BF16) == SMALL
    assert f(128, 4, 32, 32, 16, 0, FP16) == SMALL
    assert f(4, 16, 4096, 4096, 128, 0, FP16) == MAIN
    assert f(1, 1, 128, 128, 64, 0, FP32) == MAIN    # single head fp32
    assert f(96, 1, 512, 512, 128, 0, FP32) == MAIN
    assert f(4, 16, 4096, 4096, 128, 0, BF16) == MAIN
    assert f(1, 1, 65, 32, 16, 0, FP32) == MAIN
    assert f(1, 1, 32, 32, 64, 0, FP32) == MAIN
    assert f(1, 1, 32, 0, 16, 0, FP32) == -1
    assert f(1, 1, 32, 32, 24, 0, FP32) == -1
    assert f(1, 1, 32, 32, 16, 0, 7) == -1


def test_status_strings(hip_lib):
    names = {OK: "ok", INVALID: "invalid argument", UNSUPPORTED: "unsupported problem",
             MISALIGNED: "misaligned pointer", HIPERR: "HIP launch error",
             5: "problem exceeds the no-alloc scratch buffer"}
    for code, s in names.items():
        assert hip_lib.attn_status_string(code) == s
    assert hip_lib.attn_status_string(99) == "unknown status"
    assert hip_lib.attn_status_string(-1) == "unknown status"


def test_python_wrapper_rejects_before_any_gpu_call(hip_lib):
    q = torch.zeros(1, 1, 4, 16)
    with pytest.raises(ValueError):
        hip_lib.attn_fwd(q, q, q)                     # CPU tensors
    with pytest.raises(ValueError):
        hip_lib.attn_fwd(q.half(), q.half(), q.half())  # not a GPU tensor either
    assert hip_lib.default_scale(128) == ctypes.c_float(128 ** -0.5).value


# ------------------------------------------------------------- attn_bwd
def bval(hip_lib, B=2, H=3, M=100, N=70, D=64, scale=0.125, causal=0, dtype=BF16,
         **over):
    names = ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "delta")
    p = {n: A + i * SZ for i, n in enumerate(names)}
    p.update(over)
    return hip_lib.attn_bwd_validate(*(p[n] for n in names), B, H, M, N, D, scale,
                                     causal, dtype)


def test_bwd_valid_and_empty(hip_lib):
    for D in (32, 64, 128):
        for causal in (0, 1):
            assert bval(hip_lib, D=D, causal=causal) == OK
    assert bval(hip_lib, M=1, N=1) == OK
    assert bval(hip_lib, M=0, N=5) == OK        # dK = dV = 0 to write
    assert bval(hip_lib, B=0) == OK
    assert bval(hip_lib, M=0, N=0) == OK
    assert bval(hip_lib, B=0, q=None, dq=None) == OK  # nothing to do: no pointer needed
    # inputs may alias one another
    assert bval(hip_lib, k=A, v=A, o=A, dout=A) == OK


def test_bwd_invalid(hip_lib):
    assert bval(hip_lib, B=-1) == INVALID
    assert bval(hip_lib, N=-1) == INVALID
    assert bval(hip_lib, M=4, N=0) == INVALID
    assert bval(hip_lib, D=0) == INVALID
    assert bval(hip_lib, causal=2) == INVALID
    assert bval(hip_lib, dtype=7) == INVALID
    assert bval(hip_lib, scale=float("nan")) == INVALID
    assert bval(hip_lib, scale=float("inf")) == INVALID
    for n in ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "delta"):
        assert bval(hip_lib, **{n: None}) == INVALID, n
        # no query rows: only the key-side buffers are used
        expect = INVALID if n in ("k", "v", "dk", "dv") else OK
        assert bval(hip_lib, M=0, N=5, **{n: None}) == expect, n


def test_bwd_unsupported(hip_lib):
    assert bval(hip_lib, dtype=FP32) == UNSUPPORTED
    assert bval(hip_lib, dtype=FP16) == OK
    for D in (16, 8, 48, 256):
        assert bval(hip_lib, D=D) == UNSUPPORTED, D
    assert bval(hip_lib, M=1 << 31, N=10) == UNSUPPORTED   # M*D past 32 bits
    assert bval(hip_lib, B=1 << 40, H=1 << 40) == UNSUPPORTED


def test_bwd_misaligned(hip_lib):
    # each tensor moved by 8 bytes, to an address no other buffer is near
    for i, n in enumerate(("q", "k", "v", "o", "dout", "dq", "dk", "dv")):
        assert bval(hip_lib, **{n: A + (20 + i) * SZ + 8}) == MISALIGNED, n
    assert bval(hip_lib, lse=A + 4 * SZ + 2) == MISALIGNED
    assert bval(hip_lib, delta=A + 9 * SZ + 2) == MISALIGNED
    assert bval(hip_lib, lse=A + 4 * SZ + 4, delta=A + 9 * SZ + 4) == OK


def test_bwd_overlaps(hip_lib):
    # B=2, H=3, M=100, N=70, D=64 bf16: q/o/dout/dq 76800 B, k/v/dk/dv 53760 B,
    # lse/delta 2400 B.
    assert bval(hip_lib, dq=A) == INVALID               # dq on q
    assert bval(hip_lib, dk=A + 2 * SZ + 53760 - 16) == INVALID  # dk tail over v
    assert bval(hip_lib, dk=A + 2 * SZ + 53760) == OK   # dk right after v
    assert bval(hip_lib, delta=A + 4 * SZ) == INVALID   # delta on lse
    assert bval(hip_lib, dv=A + 7 * SZ + 16) == INVALID  # dv inside dk
    assert bval(hip_lib, delta=A + 6 * SZ + 76800 - 4) == INVALID  # delta over dq's end
    assert bval(hip_lib, dq=A + 5 * SZ) == INVALID      # dq on dout


def test_bwd_python_wrapper_rejects_before_any_gpu_call(hip_lib):
    q = torch.zeros(1, 1, 8, 64)
    with pytest.raises(ValueError):
        hip_lib.attn_bwd(q, q, q, q, torch.zeros(1, 1, 8), q)   # CPU tensors


def test_fwd_dv_validation(hip_lib):
    """attn_fwd_dv: Dv == D is attn_fwd's checks; Dv != D is fp32 only, with v
    and o sized by Dv."""
    L = hip_lib.lib()
    P = [A, A + SZ, A + 2 * SZ, A + 3 * SZ, A + 4 * SZ]

    def dv(*, ptrs=P, B=2, H=3, M=100, N=70, D=64, Dv=128, scale=0.125, causal=0, dtype=FP32):
        return L.attn_fwd_dv_validate(*ptrs, B, H, M, N, D, Dv, scale, causal, dtype)
    assert dv() == OK
    assert dv(D=128, Dv=16) == OK
    assert dv(Dv=64, dtype=BF16) == OK                 # equal dims: any dtype
    assert dv(dtype=BF16) == OK                        # every pair in 16 bits too
    assert dv(D=128, Dv=16, dtype=FP16) == OK
    assert dv(D=32, Dv=96, dtype=BF16) == UNSUPPORTED
    assert dv(Dv=48) == UNSUPPORTED
    assert dv(Dv=0) == INVALID
    assert dv(N=0) == INVALID
    assert dv(ptrs=[P[0], P[1], 0, P[3], P[4]]) == INVALID
    assert dv(ptrs=[P[0], P[1], P[2] + 8, P[3], P[4]]) == MISALIGNED
    assert dv(B=0, ptrs=[0] * 5) == OK
    # o overlapping the end of v: v is B*H*N*Dv*4 bytes
    vbytes = 2 * 3 * 70 * 128 * 4
    assert dv(ptrs=[P[0], P[1], P[2], P[2] + vbytes - 16, P[4]]) == INVALID
    assert dv(ptrs=[P[0], P[1], P[2], P[2] + vbytes, P[4]]) == OK


def test_bwd_noalloc_checks_before_any_hip_call(hip_lib):
    """attn_bwd_noalloc: attn_bwd's argument checks, then the scratch capacity
    (B*H*M <= MI355_ATTN_NOALLOC_MAX_ROWS), all before any HIP call (stand-in
    addresses, never dereferenced)."""
    L = hip_lib.lib()
    sz = 1 << 36
    q, k, v, o, lse, g, dq, dk, dv = ((i + 1) * sz for i in range(9))
    cap = hip_lib.MI355_ATTN_NOALLOC_MAX_ROWS
    assert cap == 1 << 20

    def call(B, H, M, N, D=128, dtype=BF16, **kw):
        p = dict(q=q, k=k, v=v, o=o, lse=lse, g=g, dq=dq, dk=dk, dv=dv)
        p.update(kw)
        return L.attn_bwd_noalloc(p["q"], p["k"], p["v"], p["o"], p["lse"], p["g"], p["dq"],
                                  p["dk"], p["dv"], B, H, M, N, D, 0.1, 0, dtype, None)

    assert call(4, 32, 8193, 64) == 5            # 4*32*8193 rows > 2^20
    assert call(1, 1, cap + 1, 64) == 5
    assert call(0, 4, 5, 5) == OK                # nothing to do
    assert call(1, 1, 5, 5, dq=None) == INVALID
    assert call(1, 1, 5, 5, D=16) == UNSUPPORTED
    assert call(1, 1, 5, 5, dtype=FP32) == UNSUPPORTED
    assert call(1, 1, 5, 5, dq=dq + 2) == MISALIGNED
    assert call(1, 1, 5, 5, dq=q) == INVALID     # output overlaps an input
    # the capacity check comes after attn_bwd's own checks
    assert call(1, 1, cap + 1, 64, dq=None) == INVALID


def test_fp8_validation_before_any_hip_call(hip_lib):
    """attn_fwd_fp8_validate: e4m3 q/k, transposed e4m3 v, bf16 o, fp32 lse;
    D in {64, 128}, N a multiple of 16; the usual pointer, alignment and
    overlap rules (stand-in addresses, never dereferenced)."""
    sz = 1 << 36
    q, k, vt, o, lse = ((i + 1) * sz for i in range(5))

    def v(B=4, H=16, M=4096, N=4096, D=128, scale=0.088, causal=0, **kw):
        p = dict(q=q, k=k, vt=vt, o=o, lse=lse)
        p.update(kw)
        return hip_lib.attn_fwd_fp8_validate(p["q"], p["k"], p["vt"], p["o"], p["lse"], B, H, M,
                                             N, D, scale, causal)

    assert v() == OK
    assert v(D=64, N=16, M=1) == OK
    assert v(B=0) == OK and v(M=0) == OK            # nothing to do
    assert v(D=32) == UNSUPPORTED and v(D=96) == UNSUPPORTED
    assert v(N=4000 + 8) == UNSUPPORTED             # N % 16 != 0
    assert v(N=0) == INVALID
    assert v(q=None) == INVALID and v(vt=None) == INVALID and v(lse=None) == INVALID
    assert v(scale=float("inf")) == INVALID and v(causal=2) == INVALID
    assert v(o=o + 8) == MISALIGNED and v(vt=vt + 4) == MISALIGNED and v(lse=lse + 2) == MISALIGNED
    assert v(o=q) == INVALID                          # output over an input
    assert v(lse=o + 1024) == INVALID                 # lse inside o


def test_bwd_work_bytes(hip_lib):
    """The one-pass backward's work area: header (256 B), one int counter per
    (head, 32-query tile, 32-wide d block), one fp32 L log2(e) per row (each
    rounded up to 256 B), fp32 dQ sums; 0 wherever the path does not apply."""
    wb = hip_lib.attn_bwd_work_bytes
    up = lambda x: -(-x // 256) * 256
    for B, H, M, N in [(4, 16, 4096, 4096), (1, 8, 1, 1), (2, 4, 33, 257), (1, 8, 300, 600)]:
        counters = up(B * H * (-(-M // 32)) * 16)
        assert wb(B, H, M, N, 128, False, BF16) == (256 + counters + up(B * H * M * 4)
                                                     + B * H * M * 128 * 4)
        assert wb(B, H, M, N, 128, False, FP16) == wb(B, H, M, N, 128, False, BF16)
    assert wb(4, 16, 4096, 4096, 128, True, BF16) == 0      # causal
    assert wb(4, 16, 4096, 4096, 64, False, BF16) == 0      # D != 128
    assert wb(1, 6, 100, 100, 128, False, BF16) > 0         # any B*H (padded to the XCDs)
    assert wb(1, 8, 100, 100, 128, False, FP32) == 0
    assert wb(1, 8, 0, 100, 128, False, BF16) == 0          # nothing to do
    assert wb(1, 8, 100, 0, 128, False, BF16) == 0
    assert wb(-1, 8, 100, 100, 128, False, BF16) == 0
    # size limits: B*H*M <= 2^30, M and N <= 2^24, at most 2^26 query tiles
    assert wb(1, 1 << 6, 1 << 24, 1, 128, False, BF16) > 0
    assert wb(1, (1 << 6) + 1, 1 << 24, 1, 128, False, BF16) == 0
    assert wb(1, 1, (1 << 24) + 1, 1, 128, False, BF16) == 0
    assert wb(1, 1, 1, (1 << 24) + 1, 128, False, BF16) == 0
    assert wb(1, 1 << 26, 1, 1, 128, False, BF16) > 0
    assert wb(1, (1 << 26) + 1, 1, 1, 128, False, BF16) == 0
    assert hip_lib.attn_bwd_work_error_offset() == 32


def test_bwd_ws_checks_the_work_area_before_any_hip_call(hip_lib):
    """attn_bwd_ws validates like attn_bwd, then refuses a misaligned or
    overlapping work area (fake addresses: nothing is dereferenced)."""
    lib = hip_lib.lib()
    B, H, M, N, D = 1, 8, 64, 64, 128
    qb, kb = B * H * M * D * 2, B * H * N * D * 2
    base = 1 << 40
    p = [base + i * (1 << 28) for i in range(10)]  # q k v o lse dout dq dk dv delta
    need = hip_lib.attn_bwd_work_bytes(B, H, M, N, D, False, BF16)
    work = base + 12 * (1 << 28)

    def call(w, nbytes, causal=0, scale=0.125):
        return lib.attn_bwd_ws(*p, B, H, M, N, D, scale, causal, BF16, w, nbytes, None)

    assert call(work + 16, need) == MISALIGNED
    assert call(p[6] + 256, need) == INVALID      # overlaps dq
    assert call(p[0], need) == INVALID            # overlaps q
    assert call(work, -1) == INVALID
    assert call(work, need, scale=float("nan")) == INVALID   # attn_bwd's own checks first
    assert lib.attn_bwd_ws(*p[:9], None, B, H, M, N, D, 0.125, 0, BF16, work, need,
                           None) == INVALID
