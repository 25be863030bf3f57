"""The C-ABI library loads, exports what include/trellis.h declares, and rejects bad
arguments before launching anything.  No GPU is needed: every call here fails validation
on the host (pointers are fake, never dereferenced)."""
import ctypes
import os

import pytest

from trellis_coded_bit_amd import binding as tb

EINVAL, EALIGN, EWORKSPACE, EUNSUPPORTED = -1, -2, -3, -4
RESERVED = 256 + 65536  # the reserved region at the start of every workspace


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tb.LIB_PATH):
        from trellis_coded_bit_amd import build
        build.build(verbose=False)
    return tb.lib()


def lin(**kw):
    d = dict(code=0x10000, rin=0x20000, rout=0x30000, s_in=0x40000, s_out=0x50000, K=2,
             in_features=512, out_features=256, cb=1)
    d.update(kw)
    return tb.CLinear(d["code"], d["rin"], d["rout"], d["s_in"], d["s_out"], d["K"], d["in_features"],
                      d["out_features"], d["cb"])


def test_exports_every_declared_symbol(L):
    names = tb.header_functions()
    assert set(names) >= {"trellis_decode_tiles", "had128_scale", "trellis_gemv", "trellis_gemm",
                          "trellis_moe_gemv", "trellis_workspace_bytes", "trellis_validate_table",
                          "trellis_last_error", "trellis_abi_version"}
    inc = os.path.dirname(tb.HEADER)
    headers = sorted(f for f in os.listdir(inc) if f.endswith(".h"))
    assert "trellis_micro.h" in headers
    for h in headers:
        declared = tb.header_functions(os.path.join(inc, h))
        assert declared, h
        for n in declared:
            assert hasattr(L, n), (h, n)
    assert L.trellis_abi_version() == 2


def test_micro_validation(L):
    """The microbenchmarks reject bad sizes and kinds before launching (fake pointers)."""
    assert L.trellis_micro_stream_read(0x10000, 8, 0, 0x20000, None) == EINVAL       # < 16 bytes
    assert L.trellis_micro_stream_read(0x10008, 64, 0, 0x20000, None) == EALIGN     # misaligned
    assert L.trellis_micro_stream_read(None, 64, 0, 0x20000, None) == EINVAL
    assert L.trellis_micro_valu(1, 0, 1, 0x10000, 0x20000, 0x30000, None) == EINVAL  # iters < 1
    assert L.trellis_micro_valu(1, 10, 9, 0x10000, 0x20000, 0x30000, None) == EINVAL  # waves/SIMD > 8
    assert L.trellis_micro_mfma(0, 10, 5, 0x10000, 0x20000, 0x30000, None) == EINVAL  # waves/SIMD > 4
    assert L.trellis_micro_mfma(0, 10, 1, 0x10004, 0x20000, 0x30000, None) == EALIGN


def test_workspace_bytes(L):
    c = lin()
    assert L.trellis_workspace_bytes(0, ctypes.byref(c), 1, 0) > 0
    assert L.trellis_workspace_bytes(0, ctypes.byref(c), 9, 0) == 0      # B out of range
    assert L.trellis_workspace_bytes(1, ctypes.byref(c), 2048, 0) >= 2048 * 512 * 2
    assert L.trellis_workspace_bytes(2, ctypes.byref(c), 1, 8) > 0
    assert L.trellis_workspace_bytes(7, ctypes.byref(c), 1, 0) == 0
    bad = lin(in_features=100)
    assert L.trellis_workspace_bytes(0, ctypes.byref(bad), 1, 0) == 0


@pytest.mark.parametrize("kw,B,status", [
    (dict(K=5), 1, EINVAL), (dict(K=1), 1, EINVAL), (dict(cb=0), 1, EINVAL),
    (dict(in_features=100), 1, EINVAL), (dict(out_features=0), 1, EINVAL),
    (dict(code=None), 1, EINVAL), (dict(rin=None), 1, EINVAL),
    (dict(code=0x10008), 1, EALIGN), (dict(s_in=0x40002), 1, EALIGN),
    (dict(), 0, EINVAL), (dict(), 9, EINVAL),
])
def test_gemv_validation(L, kw, B, status):
    c = lin(**kw)
    r = L.trellis_gemv(ctypes.byref(c), 0x60000, B, 0x70000, 0x80000, 1 << 30, None)
    assert r == status, L.trellis_last_error()
    assert L.trellis_last_error()


def test_gemv_workspace_checks(L):
    c = lin()
    need = L.trellis_workspace_bytes(0, ctypes.byref(c), 1, 0)
    assert L.trellis_gemv(ctypes.byref(c), 0x60000, 1, 0x70000, 0x80000, need - 1, None) == EWORKSPACE
    assert L.trellis_gemv(ctypes.byref(c), 0x60000, 1, 0x70000, None, need, None) == EWORKSPACE
    assert L.trellis_gemv(ctypes.byref(c), 0x60000, 1, 0x70000, 0x80010, need, None) == EWORKSPACE
    assert L.trellis_gemv(ctypes.byref(c), None, 1, 0x70000, 0x80000, need, None) == EINVAL


def test_every_workspace_starts_with_the_reserved_region(L):
    """Every entry point's workspace is at least the reserved region (error word + the
    small-batch counters) plus its own scratch, which lies after that region."""
    c = lin()
    for op, n in ((0, 1), (1, 64), (2, 8), (3, 64)):
        cc = lin(cb=2) if op == 3 else c
        assert L.trellis_workspace_bytes(op, ctypes.byref(cc), n if op != 2 else 1, 8) > RESERVED
    assert L.trellis_workspace_bytes(1, ctypes.byref(c), 64, 0) >= RESERVED + 64 * 512 * 2


def _items(*specs):
    """(layer kwargs, x address, y address) -> a ctypes array of trellis_gemv_item."""
    arr = (tb.CGemvItem * len(specs))()
    for i, (kw, x, y) in enumerate(specs):
        arr[i].L = lin(**kw)
        arr[i].x = x
        arr[i].y = y
    return arr


def test_gemv_list_validation(L):
    ok = _items((dict(), 0x100000, 0x200000), (dict(K=3, in_features=1024, out_features=384), 0x300000, 0x400000))
    need = L.trellis_gemv_list_workspace_bytes(ok, 2, 2)
    assert need > RESERVED
    # the list needs at least as much as each of its items alone
    assert need >= L.trellis_workspace_bytes(0, ctypes.byref(lin()), 2, 0) - RESERVED
    call = lambda items, n, B, nb=need, ws=0x8000000: L.trellis_gemv_list(items, n, B, ws, nb, None)
    assert call(ok, 0, 1) == EINVAL
    assert call(ok, 9, 1) == EINVAL
    assert call(ok, 2, 0) == EINVAL and call(ok, 2, 9) == EINVAL
    assert call(None, 1, 1) == EINVAL
    assert call(ok, 2, 2, need - 1) == EWORKSPACE
    assert call(ok, 2, 2, need, 0x8000010) == EWORKSPACE       # workspace not 256-byte aligned
    bad = _items((dict(), 0x100000, 0x200000), (dict(K=5), 0x300000, 0x400000))
    assert call(bad, 2, 1) == EINVAL and b"item 1" in L.trellis_last_error()
    assert L.trellis_gemv_list_workspace_bytes(bad, 2, 1) == 0
    # outputs may not overlap each other, nor any input
    y_y = _items((dict(), 0x100000, 0x200000), (dict(), 0x300000, 0x200100))
    assert call(y_y, 2, 1) == EINVAL and b"overlap" in L.trellis_last_error()
    y_x = _items((dict(), 0x100000, 0x200000), (dict(), 0x2000F0, 0x400000))
    assert call(y_x, 2, 1) == EINVAL and b"overlaps" in L.trellis_last_error()
    own = _items((dict(), 0x100000, 0x1001F0),)  # y inside its own x
    assert call(own, 1, 1) == EINVAL
    nul = _items((dict(), None, 0x200000),)
    assert call(nul, 1, 1) == EINVAL
    mis = _items((dict(), 0x100001, 0x200000),)
    assert call(mis, 1, 1) == EALIGN
    # more output column blocks than the counter region holds: valid, but not supported
    wide = _items((dict(in_features=128, out_features=128 * 16385), 0x100000, 0x10000000),)
    assert L.trellis_gemv_list_workspace_bytes(wide, 1, 1) == 0
    assert call(wide, 1, 1, 1 << 40) == EUNSUPPORTED


def test_gemm_validation(L):
    c = lin()
    need = L.trellis_workspace_bytes(1, ctypes.byref(c), 64, 0)
    assert L.trellis_gemm(ctypes.byref(c), 0x60000, -1, 0x70000, 0x80000, need, None) == EINVAL
    assert L.trellis_gemm(ctypes.byref(c), 0x60000, 0, 0x70000, 0x80000, need, None) == 0  # no-op
    assert L.trellis_gemm(ctypes.byref(c), 0x60008, 64, 0x70000, 0x80000, need, None) == EALIGN
    assert L.trellis_gemm(ctypes.byref(c), 0x60000, 64, 0x70000, 0x80000, need - 256, None) == EWORKSPACE


def test_decode_and_hadamard_validation(L):
    assert L.trellis_decode_tiles(0x10000, 5, 512, 256, 0x20000, None, None) == EINVAL
    assert L.trellis_decode_tiles(0x10000, 2, 40, 256, 0x20000, None, None) == EINVAL
    assert L.trellis_decode_tiles(0x10002, 2, 512, 256, 0x20000, None, None) == EALIGN
    assert L.trellis_decode_tiles(0x10000, 2, 0, 256, 0x20000, None, None) == 0  # empty
    assert L.trellis_decode_tiles(None, 2, 512, 256, 0x20000, None, None) == EINVAL
    assert L.had128_scale(0x10000, 0, 4, 100, None, None, 0, 0x20000, 0, None) == EINVAL
    assert L.had128_scale(0x10000, 0, 4, 128, None, None, 2, 0x20000, 0, None) == EINVAL
    assert L.had128_scale(0x10000, 0, 4, 128, None, None, 0, 0x10080, 0, None) == EINVAL  # partial overlap
    assert L.had128_scale(0x10000, 1, 4, 128, None, None, 0, 0x10000, 0, None) == EINVAL  # in place, mixed types
    assert L.had128_scale(0x10001, 0, 4, 128, None, None, 0, 0x20000, 0, None) == EALIGN
    assert L.had128_scale(0x10000, 0, 0, 128, None, None, 0, 0x20000, 0, None) == 0


def test_moe_validation_and_table(L):
    probe = lin(in_features=6144, out_features=2048)
    need = L.trellis_workspace_bytes(2, ctypes.byref(probe), 1, 8)
    args = dict(E=4, routed=0x90000, n=8, i=6144, o=2048, x=0x60000, xpe=0, sr=0xA0000, ss=None, side=0,
                y=0x70000, ws=0x80000, nb=need)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return L.trellis_moe_gemv(0x10000, a["E"], a["routed"], a["n"], a["i"], a["o"], a["x"], a["xpe"],
                                  a["sr"], a["ss"], a["side"], a["y"], a["ws"], a["nb"], None)

    assert call(side=2) == EINVAL
    assert call(side=0, sr=None) == EINVAL
    assert call(E=0) == EINVAL
    assert call(i=6000) == EINVAL
    assert call(xpe=2) == EINVAL
    assert call(nb=need - 1) == EWORKSPACE
    assert call(n=0) == 0
    table = (tb.CLinear * 4)(*[lin(in_features=6144, out_features=2048, K=k) for k in (2, 3, 4, 2)])
    assert L.trellis_validate_table(table, 4, 6144, 2048, -1) == 0
    table[3].K = 7
    assert L.trellis_validate_table(table, 4, 6144, 2048, -1) == EINVAL
    assert b"entry 3" in L.trellis_last_error()
    table[3].K = 2
    table[1].rin = None
    assert L.trellis_validate_table(table, 4, 6144, 2048, -1) == EINVAL
    assert L.trellis_validate_table(table, 4, 6144, 2048, 0) == 0  # input side shared
    table[2].out_features = 4096
    assert L.trellis_validate_table(table, 4, 6144, 2048, 0) == EINVAL


def test_moe_mlp_workspace_bytes(L):
    f = L.trellis_moe_mlp_workspace_bytes
    assert f(6144, 2048, 16, 8) > 8 * 2048 * 2
    assert f(6144, 2048, 1, 8) > 8 * 2048 * 2
    assert f(6144, 2048, 16, 0) == RESERVED
    assert f(100, 2048, 16, 8) == 0          # hidden not a multiple of 128
    assert f(6144, 2048, 3, 8) == 0          # inter not a multiple of 128 * halves
    assert f(6144, 2048, 0, 8) == 0
    assert f(6144, 2048, 16, -1) == 0


def _mlp_call(L, **kw):
    a = dict(gate_up=0x10000, down=0x20000, E=4, halves=2, routed=0x30000, router_w=0x31000, n=2,
             hidden=256, inter=256, x=0x40000, r_hi=0x50000, s_hi=0x51000, r_ho=0x52000, s_ho=0x53000,
             act=None, y=0x60000, ws=0x70000, ws_bytes=1 << 30)
    a.update(kw)
    return L.trellis_moe_mlp(a["gate_up"], a["down"], a["E"], a["halves"], a["routed"], a["router_w"], a["n"],
                             a["hidden"], a["inter"], a["x"], a["r_hi"], a["s_hi"], a["r_ho"], a["s_ho"],
                             a["act"], a["y"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(E=0), EINVAL), (dict(gate_up=None), EINVAL), (dict(down=None), EINVAL),
    (dict(halves=0), EINVAL), (dict(n=-1), EINVAL), (dict(hidden=200), EINVAL),
    (dict(inter=384), EINVAL),                      # 384 is not a multiple of 128 * 2
    (dict(y=None), EINVAL), (dict(r_ho=None), EINVAL), (dict(routed=None), EINVAL),
    (dict(router_w=None), EINVAL), (dict(x=None), EINVAL), (dict(r_hi=None), EINVAL),
    (dict(router_w=0x31002), EALIGN), (dict(gate_up=0x10004), EALIGN), (dict(act=0x80001), EALIGN),
    (dict(s_ho=0x53002), EALIGN),
    (dict(ws_bytes=255), EWORKSPACE), (dict(ws=None), EWORKSPACE), (dict(ws=0x70010), EWORKSPACE),
])
def test_moe_mlp_validation(L, kw, status):
    assert _mlp_call(L, **kw) == status, L.trellis_last_error()
    assert L.trellis_last_error()


def test_fp8_entry_validation(L):
    c1, c2 = lin(), lin(cb=2)
    need = L.trellis_workspace_bytes(3, ctypes.byref(c2), 64, 0)
    assert need >= 64 * 512
    assert L.trellis_gemm_fp8(ctypes.byref(c1), 0x60000, 64, 0x70000, 0x80000, need, None) == EINVAL  # cb=1
    assert L.trellis_gemm_fp8(ctypes.byref(c2), 0x60000, -1, 0x70000, 0x80000, need, None) == EINVAL
    assert L.trellis_gemm_fp8(ctypes.byref(c2), 0x60000, 0, 0x70000, 0x80000, need, None) == 0  # no-op
    assert L.trellis_gemm_fp8(ctypes.byref(c2), 0x60008, 64, 0x70000, 0x80000, need, None) == EALIGN
    assert L.trellis_gemm_fp8(ctypes.byref(c2), 0x60000, 64, 0x70000, 0x80000, need - 256, None) == EWORKSPACE
    assert L.trellis_gemm_fp8(ctypes.byref(lin(cb=3)), 0x60000, 64, 0x70000, 0x80000, need, None) == EINVAL
    # an unknown codebook is rejected by every product
    c3 = lin(cb=3)
    assert L.trellis_gemv(ctypes.byref(c3), 0x60000, 1, 0x70000, 0x80000, 1 << 30, None) == EINVAL
    assert L.trellis_gemm(ctypes.byref(c3), 0x60000, 64, 0x70000, 0x80000, 1 << 30, None) == EINVAL
    # decode to E4M3 bytes
    f = L.trellis_decode_tiles_e4m3
    assert f(0x10000, 5, 64, 64, 0x20000, None) == EINVAL
    assert f(0x10000, 2, 60, 64, 0x20000, None) == EINVAL
    assert f(0x10000, 2, 0, 64, 0x20000, None) == 0
    assert f(0x10008, 2, 64, 64, 0x20000, None) == EALIGN
    assert f(0x10000, 2, 64, 64, 0x20008, None) == EALIGN
    assert f(0x10000, 2, 64, 64, None, None) == EINVAL


def test_encode_validation(L):
    f = L.trellis_encode_tiles
    need = L.trellis_encode_workspace_bytes(4)
    assert need >= 4 * (1 << 20) and L.trellis_encode_workspace_bytes(-1) == 0
    ok = dict(t=0x10000, T=4, K=2, cb=1, code=0x20000, st=None, ws=0x100000, nb=need)
    call = lambda **kw: f(*[{**ok, **kw}[k] for k in ("t", "T", "K", "cb", "code", "st", "ws", "nb")], None)
    assert call(K=5) == EINVAL and call(K=1) == EINVAL
    assert call(cb=0) == EINVAL and call(cb=3) == EINVAL
    assert call(T=-1) == EINVAL
    assert call(T=0) == 0
    assert call(t=None) == EINVAL and call(code=None) == EINVAL
    assert call(t=0x10002) == EALIGN and call(code=0x20002) == EALIGN and call(st=0x30001) == EALIGN
    assert call(nb=need - 1) == EWORKSPACE and call(ws=None) == EWORKSPACE and call(ws=0x100010) == EWORKSPACE


def test_abi_layer_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    """csrc/api.cpp (the C-ABI layer: validation, error strings, marshalling) built with the
    host compiler under AddressSanitizer and UndefinedBehaviorSanitizer, warnings as errors,
    against stub launchers (tests/sanitize/abi_driver.cpp), and every entry point called
    with good and bad arguments: no sanitizer report, every expectation met."""
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    exe = str(tmp_path / "abi_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-Werror", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           os.path.join(root, "trellis_coded_bit_amd", "csrc", "api.cpp"),
           os.path.join(root, "tests", "sanitize", "abi_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "failures 0" in r.stdout
