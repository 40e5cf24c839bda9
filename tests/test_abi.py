"""The C-ABI library loads on the host and exports what include/mcs.h declares.

No kernel is launched here: the only calls made are the pure host functions
(version, status strings, workspace queries) and calls whose arguments fail
validation, which the library rejects before touching HIP.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mcs.h")
LIB = os.path.join(ROOT, "token_sparse_attention_amd", "libmcs.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmcs.so not built")


def _header():
    with open(HEADER) as f:
        return f.read()


def _declared():
    return re.findall(r"MCS_API\s+[\w\s\*]+?\b(mcs_\w+)\s*\(", _header())


def _status_codes():
    return {m[0]: int(m[1]) for m in re.findall(r"(MCS_\w+)\s*=\s*(\d+)", _header())}


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32), ("D", ctypes.c_int32)]


@pytest.fixture(scope="module")
def lib():
    lib = ctypes.CDLL(LIB)
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    lib.mcs_dense_attn.argtypes = [P, P, P, P, P, Dims, F, P]
    lib.mcs_sparse_attn.argtypes = [P, P, P, P, P, P, P, Dims, I32, I32, F, P]
    lib.mcs_dense_attn_f32out.argtypes = [P, P, P, P, P, Dims, F, P]
    lib.mcs_sparse_attn_f32out.argtypes = [P, P, P, P, P, P, P, Dims, I32, I32, F, P]
    lib.mcs_residual_update.argtypes = [P, P, P, I64, P]
    lib.mcs_select.argtypes = [P, P, P, P, P, Dims, I32, I32, F, P, SZ, P]
    lib.mcs_select_two_pass.argtypes = [P, P, P, P, P, Dims, I32, I32, F, P, SZ, P]
    lib.mcs_topk.argtypes = [P, P, I64, I32, I32, P]
    lib.mcs_group.argtypes = [P, P, Dims, I32, I32, P, SZ, P]
    lib.mcs_group_noalloc.argtypes = [P, P, Dims, I32, I32, P]
    lib.mcs_group_workspace.argtypes = [Dims, I32]
    lib.mcs_group_workspace.restype = SZ
    lib.mcs_select_workspace.argtypes = [Dims, I32, I32]
    lib.mcs_select_workspace.restype = SZ
    lib.mcs_select_workspace_all_heads.argtypes = [Dims, I32, I32]
    lib.mcs_select_workspace_all_heads.restype = SZ
    lib.mcs_sparse_attn_ex.argtypes = [P, P, P, P, P, P, P, P, I32, P, Dims, I32, I32, F, P]
    lib.mcs_select_blocks.argtypes = [P, P, P, P, P, Dims, I32, I32, F, P, SZ, P]
    lib.mcs_select_blocks_workspace.argtypes = [Dims]
    lib.mcs_select_blocks_workspace.restype = SZ
    lib.mcs_query_quality.argtypes = [P, P, P, P, P, P, P, Dims, P]
    lib.mcs_row_sums.argtypes = [P, P, I64, I64, P]
    lib.mcs_kmeans.argtypes = [P, P, I32, I32, I32, I32, P, P, P, P, P, SZ, P]
    lib.mcs_kmeans_workspace.argtypes = [I32, I32]
    lib.mcs_kmeans_workspace.restype = SZ
    lib.mcs_status_string.restype = ctypes.c_char_p
    lib.mcs_last_error.restype = ctypes.c_char_p
    return lib


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) == 23, names
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    ver = int(re.search(r"#define MCS_VERSION (\d+)", _header()).group(1))
    assert lib.mcs_version() == ver
    codes = _status_codes()
    assert codes["MCS_OK"] == 0
    seen = set()
    for name, v in codes.items():
        s = lib.mcs_status_string(v).decode()
        assert s and s != "unknown status", name
        seen.add(s)
    assert len(seen) == len(codes)
    assert lib.mcs_status_string(999).decode() == "unknown status"


# fake, 16-byte aligned, never dereferenced: every call below fails validation first
A, B_, C_, D_, E_ = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000


def _codes():
    return _status_codes()


def test_dense_validation(lib):
    c = _codes()
    d = Dims(1, 2, 100, 128)
    assert lib.mcs_dense_attn(None, B_, C_, D_, None, d, 0.1, None) == c["MCS_E_NULL"]
    assert b"q is NULL" in lib.mcs_last_error()
    assert lib.mcs_dense_attn(A + 2, B_, C_, D_, None, d, 0.1, None) == c["MCS_E_ALIGN"]
    assert lib.mcs_dense_attn(A, B_, C_, D_, E_ + 4, d, 0.1, None) == c["MCS_E_ALIGN"]
    assert lib.mcs_dense_attn(A, B_, C_, D_, None, Dims(1, 2, 100, 96), 0.1, None) == c["MCS_E_HEAD_DIM"]
    assert lib.mcs_dense_attn(A, B_, C_, D_, None, Dims(0, 2, 100, 64), 0.1, None) == c["MCS_E_SHAPE"]
    assert lib.mcs_dense_attn(A, B_, C_, D_, None, Dims(1, 1 << 16, 100, 64), 0.1, None) == c["MCS_E_SHAPE"]
    assert lib.mcs_dense_attn(A, B_, C_, D_, None, Dims(1, 40, 1 << 26, 64), 0.1, None) == c["MCS_E_SHAPE"]
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert lib.mcs_dense_attn(A, B_, C_, D_, None, d, bad, None) == c["MCS_E_SCALE"]
    assert lib.mcs_dense_attn_f32out(A, B_, C_, None, None, d, 0.1, None) == c["MCS_E_NULL"]
    assert b"mcs_dense_attn_f32out: o is NULL" in lib.mcs_last_error()


def test_sparse_validation(lib):
    c = _codes()
    d = Dims(1, 2, 100, 64)
    args = lambda **kw: [kw.get(k, v) for k, v in
                         dict(q=A, k=B_, v=C_, perm=D_, idx=E_, res=None, o=0x60000).items()]
    assert lib.mcs_sparse_attn(*args(perm=None), d, 64, 10, 0.1, None) == c["MCS_E_NULL"]
    assert lib.mcs_sparse_attn(*args(idx=None), d, 64, 10, 0.1, None) == c["MCS_E_NULL"]
    assert lib.mcs_sparse_attn(*args(res=0x70008), d, 64, 10, 0.1, None) == c["MCS_E_ALIGN"]
    assert lib.mcs_sparse_attn(*args(), d, 32, 10, 0.1, None) == c["MCS_E_GROUP_SIZE"]
    assert lib.mcs_sparse_attn(*args(), d, 64, 0, 0.1, None) == c["MCS_E_BUDGET"]
    assert lib.mcs_sparse_attn(*args(), d, 64, 101, 0.1, None) == c["MCS_E_BUDGET"]
    assert lib.mcs_sparse_attn(*args(), d, 64, 10, -0.1, None) == c["MCS_E_SCALE"]
    assert lib.mcs_sparse_attn_f32out(*args(o=0x60004), d, 64, 10, 0.1, None) == c["MCS_E_ALIGN"]


def test_select_group_topk_residual_validation(lib):
    c = _codes()
    d = Dims(1, 2, 1000, 128)
    need = lib.mcs_select_workspace(d, 128, 100)
    assert need == 8 * 1000 * 4
    assert lib.mcs_select_workspace_all_heads(d, 128, 100) == 2 * need
    assert lib.mcs_select(A, B_, C_, D_, E_, d, 128, 100, 0.1, None, need, None) == c["MCS_E_WORKSPACE"]
    assert lib.mcs_select(A, B_, C_, D_, E_, d, 128, 100, 0.1, 0x80000, need - 1, None) == c["MCS_E_WORKSPACE"]
    assert lib.mcs_select(A, B_, None, D_, E_, d, 128, 100, 0.1, 0x80000, need, None) == c["MCS_E_NULL"]
    for fn in (lib.mcs_select, lib.mcs_select_two_pass):
        assert fn(A, B_, C_, D_, E_, d, 128, 100, 0.1, 0x80000, need - 1, None) == c["MCS_E_WORKSPACE"]
        assert fn(A, B_, C_, None, E_, d, 128, 100, 0.1, 0x80000, need, None) == c["MCS_E_NULL"]
        assert fn(A, B_, C_, D_, E_, d, 100, 100, 0.1, 0x80000, need, None) == c["MCS_E_GROUP_SIZE"]
        assert fn(A, B_, C_, D_, E_, Dims(1, 2, 1000, 96), 128, 100, 0.1, 0x80000, need, None) == c["MCS_E_HEAD_DIM"]
        assert fn(A, B_, C_, D_, E_, d, 128, 1001, 0.1, 0x80000, need, None) == c["MCS_E_BUDGET"]
        assert fn(A, B_, C_, D_, E_, d, 128, 100, 0.1, 0x80004, need, None) == c["MCS_E_ALIGN"]
    gws = lib.mcs_group_workspace(d, 128)
    assert gws >= 2 * 2 * 1000 * 4
    assert lib.mcs_group(A, B_, d, 128, 0, 0x80000, gws - 1, None) == c["MCS_E_WORKSPACE"]
    assert lib.mcs_group(A, B_, d, 128, 65, 0x80000, gws, None) == c["MCS_E_ARG"]    # lanczos_steps <= 64
    assert lib.mcs_group(A, B_, d, 100, 0, 0x80000, gws, None) == c["MCS_E_GROUP_SIZE"]
    assert lib.mcs_group_workspace(Dims(1, 2, 1000, 128), 100) == 0
    assert lib.mcs_topk(A, B_, 0, 10, 5, None) == c["MCS_E_SHAPE"]
    assert lib.mcs_topk(A, B_, 3, 10, 11, None) == c["MCS_E_BUDGET"]
    assert lib.mcs_topk(None, B_, 3, 10, 5, None) == c["MCS_E_NULL"]
    assert lib.mcs_residual_update(A, B_, C_, 0, None) == c["MCS_E_SHAPE"]
    assert lib.mcs_residual_update(A, B_ + 8, C_, 10, None) == c["MCS_E_ALIGN"]


def test_group_noalloc_validation(lib):
    # every check runs on the host before the scratch is looked up, so none
    # of these needs a device
    c = _codes()
    d = Dims(1, 2, 1000, 128)
    assert lib.mcs_group_noalloc(None, B_, d, 128, 0, None) == c["MCS_E_NULL"]
    assert lib.mcs_group_noalloc(A + 4, B_, d, 128, 0, None) == c["MCS_E_ALIGN"]
    assert lib.mcs_group_noalloc(A, B_, Dims(1, 2, 1000, 96), 128, 0, None) == c["MCS_E_HEAD_DIM"]
    assert lib.mcs_group_noalloc(A, B_, d, 100, 0, None) == c["MCS_E_GROUP_SIZE"]
    assert lib.mcs_group_noalloc(A, B_, d, 128, 65, None) == c["MCS_E_ARG"]
    # one head of N = 8388607, D = 128 needs more workspace than the 64 MiB scratch
    big = Dims(1, 1, 8388607, 128)
    assert lib.mcs_group_workspace(big, 128) > 64 << 20
    assert lib.mcs_group_noalloc(A, B_, big, 128, 0, None) == c["MCS_E_WORKSPACE"]
    assert b"scratch" in lib.mcs_last_error()


def test_block_sparse_and_diagnostic_validation(lib):
    c = _codes()
    d = Dims(1, 2, 1000, 128)
    W = 0x80000
    # sparse attention with counts / LSE
    ex = lambda **kw: [kw.get(k, v) for k, v in dict(q=A, k=B_, v=C_, perm=D_, idx=E_, cnt=None, res=None,
                                                     o=0x60000, f32=0, lse=None).items()]
    assert lib.mcs_sparse_attn_ex(*ex(res=0x70000, lse=0x90000), d, 128, 64, 0.1, None) == c["MCS_E_ARG"]
    assert b"residual and lse" in lib.mcs_last_error()
    assert lib.mcs_sparse_attn_ex(*ex(cnt=0x90004), d, 128, 64, 0.1, None) == c["MCS_E_ALIGN"]
    assert lib.mcs_sparse_attn_ex(*ex(idx=None), d, 128, 64, 0.1, None) == c["MCS_E_NULL"]
    assert lib.mcs_sparse_attn_ex(*ex(), d, 128, 1001, 0.1, None) == c["MCS_E_BUDGET"]
    # block selection: K whole 64-key blocks, at most the head's block count
    need = lib.mcs_select_blocks_workspace(d)
    assert need == 2 * 16 * 128 * 4                       # fp32 mean key per block, ceil(1000 / 64) = 16
    assert lib.mcs_select_blocks_workspace(Dims(1, 2, 1000, 96)) == 0
    sb = lambda K, cnt=0x90000, ws=W, nb=need, dims=d: lib.mcs_select_blocks(A, B_, C_, D_, cnt, dims, 128, K, 0.1,
                                                                             ws, nb, None)
    for K in (0, 63, 100, 17 * 64):
        assert sb(K) == c["MCS_E_BUDGET"], K
    assert sb(128, cnt=None) == c["MCS_E_NULL"]
    assert sb(128, nb=need - 1) == c["MCS_E_WORKSPACE"]
    assert sb(128, ws=None) == c["MCS_E_WORKSPACE"]
    assert sb(128, ws=W + 8) == c["MCS_E_ALIGN"]
    big = Dims(1, 1, 4096 * 64 + 1, 64)                   # one key block more than the selector holds
    assert sb(128, dims=big, nb=1 << 40) == c["MCS_E_SHAPE"]
    # per-query recall and L1 terms; fixed-order row sums
    assert lib.mcs_query_quality(A, None, C_, D_, E_, 0x60000, 0x70000, d, None) == c["MCS_E_NULL"]
    assert lib.mcs_query_quality(A, B_, C_, D_, E_, 0x60000, 0x70000, Dims(1, 2, 1000, 96), None) == c["MCS_E_HEAD_DIM"]
    assert lib.mcs_row_sums(A, B_, 0, 10, None) == c["MCS_E_SHAPE"]
    assert lib.mcs_row_sums(A, B_, 3, 0, None) == c["MCS_E_SHAPE"]
    assert lib.mcs_row_sums(None, B_, 3, 10, None) == c["MCS_E_NULL"]
    # k-means
    kws = lib.mcs_kmeans_workspace(1000, 8)
    assert kws >= (1000 + 8) * 4
    assert lib.mcs_kmeans_workspace(0, 8) == 0
    km = lambda n=1000, D=128, k=8, rounds=20, ws=W, nb=kws: lib.mcs_kmeans(A, B_, n, D, k, rounds, C_, D_, E_,
                                                                          0x60000, ws, nb, None)
    assert km(D=96) == c["MCS_E_HEAD_DIM"]
    assert km(k=0) == c["MCS_E_ARG"] and km(k=1001) == c["MCS_E_ARG"]
    assert km(rounds=0) == c["MCS_E_ARG"]
    assert km(n=0) == c["MCS_E_SHAPE"] and km(n=1 << 24) == c["MCS_E_SHAPE"]   # n * D >= 2^31
    assert km(nb=kws - 1) == c["MCS_E_WORKSPACE"]
    assert km(ws=W + 4) == c["MCS_E_ALIGN"]


def test_group_workspace_grows_with_partials(lib):
    # large nodes near the root keep partial moments; small problems need none
    small = lib.mcs_group_workspace(Dims(1, 1, 1024, 64), 64)
    assert small >= 8 * 1024
    large = lib.mcs_group_workspace(Dims(1, 40, 75600, 128), 128)
    assert large > 8 * 40 * 75600 + 40 * 37 * (128 * 128 + 128) * 4


def test_layout_helpers_round_trip():
    import torch
    from token_sparse_attention_amd import binding
    x = torch.arange(2 * 5 * 3 * 4, dtype=torch.float32).reshape(2, 5, 3, 4)      # [B, N, H, D]
    y = binding.heads_major(x)
    assert y.shape == (2, 3, 5, 4) and y.is_contiguous()
    assert torch.equal(y[1, 2, 4], x[1, 4, 2])
    z = binding.tokens_major(y)
    assert z.is_contiguous() and torch.equal(z, x)


def test_header_is_plain_c_and_links(lib, tmp_path):
    """include/mcs.h is a C header: a C99 program includes it, links against
    the library and calls a host-only query (no GPU work)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    src = tmp_path / "use_mcs.c"
    src.write_text('#include "mcs.h"\n'
                   "int main(void) {\n"
                   "  mcs_dims d = {1, 2, 1000, 128};\n"
                   "  return mcs_select_workspace(d, 128, 100) == 8 * 1000 * 4 && mcs_version() == MCS_VERSION ? 0 : 1;\n"
                   "}\n")
    lib_dir = os.path.join(root, "token_sparse_attention_amd")
    exe = tmp_path / "use_mcs"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(root, "include"),
                    str(src), "-L", lib_dir, "-lmcs", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)], check=True)
    assert subprocess.run([str(exe)]).returncode == 0


def test_validation_under_address_and_ub_sanitizers(tmp_path):
    """The C-ABI layer (api.hip) built with ASan and UBSan on the host code and
    linked with host stand-ins for the launchers (tests/abi_sanitize): every
    entry point's checks and accepting path run clean on a machine without a
    GPU.  Sanitizers apply to the host code only (each -fsanitize= follows
    -Xarch_host)."""
    import shlex
    hipcc = "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    here = os.path.join(ROOT, "tests", "abi_sanitize")
    exe = str(tmp_path / "abi_sanitize")
    san = shlex.split("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                      "-Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer")
    cmd = [hipcc, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", *san, "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "token_sparse_attention_amd", "csrc", "api.hip"), os.path.join(here, "stubs.cpp"),
           os.path.join(here, "driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and "sanitize ok" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
