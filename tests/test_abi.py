"""C ABI checks that need no GPU: the library loads, exports what the header
declares, sizes follow the packed format, and every argument error is caught
on the host before any HIP call (fake pointers are never dereferenced)."""
import ctypes
import os
import re

import numpy as np
import pytest

import structured_sparse_gemm_nm_amd as nm
from oracle import nm_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nmsparse.h")

pytestmark = pytest.mark.skipif(not os.path.exists(nm.lib_path()),
                                reason="libnmsparse.so not built")


def header_text():
    with open(HEADER) as f:
        return f.read()


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", header_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(nm_[a-z_]+)\s*\(", text)))


def header_enum(name):
    text = header_text()
    return int(re.search(rf"\b{name}\s*=\s*(\d+)", text).group(1))


def test_exports_every_declared_symbol():
    L = nm.lib()
    names = declared_functions()
    assert {"nm_compress", "nm_spmm", "nm_spmm_perm", "nm_decompress", "nm_packed_sizes"} <= set(names)
    for name in names:
        assert hasattr(L, name), name
    assert L.nm_version() == 102


def test_status_codes_match_header():
    for name, val in (("NM_OK", 0), ("NM_ERR_NULL", 1), ("NM_ERR_SHAPE", 2),
                      ("NM_ERR_UNSUPPORTED", 3), ("NM_ERR_STRIDE", 4), ("NM_ERR_ALIAS", 5),
                      ("NM_ERR_HIP", 6), ("NM_ERR_ALIGN", 7)):
        assert header_enum(name) == val
        assert nm.lib().nm_status_string(val).decode() == name
    assert header_enum("NM_F16") == nm.NM_F16 and header_enum("NM_BF16") == nm.NM_BF16
    assert header_enum("NM_F32") == nm.NM_F32


@pytest.mark.parametrize("n,m", nm.PATTERNS)
@pytest.mark.parametrize("R,K", [(1, 16), (7, 48), (256, 256), (4096, 4096), (11008, 4096),
                                 (3072, 768), (5, 1040)])
def test_packed_sizes_match_oracle(R, K, n, m):
    if K % m:
        pytest.skip("K not a multiple of m")
    vb, ib, words = nm.nm_packed_sizes(R, K, n, m, nm.NM_F16)
    assert words == O.idx_words_per_row(K, n, m)
    assert vb == R * O.survivors_per_row(K, n, m) * 2
    assert ib == R * words * 4


def test_packed_sizes_36_bits_per_group():
    # one FP16 2:4 group costs 36 bits when rows fill whole index words
    vb, ib, _ = nm.nm_packed_sizes(256, 256, 2, 4, nm.NM_F16)
    assert (vb + ib) * 8 == 256 * (256 // 4) * 36
    assert vb + ib == 73728


FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation first


def st_compress(W=FAKE, R=4, K=64, ldw=64, dt=nm.NM_F16, n=2, m=4, v=FAKE * 2, i=FAKE * 3):
    return nm.lib().nm_compress(W, R, K, ldw, dt, n, m, v, i, None)


def st_spmm(values=FAKE, idx=FAKE * 2, R=32, K=64, n=2, m=4, dt=nm.NM_F16, act=FAKE * 3, T=8,
            ldx=64, Y=FAKE * 4, ldy=32, od=nm.NM_F32, perm=None):
    L = nm.lib()
    if perm is None:
        return L.nm_spmm(values, idx, R, K, n, m, dt, act, T, ldx, Y, ldy, od, None)
    return L.nm_spmm_perm(values, idx, R, K, n, m, dt, act, T, ldx, perm, Y, ldy, od, None)


def test_compress_errors():
    assert st_compress(W=None) == 1
    assert st_compress(v=None) == 1
    assert st_compress(K=15, ldw=16) == 2
    assert st_compress(K=20, ldw=24) == 2          # K % 16
    assert st_compress(K=0) == 2
    assert st_compress(R=-1) == 2
    assert st_compress(n=3, m=4) == 3
    assert st_compress(n=2, m=8) == 3
    assert st_compress(dt=nm.NM_F32) == 3
    assert st_compress(dt=9) == 3
    assert st_compress(ldw=48) == 4
    assert st_compress(ldw=68) == 7                # ldw % 8
    assert st_compress(W=FAKE + 2) == 7            # misaligned pointer
    assert st_compress(v=FAKE + 8) == 7
    # values overlapping W
    assert st_compress(v=FAKE + 64) == 5
    assert "NM_ERR_ALIAS" in nm.lib().nm_last_error().decode()
    # empty input is a no-op that touches nothing
    assert st_compress(W=None, v=None, i=None, R=0) == 0


def test_spmm_errors():
    assert st_spmm(values=None) == 1
    assert st_spmm(act=None) == 1
    assert st_spmm(Y=None) == 1
    assert st_spmm(perm=0) == 1                    # nm_spmm_perm with NULL perm
    assert st_spmm(K=40, ldx=40) == 2              # K % 16
    assert st_spmm(K=8, ldx=8) == 2
    assert st_spmm(T=-1) == 2
    assert st_spmm(n=1, m=2) == 3
    assert st_spmm(dt=nm.NM_F16, od=nm.NM_BF16) == 3
    assert st_spmm(dt=nm.NM_F32) == 3
    assert st_spmm(ldx=32) == 4
    assert st_spmm(ldy=16) == 4
    assert st_spmm(ldx=68) == 7
    assert st_spmm(ldy=34, Y=None) == 1            # any ldy >= R is accepted
    assert st_spmm(act=FAKE * 3 + 4) == 7
    assert st_spmm(Y=FAKE * 4 + 8) == 7
    assert st_spmm(perm=FAKE * 5 + 4) == 7
    # Y overlapping act / values / idx / perm
    assert st_spmm(Y=FAKE * 3 + 16) == 5
    assert st_spmm(Y=FAKE + 32) == 5
    assert st_spmm(Y=FAKE * 2) == 5
    assert st_spmm(perm=FAKE * 4 + 64) == 5
    # empty products are no-ops
    assert st_spmm(T=0, values=None, idx=None, act=None, Y=None) == 0
    assert st_spmm(R=0, values=None, idx=None, act=None, Y=None, ldy=0) == 0
    assert nm.lib().nm_last_error().decode() == ""


def test_int8_sizes_and_rules():
    # 20 bits per INT8 2:4 group (one byte per value, 2 index bits each);
    # the reduction length must be a multiple of 32 (COE-592 lecture 04-2,
    # "M:N sparsity on NVIDIA tensor cores", section "Where this sits among
    # the three case studies")
    vb, ib, words = nm.nm_packed_sizes(4096, 4096, 2, 4, nm.NM_I8)
    assert (vb + ib) * 8 == 4096 * (4096 // 4) * 20
    assert vb == 4096 * 2048 and words == 4096 // 32
    L = nm.lib()
    st = lambda K, n=2, m=4: L.nm_packed_sizes(8, K, n, m, nm.NM_I8, None, None, None)
    assert st(64) == 0 and st(32) == 0
    assert st(48) == 2                             # K % 32 for int8
    assert st(64, 1, 4) == 3 and st(64, 1, 8) == 3  # int8 takes 2:4 only
    # compress: int8 rows must be 16-byte aligned (ldw % 16)
    assert st_compress(dt=nm.NM_I8, ldw=72) == 7
    assert st_compress(dt=nm.NM_I8, K=48, ldw=48) == 2
    assert st_compress(dt=nm.NM_I8, n=1, m=8) == 3
    # spmm: int32 output only, no permuted form, ldx % 16
    assert st_spmm(dt=nm.NM_I8, od=nm.NM_F32) == 3
    assert st_spmm(dt=nm.NM_I8, od=nm.NM_I8) == 3
    assert st_spmm(dt=nm.NM_I8, od=nm.NM_I32, perm=FAKE * 5) == 3
    assert st_spmm(dt=nm.NM_I8, od=nm.NM_I32, ldx=72) == 7
    assert st_spmm(dt=nm.NM_I8, od=nm.NM_I32, K=96, ldx=96, values=None) == 1
    assert st_spmm(dt=nm.NM_I8, od=nm.NM_I32, K=80, ldx=80) == 2
    # NM_I32 is an output type only
    assert st_spmm(dt=nm.NM_I32, od=nm.NM_I32) == 3
    # Y (int32) overlapping act (int8)
    assert st_spmm(dt=nm.NM_I8, od=nm.NM_I32, Y=FAKE * 3 + 16) == 5


def test_fp8_sizes_and_rules():
    # E4M3 takes the one-byte layout and every 8-bit rule; its output is fp32
    assert header_enum("NM_FP8") == nm.NM_FP8 == 5
    assert nm.nm_packed_sizes(4096, 4096, 2, 4, nm.NM_FP8) == nm.nm_packed_sizes(4096, 4096, 2, 4, nm.NM_I8)
    L = nm.lib()
    st = lambda K, n=2, m=4: L.nm_packed_sizes(8, K, n, m, nm.NM_FP8, None, None, None)
    assert st(64) == 0 and st(48) == 2 and st(64, 1, 4) == 3
    assert st_compress(dt=nm.NM_FP8, ldw=72) == 7
    assert st_compress(dt=nm.NM_FP8, K=48, ldw=48) == 2
    assert st_spmm(dt=nm.NM_FP8, od=nm.NM_I32) == 3
    assert st_spmm(dt=nm.NM_FP8, od=nm.NM_FP8) == 3
    assert st_spmm(dt=nm.NM_FP8, od=nm.NM_F32, perm=FAKE * 5) == 3
    assert st_spmm(dt=nm.NM_FP8, od=nm.NM_F32, ldx=72) == 7
    assert st_spmm(dt=nm.NM_FP8, od=nm.NM_F32, K=96, ldx=96, values=None) == 1
    assert st_spmm(dt=nm.NM_FP8, od=nm.NM_F32, Y=FAKE * 3 + 16) == 5


def test_fp8_inputs_are_e4m3_patterns():
    import nm_inputs
    b = nm_inputs.normal_fp8((64, 256), 1.0, 7, 0)
    assert b.dtype == np.uint8 and b.shape == (64, 256)
    v = O.fp8_to_f64(b)
    assert np.all(np.isfinite(v)) and np.abs(v).max() <= 448.0
    assert np.array_equal(b, nm_inputs.normal_fp8((64, 256), 1.0, 7, 0))  # seeded


def test_decompress_and_misc_errors():
    L = nm.lib()
    assert L.nm_decompress(None, FAKE, 4, 64, 2, 4, nm.NM_F16, FAKE * 2, 64, None) == 1
    assert L.nm_decompress(FAKE, FAKE * 2, 4, 64, 2, 4, nm.NM_F16, FAKE * 3, 32, None) == 4
    assert L.nm_decompress(FAKE, FAKE * 2, 4, 64, 2, 4, nm.NM_F16, FAKE, 64, None) == 5
    assert L.nm_check_perm(None, 16, None) == 1
    assert L.nm_check_perm(FAKE, 0, None) == 2
    assert L.nm_set_variant(8) == 3
    assert L.nm_set_variant(7) == 3
    assert L.nm_set_variant(-1) == 3
    for v in range(7):
        assert L.nm_set_variant(v) == 0
    assert L.nm_set_variant(0) == 0


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    W = torch.zeros((4, 64), dtype=torch.float16)
    with pytest.raises(ValueError):
        nm.nm_compress(W, 2, 4)
