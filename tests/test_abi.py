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
    assert L.nm_version() == 201
    assert not hasattr(L, "nm_set_variant")  # no process-wide kernel state


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
            ldx=64, Y=FAKE * 4, ldy=32, od=nm.NM_F32, perm=None, ws=None, ws_bytes=0):
    L = nm.lib()
    if perm is None:
        return L.nm_spmm(values, idx, R, K, n, m, dt, act, T, ldx, Y, ldy, od, None)
    return L.nm_spmm_perm(values, idx, R, K, n, m, dt, act, T, ldx, perm, Y, ldy, od, ws, ws_bytes, None)


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
    # leading dimensions are bounded before any size product is formed
    assert st_spmm(ldx=(1 << 62)) == 2
    assert st_spmm(ldy=(1 << 62)) == 2
    assert st_compress(ldw=(1 << 62)) == 2
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

    # the kernel family is an argument of the call: out-of-range families are
    # refused; in-range ones with an empty product enqueue nothing
    def st_var(v, perm=None, T=8):
        return L.nm_spmm_variant(FAKE, FAKE * 2, 32, 64, 2, 4, nm.NM_F16, FAKE * 3, T, 64, perm,
                                 FAKE * 4, 32, nm.NM_F32, None, 0, v, None)
    assert st_var(7) == 3 and st_var(-1) == 3 and st_var(100) == 3
    for v in range(7):
        assert st_var(v, T=0) == 0
        assert st_var(v, perm=FAKE * 5, T=0) == 0
    assert st_var(3, perm=FAKE * 5 + 4) == 7       # misaligned map
    assert st_var(3, perm=FAKE * 4 + 64) == 5      # Y overlapping the map


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    W = torch.zeros((4, 64), dtype=torch.float16)
    with pytest.raises(ValueError):
        nm.nm_compress(W, 2, 4)


def test_binding_checks_packed_shapes_before_the_device():
    # The C ABI sees bare pointers, so the binding checks every tensor's shape,
    # dtype, layout and device; these checks come before the device check and
    # run here on CPU tensors.
    torch = pytest.importorskip("torch")
    R, K, T = 8, 64, 4
    vals = torch.zeros((R, K // 2), dtype=torch.float16)
    idx = torch.zeros((R, K // 32), dtype=torch.int32)
    act = torch.zeros((T, K), dtype=torch.float16)

    def err(fn):
        with pytest.raises((ValueError, TypeError)) as e:
            fn()
        return str(e.value)

    assert "contiguous [8, 32]" in err(lambda: nm.nm_spmm(vals[:, :16], idx, act, K))
    assert "int32 [4, 2]" in err(lambda: nm.nm_spmm(vals[:4], idx, act, K))   # R is values' row count
    assert "int32 [8, 2]" in err(lambda: nm.nm_spmm(vals, idx[:, :1], act, K))
    assert "int32 [8, 2]" in err(lambda: nm.nm_spmm(vals, idx.to(torch.int64), act, K))
    assert "int32 [8, 2]" in err(lambda: nm.nm_spmm(vals, idx.t().contiguous().t(), act, K))
    assert "[T, 64]" in err(lambda: nm.nm_spmm(vals, idx, act[:, :32], K))
    assert "out must be" in err(lambda: nm.nm_spmm(vals, idx, act, K, out=torch.zeros((T, R + 1))))
    assert "perm must be" in err(lambda: nm.nm_spmm_perm(vals, idx, act, torch.arange(K - 8, dtype=torch.int32), K))
    assert "perm must be" in err(lambda: nm.nm_spmm_perm(vals, idx, act, torch.arange(K), K))
    assert "out must be" in err(lambda: nm.nm_decompress(vals, idx, K, out=torch.zeros((R, K - 16), dtype=torch.float16)))
    assert "contiguous [8, 32]" in err(lambda: nm.nm_decompress(vals[:, :8], idx, K))
    assert "int32 [8, 2]" in err(lambda: nm.nm_compress(torch.zeros((R, K), dtype=torch.float16), 2, 4,
                                                         idx=torch.zeros((R, 1), dtype=torch.int32)))
    # right shapes: only the device is wrong
    assert "HIP device" in err(lambda: nm.nm_spmm(vals, idx, act, K))
    assert "HIP device" in err(lambda: nm.nm_spmm_perm(vals, idx, act, torch.arange(K, dtype=torch.int32), K))
    assert "HIP device" in err(lambda: nm.nm_decompress(vals, idx, K))


def test_perm_workspace_size_and_checks():
    # the gather pass takes T * K * 2 bytes of caller memory for 16-bit weights
    # with K % 8 == 0, K <= 65536 and more than 16 tokens; otherwise the map is
    # applied inside the kernel and no workspace is used
    ws = nm.nm_spmm_perm_workspace_size
    assert ws(3072, 768, 12608, 2, 4, nm.NM_F16) == 12608 * 768 * 2
    assert ws(3072, 768, 12608, 1, 8, nm.NM_BF16) == 12608 * 768 * 2
    assert ws(3072, 768, 16, 2, 4, nm.NM_F16) == 0            # few tokens: in the kernel
    assert ws(4096, 65536 + 16, 64, 2, 4, nm.NM_F16) == 0     # rows too long for the gather
    assert ws(0, 768, 64, 2, 4, nm.NM_F16) == 0
    assert ws(64, 768, 64, 2, 4, nm.NM_I8) == 0
    L = nm.lib()
    assert L.nm_spmm_perm_workspace_size(8, 60, 64, 2, 4, nm.NM_F16, None) == 2   # K % 16
    assert L.nm_spmm_perm_workspace_size(8, 64, 64, 2, 4, nm.NM_F16, None) == 1   # NULL out
    # a workspace must be aligned and must not overlap any argument
    P = FAKE * 5
    assert st_spmm(perm=P, ws=FAKE * 6 + 8, ws_bytes=4096) == 7
    assert st_spmm(perm=P, ws=FAKE * 3 + 256, ws_bytes=4096) == 5   # overlaps act
    assert st_spmm(perm=P, ws=FAKE * 4 - 64, ws_bytes=4096) == 5    # overlaps Y
    assert st_spmm(perm=P, ws=FAKE * 5 - 16, ws_bytes=64) == 5      # overlaps perm
    # a zero-size workspace is no workspace (only the shape is checked here)
    assert st_spmm(perm=P, ws=FAKE * 6 + 8, ws_bytes=0, T=0) == 0


def test_static_workspace_refuses_oversize_on_host():
    # nm_spmm_perm_static holds a 32 MiB array per GPU: a gather needing more is
    # refused during validation, before any HIP call (fake pointers)
    L = nm.lib()
    G = 1 << 36   # fake buffers far apart, so the large extents do not overlap
    def st(K, T):
        return L.nm_spmm_perm_static(G, 2 * G, 32, K, 2, 4, nm.NM_F16, 3 * G, T, K, 5 * G,
                                     4 * G, 32, nm.NM_F32, None)
    assert st(4096, 4097) == 2                     # 4096 * 4097 * 2 > 32 MiB
    assert "static workspace" in L.nm_last_error().decode()
    assert st(4096, 0) == 0                        # empty product


# ---------------------------------------------------------------------------
# hybrid dense / 2:4 tiles: layout (host), argument checks (fake pointers)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("R,K,tr,tc,frac", [(300, 1024, 64, 128, 0.5), (4096, 4096, 128, 128, 0.5),
                                            (64, 64, 64, 64, 1.0), (130, 512, 64, 64, 0.0),
                                            (1000, 768, 128, 64, 0.6)])
def test_hybrid_layout_matches_oracle(R, K, tr, tc, frac):
    import nm_inputs
    from oracle import nm_hybrid as H
    flags = nm_inputs.tile_flags(H.tile_grid(R, K, tr, tc), frac, 90, R)
    L = nm.nm_hybrid_layout(R, K, tr, tc, flags)
    tm, rm, nv, ni = H.hybrid_layout(R, K, tr, tc, flags)
    assert np.array_equal(L.tile_meta, tm) and np.array_equal(L.row_meta, rm)
    assert (L.values_count, L.idx_bytes) == (nv, ni)


def test_hybrid_layout_errors():
    L = nm.lib()
    f = np.zeros((4, 4), dtype=np.uint8)
    nv, ni = ctypes.c_int64(), ctypes.c_int64()

    def lay(R, K, tr, tc, flags=f):
        p = None if flags is None else flags.ctypes.data
        return L.nm_hybrid_layout(R, K, tr, tc, p, None, None, ctypes.byref(nv), ctypes.byref(ni))
    assert lay(256, 256, 64, 64) == 0 and (nv.value, ni.value) == (256 * 128, 256 * 32)
    assert lay(256, 256, 32, 64) == 2          # tile_rows not a multiple of 64
    assert lay(256, 256, 64, 96) == 2          # tile_cols not a multiple of 64
    assert lay(256, 320, 64, 128) == 2         # tile_cols does not divide K
    assert lay(256, 32, 64, 64) == 2           # K < 64
    assert lay(256, 256, 64, 64, None) == 1    # flags NULL
    bad = f.copy()
    bad[2, 3] = 2
    assert lay(256, 256, 64, 64, bad) == 2 and "flag" in L.nm_last_error().decode()
    assert lay(0, 256, 64, 64, None) == 0 and (nv.value, ni.value) == (0, 0)
    assert lay(64, 64 * 8193, 64, 64, np.zeros((1, 8193), np.uint8)) == 2   # too many tile-columns


def test_hybrid_compress_and_spmm_errors():
    L = nm.lib()
    F = FAKE
    # a valid 256 x 256 layout (all 2:4, 64 x 64 tiles): 32768 values, 8192 index bytes
    def comp(W=F, R=256, K=256, ldw=256, dt=nm.NM_F16, tr=64, tc=64, tm=5 * F, rm=6 * F, nv=32768, ni=8192,
             v=2 * F, i=3 * F):
        return L.nm_hybrid_compress(W, R, K, ldw, dt, tr, tc, tm, rm, nv, ni, v, i, None)
    assert comp(dt=nm.NM_I8) == 3
    assert comp(tr=48) == 2
    assert comp(ldw=200) == 4
    assert comp(W=None) == 1
    assert comp(i=None) == 1
    assert comp(i=None, ni=0, v=F + 64) == 5   # every tile dense: idx may be NULL (then the alias check)
    assert comp(v=2 * F + 8) == 7
    assert comp(tm=5 * F + 4) == 7             # layout tables 8-byte aligned
    assert comp(v=F + 64) == 5                 # values overlap W
    assert comp(nv=1 << 30) == 2               # 2 GiB of values
    assert comp(R=0) == 0

    def mm(v=2 * F, i=3 * F, tm=5 * F, rm=6 * F, R=256, K=256, tr=64, tc=64, nv=32768, ni=8192,
           dt=nm.NM_F16, act=F, T=64, ldx=256, Y=4 * F, ldy=256, od=nm.NM_F32):
        return L.nm_hybrid_spmm(v, i, tm, rm, R, K, tr, tc, nv, ni, dt, act, T, ldx, Y, ldy, od, None)
    assert mm(od=nm.NM_BF16) == 3
    assert mm(ldx=128) == 4
    assert mm(ldy=100) == 4
    assert mm(ldx=(1 << 22) + 8) == 2
    assert mm(act=None) == 1
    assert mm(Y=F + 256) == 5                  # Y overlaps act
    assert mm(Y=5 * F - 64) == 5               # Y overlaps the tile table
    assert mm(T=0) == 0


def test_train_argument_errors():
    # every call here fails validation (or has nothing to do) before any HIP call
    L = nm.lib()
    F = FAKE

    def dx(v=F, i=2 * F, R=256, K=256, n=2, m=4, dt=nm.NM_F16, G=3 * F, T=64, ldg=256, X=4 * F, ldo=256,
           od=nm.NM_F32):
        return L.nm_spmm_dx(v, i, R, K, n, m, dt, G, T, ldg, X, ldo, od, None)
    assert dx(dt=nm.NM_I8) == 3
    assert dx(od=nm.NM_BF16) == 3
    assert dx(n=3) == 3
    assert dx(K=100) == 2
    assert dx(K=272) == 2                    # K % 32
    assert dx(R=260) == 2                    # R % 8
    assert dx(T=-1) == 2
    assert dx(ldg=128) == 4
    assert dx(ldo=128) == 4
    assert dx(T=0) == 0                      # empty dX: nothing enqueued
    assert dx(G=None) == 1
    assert dx(X=None) == 1
    assert dx(ldg=260) == 7                  # G rows must be whole 16-byte pieces
    assert dx(G=3 * F + 8) == 7
    assert dx(X=3 * F) == 5                  # dX overlaps G

    def dw(i=F, R=256, K=256, n=2, m=4, dt=nm.NM_BF16, G=2 * F, T=64, ldg=256, a=3 * F, ldx=256, W=4 * F,
           od=nm.NM_F32):
        return L.nm_spmm_dw(i, R, K, n, m, dt, G, T, ldg, a, ldx, W, od, None)
    assert dw(dt=nm.NM_FP8) == 3
    assert dw(od=nm.NM_F16) == 3
    assert dw(ldx=200) == 4
    assert dw(ldg=200) == 4
    assert dw(R=0) == 0                      # no weights: nothing enqueued
    assert dw(i=None) == 1
    assert dw(a=None) == 1
    assert dw(ldx=260) == 7
    assert dw(W=3 * F) == 5                  # dW overlaps act


def test_train_binding_checks_before_the_device():
    torch = pytest.importorskip("torch")
    v = torch.zeros((8, 32), dtype=torch.float16)
    i = torch.zeros((8, 4), dtype=torch.int32)
    G = torch.zeros((4, 8), dtype=torch.float16)
    a = torch.zeros((4, 64), dtype=torch.float16)
    with pytest.raises((ValueError, TypeError)):
        nm.nm_spmm_dx(v, i, G[:, :7], 64)               # G's width is not R
    with pytest.raises(TypeError):
        nm.nm_spmm_dx(v.to(torch.int8), i, G.to(torch.int8), 64)
    with pytest.raises(ValueError):
        nm.nm_spmm_dw(i[:, :3], G, a, 64)               # idx of the wrong width
    with pytest.raises(TypeError):
        nm.nm_spmm_dw(i, G, a, 64, out_dtype=torch.bfloat16)
    with pytest.raises(ValueError):                     # CPU tensors never reach the C ABI
        nm.nm_spmm_dw(i, G, a, 64)


def test_block_structure_matches_oracle():
    from oracle import nm_hosts as H
    rng = np.random.default_rng(4)
    mask = (rng.random((5, 7)) < 0.4).astype(np.uint8)
    mask[2] = 0                                   # an empty block-row
    row_ptr, col = nm.nm_block_structure(160, 224, mask)
    ref_ptr, ref_col = H.block_structure(mask)
    assert row_ptr.tolist() == ref_ptr.tolist() and col.tolist() == ref_col.tolist()
    L = nm.lib()
    n = ctypes.c_int64()
    assert L.nm_block_structure(100, 64, None, None, None, ctypes.byref(n)) == 2     # R % 32
    assert L.nm_block_structure(64, 48, None, None, None, ctypes.byref(n)) == 2      # K % 32
    assert L.nm_block_structure(64, 64, None, None, None, ctypes.byref(n)) == 1      # mask NULL
    bad = np.array([1, 2, 0, 0], dtype=np.uint8)
    assert L.nm_block_structure(64, 64, bad.ctypes.data, None, None, ctypes.byref(n)) == 2


def test_block_and_diag_argument_errors():
    # every call here fails validation (or has nothing to do) before any HIP call
    L = nm.lib()
    F = FAKE

    def bs(v=F, rp=2 * F, col=3 * F, nnzb=4, R=64, K=96, dt=nm.NM_F16, act=4 * F, T=16, ldx=96, perm=None,
           Y=5 * F, ldy=64, od=nm.NM_F32):
        return L.nm_block_spmm(v, rp, col, nnzb, R, K, dt, act, T, ldx, perm, Y, ldy, od, None)
    assert bs(dt=nm.NM_I8) == 3
    assert bs(od=nm.NM_BF16) == 3
    assert bs(R=48) == 2                                  # R % 32
    assert bs(K=80, ldx=80) == 2                          # K % 32
    assert bs(nnzb=7) == 2                                # more blocks than the grid holds
    assert bs(ldx=64) == 4
    assert bs(ldy=32) == 4
    assert bs(T=0) == 0                                   # nothing enqueued
    assert bs(rp=None) == 1
    assert bs(v=None) == 1
    assert bs(ldx=100) == 7
    assert bs(perm=6 * F + 4) == 7
    assert bs(Y=4 * F) == 5                               # Y overlaps act
    assert bs(perm=5 * F + 64) == 5                       # Y overlaps the map

    def bc(W=F, R=64, K=96, ldw=96, dt=nm.NM_BF16, rp=2 * F, col=3 * F, nnzb=4, v=4 * F):
        return L.nm_block_compress(W, R, K, ldw, dt, rp, col, nnzb, v, None)
    assert bc(dt=nm.NM_FP8) == 3
    assert bc(ldw=64) == 4
    assert bc(nnzb=0) == 0
    assert bc(col=None) == 1
    assert bc(ldw=100) == 7
    assert bc(v=F + 64) == 5                              # values overlaps W

    def ds(v=F, off=2 * F, D=8, R=100, K=64, dt=nm.NM_F16, act=3 * F, T=16, ldx=64, perm=None, Y=4 * F,
           ldy=100, od=nm.NM_F32):
        return L.nm_diag_spmm(v, off, D, R, K, dt, act, T, ldx, perm, Y, ldy, od, None)
    assert ds(K=4096, ldx=4096) == 2                      # K above the staged limit
    assert ds(K=60, ldx=64) == 2                          # K % 8
    assert ds(D=65) == 2                                  # more diagonals than columns
    assert ds(od=nm.NM_F16, dt=nm.NM_BF16) == 3
    assert ds(ldy=64) == 4
    assert ds(R=0) == 0
    assert ds(off=None) == 1
    assert ds(D=0, v=None, off=None, Y=None) == 1         # Y is still required
    assert ds(act=3 * F + 8) == 7
    assert ds(Y=3 * F) == 5

    def dc(W=F, R=100, K=64, ldw=64, dt=nm.NM_F16, off=2 * F, D=8, v=3 * F):
        return L.nm_diag_compress(W, R, K, ldw, dt, off, D, v, None)
    assert dc(ldw=32) == 4
    assert dc(D=0) == 0
    assert dc(v=None) == 1
    assert dc(v=F + 32) == 5                              # values overlaps W


def test_block_and_diag_binding_checks_before_the_device():
    torch = pytest.importorskip("torch")
    act = torch.zeros((4, 64), dtype=torch.float16)
    rp = torch.zeros(3, dtype=torch.int32)
    col = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError):
        nm.nm_block_spmm(torch.zeros((2, 32, 16), dtype=torch.float16), rp, col, act)   # block of the wrong shape
    with pytest.raises(ValueError):
        nm.nm_block_spmm(torch.zeros((2, 32, 32), dtype=torch.float16), rp.to(torch.int64), col, act)
    with pytest.raises(ValueError):
        nm.nm_diag_spmm(torch.zeros((3, 8), dtype=torch.float16), torch.zeros(2, dtype=torch.int32), act)
    with pytest.raises(ValueError):
        nm.nm_block_spmm(torch.zeros((2, 32, 32), dtype=torch.float16), rp, col, act)   # CPU tensors
