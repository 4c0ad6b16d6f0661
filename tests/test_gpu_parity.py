"""Parity of the HIP path (through the C ABI) with the CPU oracle on MI355X.

Pack: values and index words bit-exact.  GEMM: max floored relative error
<= 1e-2 against the fp64 oracle, and every element inside the fp32
summation bound; exact-arithmetic cases bit-exact.
"""
import numpy as np
import pytest

import nm_inputs
import structured_sparse_gemm_nm_amd as nm
from oracle import nm_oracle as O
from gpu_util import (assert_close, bits_of, error_bound, log, oracle_pack, to_dev, torch_dtype,
                      words_of)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W_CASES = [(1, 2, 4), (2, 2, 4), (3, 2, 4), (4, 1, 4), (4, 1, 8), (5, 2, 4)]


def gpu_compress(w_bits, dt, n, m, ldw=None):
    R, K = w_bits.shape
    if ldw is not None and ldw != K:
        big = np.zeros((R, ldw), dtype=np.uint16)
        big[:, :K] = w_bits
        Wd = to_dev(big, dt)[:, :K]
    else:
        Wd = to_dev(w_bits, dt)
    vals, idx = nm.nm_compress(Wd, n, m)
    torch.cuda.synchronize()
    return vals, idx


# ---------------------------------------------------------------------------
# prune + pack
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("wid,n,m", W_CASES)
def test_compress_workloads_bit_exact(wid, n, m):
    wl = nm_inputs.WORKLOADS[wid]
    log(f"compress workload {wid} {wl.R}x{wl.K} {n}:{m} {wl.dtype}")
    w, ref_vals, ref_idx = oracle_pack(wid, n, m)
    vals, idx = gpu_compress(w, wl.dtype, n, m)
    assert np.array_equal(bits_of(vals), ref_vals)
    assert np.array_equal(words_of(idx), ref_idx)


@pytest.mark.parametrize("n,m", nm.PATTERNS)
@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("R,K,ldw", [(1, 16, 16), (3, 48, 56), (37, 80, 80), (129, 1040, 1048),
                                     (5, 272, 272), (64, 256, 320)])
def test_compress_ragged_and_ties(R, K, ldw, n, m, dt):
    if K % m:
        pytest.skip("K not a multiple of m")
    log(f"compress ragged R={R} K={K} ldw={ldw} {n}:{m} {dt}")
    # small integers with random signs: ties everywhere, +-0 included
    w = nm_inputs.integer_half((R, K), -3, 3, dt, 40, 0, R * 7 + K)
    vals, idx = gpu_compress(w, dt, n, m, ldw=ldw)
    ref_vals, ref_idx = O.prune_pack(w, n, m)
    assert np.array_equal(bits_of(vals), ref_vals)
    assert np.array_equal(words_of(idx), ref_idx)
    # and a normal draw
    w2 = nm_inputs.normal_half((R, K), 0.02, dt, 41, 0, R + K)
    vals, idx = gpu_compress(w2, dt, n, m, ldw=ldw)
    ref_vals, ref_idx = O.prune_pack(w2, n, m)
    assert np.array_equal(bits_of(vals), ref_vals)
    assert np.array_equal(words_of(idx), ref_idx)


def test_compress_worked_row():
    log("compress worked row")
    row = [0.5, 0.0, 0.0, -2.0, 0.0, 3.0, -1.0, 0.0] * 2
    w = np.asarray([row], dtype=np.float16).view(np.uint16)
    vals, idx = gpu_compress(w, "f16", 2, 4)
    assert words_of(idx)[0, 0] & 0xFF == 0x9C
    assert np.array_equal(words_of(idx), O.prune_pack(w, 2, 4)[1])


# fp16 / bf16 bit patterns of +inf, -inf, a quiet NaN, a NaN with the lowest
# payload, a negative NaN, and the largest finite value
SPECIALS = {"f16": (0x7C00, 0xFC00, 0x7E00, 0x7C01, 0xFE00, 0x7BFF),
            "bf16": (0x7F80, 0xFF80, 0x7FC0, 0x7F81, 0xFFC0, 0x7F7F)}


@pytest.mark.parametrize("n,m", nm.PATTERNS)
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_compress_nan_inf_weights(dt, n, m):
    # Magnitude is the stored pattern without its sign bit, so NaN (exponent
    # all ones, payload > 0) outranks inf, which outranks every finite value;
    # +inf and -inf tie and the lower position wins.  Pack bit-exact; in the
    # product a kept NaN makes the whole output row NaN and a kept inf makes it
    # +-inf (activations here are never zero), exactly as the fp64 oracle says.
    log(f"compress NaN/inf weights {dt} {n}:{m}")
    R, K, T = 256, 256, 128
    pinf, ninf, qnan, lnan, nnan, big = SPECIALS[dt]
    w = nm_inputs.normal_half((R, K), 1.0, dt, 74, 0)
    act = nm_inputs.normal_half((T, K), 1.0, dt, 74, 1)
    act[act & 0x7FFF == 0] = 0x3C00 if dt == "f16" else 0x3F80   # no zero activations
    plant = [(3, 5, qnan), (100, 130, nnan),                    # one NaN in a group
             (200, 8, qnan), (200, 9, lnan),                    # two NaNs with different payloads
             (10, 17, pinf), (50, 64, ninf),                    # one inf
             (150, 40, pinf), (150, 41, ninf),                  # +inf and -inf tie
             (60, 72, big), (60, 73, pinf),                     # inf beats the largest finite
             (70, 96, pinf), (70, 97, qnan)]                    # NaN beats inf
    for r, c, b in plant:
        w[r, c] = b
    vals, idx = gpu_compress(w, dt, n, m)
    ref_vals, ref_idx = O.prune_pack(w, n, m)
    assert np.array_equal(bits_of(vals), ref_vals)
    assert np.array_equal(words_of(idx), ref_idx)
    y = nm.nm_spmm(vals, idx, to_dev(act, dt), K, n, m)
    torch.cuda.synchronize()
    yv = y.cpu().numpy().astype(np.float64).T   # [R, T]
    with np.errstate(invalid="ignore", over="ignore"):
        yref = O.spmm_ref(ref_vals, ref_idx, K, n, m, act, dt)
    special = ~np.all(np.isfinite(yref), axis=1)
    assert special.any()
    # A finite bf16 weight near its largest value times |x| > 1 overflows the
    # fp32 accumulator although the fp64 oracle does not: on such rows the
    # output only has to be non-finite wherever the oracle's is.
    wd = O.half_bits_to_f64(O.decompress(ref_vals, ref_idx, K, n, m), dt)
    xa = np.abs(O.half_bits_to_f64(act, dt))
    wmax = np.max(np.where(np.isfinite(wd), np.abs(wd), 0.0), axis=1)
    ovf = wmax * xa.max() >= 2.0 ** 128
    assert np.all(~np.isfinite(yv[ovf]) >= ~np.isfinite(yref[ovf]))
    for name, f in (("nan", np.isnan), ("+inf", np.isposinf), ("-inf", np.isneginf)):
        bad = np.argwhere((f(yv) != f(yref)) & ~ovf[:, None])
        assert bad.size == 0, (f"{name} mask differs at {len(bad)} outputs, e.g. (row, token) "
                               f"{bad[:6].tolist()}: gpu {[yv[r, t] for r, t in bad[:6]]} "
                               f"oracle {[yref[r, t] for r, t in bad[:6]]}")
    rest = np.flatnonzero(~special & ~ovf)
    assert_close(y[:, rest], yref[rest], tol=1e-2)


@pytest.mark.parametrize("n,m", nm.PATTERNS)
def test_decompress_round_trip(n, m):
    log(f"decompress {n}:{m}")
    w = nm_inputs.normal_half((70, 208), 1.0, "bf16", 42, 0, m)
    vals, idx = gpu_compress(w, "bf16", n, m)
    dense = nm.nm_decompress(vals, idx, 208, n, m)
    torch.cuda.synchronize()
    ref_vals, ref_idx = O.prune_pack(w, n, m)
    assert np.array_equal(bits_of(dense), O.decompress(ref_vals, ref_idx, 208, n, m))


# ---------------------------------------------------------------------------
# GEMM on the five workloads
# ---------------------------------------------------------------------------

def run_workload(wid, n, m, T, out_dtype=None):
    wl = nm_inputs.WORKLOADS[wid]
    w, ref_vals, ref_idx = oracle_pack(wid, n, m)
    act = wl.activations(T)
    perm = wl.permutation()
    log(f"spmm workload {wid} R={wl.R} K={wl.K} T={T} {n}:{m} {wl.dtype} perm={perm is not None} out={out_dtype}")
    vals, idx = gpu_compress(w, wl.dtype, n, m)
    A = to_dev(act, wl.dtype)
    if perm is None:
        y = nm.nm_spmm(vals, idx, A, wl.K, n, m, out_dtype=out_dtype)
    else:
        y = nm.nm_spmm_perm(vals, idx, A, torch.from_numpy(perm).cuda(), wl.K, n, m,
                            out_dtype=out_dtype)
    torch.cuda.synchronize()
    yref = O.spmm_ref(ref_vals, ref_idx, wl.K, n, m, act, wl.dtype, perm=perm)
    bound = error_bound(ref_vals, ref_idx, wl.K, n, m, act, wl.dtype, perm=perm)
    return y, yref, bound, wl


@pytest.mark.parametrize("wid,n,m,T", [(1, 2, 4, 64), (2, 2, 4, 2048), (3, 2, 4, 1), (3, 2, 4, 8),
                                       (3, 2, 4, 16), (4, 1, 4, 512), (4, 1, 8, 512),
                                       (5, 2, 4, 12608)])
def test_spmm_workloads(wid, n, m, T):
    y, yref, bound, wl = run_workload(wid, n, m, T)
    max_rel, norm_rel = assert_close(y, yref, bound)
    log(f"  max_rel={max_rel:.3e} norm_rel={norm_rel:.3e}")


@pytest.mark.parametrize("wid,n,m,T", [(1, 2, 4, 64), (4, 1, 8, 512), (3, 2, 4, 16), (2, 2, 4, 2048)])
def test_spmm_half_output(wid, n, m, T):
    wl = nm_inputs.WORKLOADS[wid]
    od = torch.float16 if wl.dtype == "f16" else torch.bfloat16
    y, yref, bound, wl = run_workload(wid, n, m, T, out_dtype=od)
    assert y.dtype == od
    assert_close(y, yref, bound, out_half=wl.dtype)


# ---------------------------------------------------------------------------
# exact-arithmetic cases: bit-exact regardless of summation order
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,m", nm.PATTERNS)
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_identity_activations_exact(n, m, dt):
    # act = I (T = K): Y^T = W_nm^T exactly; every index decides one output
    R, K = 96, 256
    log(f"identity X {n}:{m} {dt}")
    w = nm_inputs.normal_half((R, K), 1.0, dt, 43, 0, m)
    vals, idx = gpu_compress(w, dt, n, m)
    eye = nm_inputs.to_half_bits(np.eye(K, dtype=np.float32), dt)
    y = nm.nm_spmm(vals, idx, to_dev(eye, dt), K, n, m)
    torch.cuda.synchronize()
    ref_vals, ref_idx = O.prune_pack(w, n, m)
    want = O.half_bits_to_f64(O.decompress(ref_vals, ref_idx, K, n, m), dt)
    assert np.array_equal(y.cpu().numpy().astype(np.float64).T, want)


@pytest.mark.parametrize("n,m", nm.PATTERNS)
@pytest.mark.parametrize("R,K,T", [(256, 4096, 256), (100, 80, 37), (33, 16, 5), (300, 1024, 130)])
def test_integer_gemm_exact(R, K, T, n, m):
    if K % m:
        pytest.skip("K not a multiple of m")
    log(f"integer gemm R={R} K={K} T={T} {n}:{m}")
    w = nm_inputs.integer_half((R, K), -3, 3, "f16", 44, 0, K)
    act = nm_inputs.integer_half((T, K), -2, 2, "f16", 44, 1, K)
    vals, idx = gpu_compress(w, "f16", n, m)
    y = nm.nm_spmm(vals, idx, to_dev(act, "f16"), K, n, m)
    # the resident-tile family (2:4, K % 256 == 0) on the same input
    y5 = nm.nm_spmm(vals, idx, to_dev(act, "f16"), K, n, m, variant=5)
    torch.cuda.synchronize()
    ref_vals, ref_idx = O.prune_pack(w, n, m)
    yref = O.spmm_ref(ref_vals, ref_idx, K, n, m, act, "f16")
    assert np.array_equal(y.cpu().numpy().astype(np.float64).T, yref)
    assert np.array_equal(y5.cpu().numpy().astype(np.float64).T, yref)


# ---------------------------------------------------------------------------
# permutation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,m", nm.PATTERNS)
def test_perm_properties(n, m):
    R, K, T = 200, 768, 300
    log(f"perm properties {n}:{m}")
    w = nm_inputs.normal_half((R, K), 0.02, "f16", 45, 0, m)
    act = nm_inputs.normal_half((T, K), 1.0, "f16", 45, 1, m)
    perm = nm_inputs.random_permutation(K, 45, m)
    vals, idx = gpu_compress(w, "f16", n, m)
    A = to_dev(act, "f16")
    P = torch.from_numpy(perm).cuda()
    nm.nm_check_perm(P)
    ident = torch.arange(K, dtype=torch.int32, device="cuda")
    A_perm = A[:, P.long()].contiguous()
    ref_vals, ref_idx = O.prune_pack(w, n, m)
    yref = O.spmm_ref(ref_vals, ref_idx, K, n, m, act, "f16", perm=perm)
    bound = error_bound(ref_vals, ref_idx, K, n, m, act, "f16", perm=perm)
    yref_id = O.spmm_ref(ref_vals, ref_idx, K, n, m, act, "f16")
    bound_id = error_bound(ref_vals, ref_idx, K, n, m, act, "f16")
    # the gather pass into a workspace, then the kernel the plain product takes
    y_perm = nm.nm_spmm_perm(vals, idx, A, P, K, n, m)
    y_id = nm.nm_spmm_perm(vals, idx, A, ident, K, n, m)
    y_copy = nm.nm_spmm(vals, idx, A_perm, K, n, m)
    y_plain = nm.nm_spmm(vals, idx, A, K, n, m)
    # the map applied inside the kernel (no workspace): compared with the
    # family it takes, named, on the explicitly permuted copy
    fam = 5 if (n, m) == (2, 4) else 1
    z_perm = nm.nm_spmm_perm(vals, idx, A, P, K, n, m, workspace=None)
    z_id = nm.nm_spmm_perm(vals, idx, A, ident, K, n, m, workspace=None)
    z_copy = nm.nm_spmm(vals, idx, A_perm, K, n, m, variant=fam)
    z_plain = nm.nm_spmm(vals, idx, A, K, n, m, variant=fam)
    torch.cuda.synchronize()
    assert torch.equal(y_perm, y_copy) and torch.equal(z_perm, z_copy)   # map = permuted copy
    assert torch.equal(y_id, y_plain) and torch.equal(z_id, z_plain)     # identity map = plain
    for y in (y_perm, z_perm):
        assert_close(y, yref, bound)
    for y in (y_id, z_id):
        assert_close(y, yref_id, bound_id)


# Every kernel family that reads activations through the map, on shapes that
# span several tiles and ragged tails: the resident-tile kernel (5: 64, 32 and
# 16 tokens per tile; row passes split across units when tokens are few; a
# partial last pass and token tile; fp32 and half outputs), the generic kernel
# (1) and the few-token kernel (4), each against the oracle and bit for bit
# against the same family on an explicitly permuted copy of the activations.
PERM_CASES = [
    # (R, K, T, dtype, family, out)
    (3072, 768, 12608, "f16", 5, "f32"),    # the permuted ViT-B/16 fc1 workload at full size
    (3072, 768, 197, "f16", 5, "f32"),      # one ViT image's tokens: a partial token tile
    (300, 768, 100, "bf16", 5, "f32"),      # ragged rows: a partial pass of 512
    (300, 768, 100, "f16", 5, "half"),
    (1000, 512, 700, "bf16", 5, "half"),    # R % 8 == 0 (unconditional half stores)
    (520, 1024, 130, "f16", 5, "f32"),      # K = 1024: 64-token tiles at the LDS limit
    (700, 2048, 70, "bf16", 5, "f32"),      # 32-token tiles
    (256, 4096, 40, "f16", 5, "half"),      # 16-token tiles
    (130, 256, 1500, "bf16", 5, "f32"),     # one block pair per pass, many units per CU
    (300, 768, 100, "f16", 1, "f32"),       # generic, element gather
    (258, 640, 65, "bf16", 1, "half"),      # generic, K % 128 != 0
    (77, 336, 7, "f16", 4, "f32"),          # few tokens
    (1030, 1024, 16, "bf16", 4, "half"),
]


@pytest.mark.parametrize("R,K,T,dt,fam,out", PERM_CASES)
def test_perm_families(R, K, T, dt, fam, out):
    log(f"perm family {fam} R={R} K={K} T={T} {dt} out={out}")
    w = nm_inputs.normal_half((R, K), 0.02, dt, 48, 0, R + K + T)
    act = nm_inputs.normal_half((T, K), 1.0, dt, 48, 1, R + K + T)
    perm = nm_inputs.random_permutation(K, 48, R + T)
    vals, idx = gpu_compress(w, dt, 2, 4)
    A = to_dev(act, dt)
    P = torch.from_numpy(perm).cuda()
    od = torch_dtype(dt) if out == "half" else torch.float32
    y = nm.nm_spmm_perm(vals, idx, A, P, K, 2, 4, out_dtype=od, variant=fam, workspace=None)
    y_copy = nm.nm_spmm(vals, idx, A[:, P.long()].contiguous(), K, 2, 4, out_dtype=od, variant=fam)
    torch.cuda.synchronize()
    assert torch.equal(y, y_copy)
    ref_vals, ref_idx = O.prune_pack(w, 2, 4)
    yref = O.spmm_ref(ref_vals, ref_idx, K, 2, 4, act, dt, perm=perm)
    assert_close(y, yref, error_bound(ref_vals, ref_idx, K, 2, 4, act, dt, perm=perm),
                 **({"out_half": dt} if out == "half" else {}))


# The default choice for the permuted product, with a workspace (the gather
# pass, walking more row blocks than workgroups for (128, 768, 11000) and
# (128, 8192, 2100); rows longer than the walking variant takes for
# (130, 8448, 70)) and without one (the map inside the kernel), on shapes of
# every family; with a workspace the result equals the plain product of the
# explicitly permuted copy bit for bit.
@pytest.mark.parametrize("ws", ["auto", None])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("R,K,T", [(300, 768, 100), (512, 128, 64), (256, 640, 130), (3072, 768, 197),
                                   (128, 768, 11000), (128, 8192, 2100), (130, 8448, 70)])
def test_perm_prefill(R, K, T, dt, ws):
    log(f"perm prefill R={R} K={K} T={T} {dt} workspace={ws}")
    w = nm_inputs.normal_half((R, K), 0.02, dt, 48, 0, R + K + T)
    act = nm_inputs.normal_half((T, K), 1.0, dt, 48, 1, R + K + T)
    perm = nm_inputs.random_permutation(K, 48, R + T)
    vals, idx = gpu_compress(w, dt, 2, 4)
    A = to_dev(act, dt)
    P = torch.from_numpy(perm).cuda()
    y = nm.nm_spmm_perm(vals, idx, A, P, K, 2, 4, workspace=ws)
    if ws is not None:
        y_copy = nm.nm_spmm(vals, idx, A[:, P.long()].contiguous(), K, 2, 4)
    torch.cuda.synchronize()
    if ws is not None:
        assert torch.equal(y, y_copy)
    ref_vals, ref_idx = O.prune_pack(w, 2, 4)
    yref = O.spmm_ref(ref_vals, ref_idx, K, 2, 4, act, dt, perm=perm)
    assert_close(y, yref, error_bound(ref_vals, ref_idx, K, 2, 4, act, dt, perm=perm))


def test_perm_workspace_caller_tensor():
    # a caller-owned workspace with room to spare is used and left to the caller;
    # one too small makes the kernel apply the map itself
    R, K, T, dt = 256, 512, 300, "bf16"
    log("perm caller workspace")
    w = nm_inputs.normal_half((R, K), 0.02, dt, 49, 0, 1)
    act = nm_inputs.normal_half((T, K), 1.0, dt, 49, 1, 1)
    perm = nm_inputs.random_permutation(K, 49, 1)
    vals, idx = gpu_compress(w, dt, 2, 4)
    A = to_dev(act, dt)
    P = torch.from_numpy(perm).cuda()
    need = nm.nm_spmm_perm_workspace_size(R, K, T, 2, 4, nm.NM_BF16)
    assert need == T * K * 2
    big = torch.full((need + 4096,), 7, dtype=torch.uint8, device="cuda")
    small = torch.full((need - 16,), 7, dtype=torch.uint8, device="cuda")
    y_big = nm.nm_spmm_perm(vals, idx, A, P, K, 2, 4, workspace=big)
    y_small = nm.nm_spmm_perm(vals, idx, A, P, K, 2, 4, workspace=small)
    torch.cuda.synchronize()
    assert torch.all(big[need:] == 7)          # nothing written past T * K * 2
    assert torch.all(small == 7)               # too small: not touched
    ref_vals, ref_idx = O.prune_pack(w, 2, 4)
    yref = O.spmm_ref(ref_vals, ref_idx, K, 2, 4, act, dt, perm=perm)
    bound = error_bound(ref_vals, ref_idx, K, 2, 4, act, dt, perm=perm)
    assert_close(y_big, yref, bound)
    assert_close(y_small, yref, bound)


def test_check_perm_rejects_non_permutation():
    bad = torch.tensor([0, 1, 1, 3] * 4, dtype=torch.int32, device="cuda")
    with pytest.raises(nm.NMError):
        nm.nm_check_perm(bad)


# ---------------------------------------------------------------------------
# ragged shapes, strides, canaries, determinism
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,m", nm.PATTERNS)
@pytest.mark.parametrize("R,K,T", [(1, 16, 1), (17, 48, 3), (255, 80, 129), (258, 208, 65),
                                   (513, 1040, 17), (64, 64, 200), (1000, 512, 2),
                                   (300, 1152, 257), (520, 1088, 300), (256, 128, 128)])
def test_spmm_ragged(R, K, T, n, m):
    if K % m:
        pytest.skip("K not a multiple of m")
    log(f"spmm ragged R={R} K={K} T={T} {n}:{m}")
    dt = "bf16"
    w = nm_inputs.normal_half((R, K), 0.5, dt, 46, 0, R + K + T)
    act = nm_inputs.normal_half((T, K), 1.0, dt, 46, 1, R + K + T)
    vals, idx = gpu_compress(w, dt, n, m)
    # act with a wider leading dimension, Y with padding columns holding a canary
    ldx = K + 24
    big = np.zeros((T, ldx), dtype=np.uint16)
    big[:, :K] = act
    A = to_dev(big, dt)[:, :K]
    ldy = (R + 3) // 4 * 4 + 8
    Yfull = torch.full((T, ldy), 12345.0, dtype=torch.float32, device="cuda")
    Y = Yfull[:, :R]
    nm.nm_spmm(vals, idx, A, K, n, m, out=Y)
    torch.cuda.synchronize()
    assert torch.all(Yfull[:, R:] == 12345.0), "write outside the output"
    ref_vals, ref_idx = O.prune_pack(w, n, m)
    yref = O.spmm_ref(ref_vals, ref_idx, K, n, m, act, dt)
    assert_close(Y, yref, error_bound(ref_vals, ref_idx, K, n, m, act, dt))


# half outputs of the tile kernels store 8 rows per lane (fragment pairs
# exchanged across lane quarters): ragged rows, a leading dimension that is or
# is not a multiple of 8, and canary columns past R
@pytest.mark.parametrize("fam", [3, 5])
@pytest.mark.parametrize("R,ldy_pad", [(300, 4), (300, 8), (301, 7), (512, 0)])
def test_half_output_edges(R, ldy_pad, fam):
    K, T, dt = 512, 200, "bf16"
    log(f"half edges R={R} pad={ldy_pad} family={fam}")
    w = nm_inputs.normal_half((R, K), 0.5, dt, 54, 0, R + ldy_pad)
    act = nm_inputs.normal_half((T, K), 1.0, dt, 54, 1, R + ldy_pad)
    vals, idx = gpu_compress(w, dt, 2, 4)
    A = to_dev(act, dt)
    ldy = R + ldy_pad
    Yfull = torch.full((T, ldy), 77.0, dtype=torch.bfloat16, device="cuda")
    Y = Yfull[:, :R]
    nm.nm_spmm(vals, idx, A, K, 2, 4, out_dtype=torch.bfloat16, out=Y, variant=fam)
    y1 = nm.nm_spmm(vals, idx, A, K, 2, 4, out_dtype=torch.bfloat16, variant=1)
    torch.cuda.synchronize()
    assert torch.all(Yfull[:, R:] == 77.0), "write outside the output"
    assert torch.equal(Y, y1)     # same sums, same rounding as the generic family
    ref_vals, ref_idx = O.prune_pack(w, 2, 4)
    yref = O.spmm_ref(ref_vals, ref_idx, K, 2, 4, act, dt)
    assert_close(Y, yref, error_bound(ref_vals, ref_idx, K, 2, 4, act, dt), out_half=dt)


def test_spmm_deterministic_and_empty():
    log("determinism")
    wl = nm_inputs.WORKLOADS[1]
    w, _, _ = oracle_pack(1, 2, 4)
    vals, idx = gpu_compress(w, "f16", 2, 4)
    A = to_dev(wl.activations(), "f16")
    y1 = nm.nm_spmm(vals, idx, A, wl.K, 2, 4)
    y2 = nm.nm_spmm(vals, idx, A, wl.K, 2, 4)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    empty = nm.nm_spmm(vals, idx, A[:0], wl.K, 2, 4)
    assert empty.shape == (0, wl.R)


# ---------------------------------------------------------------------------
# few tokens (the decode kernel): ragged rows, odd T, a partial last K step,
# with and without the permutation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,m", nm.PATTERNS)
@pytest.mark.parametrize("R,K,T,permuted", [(100, 4096, 13, False), (77, 336, 7, True),
                                            (1030, 1024, 16, True), (5, 16, 1, False),
                                            (600, 2064, 4, False)])
def test_spmm_few_tokens(R, K, T, permuted, n, m):
    if K % m:
        pytest.skip("K not a multiple of m")
    log(f"few tokens R={R} K={K} T={T} perm={permuted} {n}:{m}")
    dt = "f16"
    w = nm_inputs.normal_half((R, K), 0.02, dt, 47, 0, R + K)
    act = nm_inputs.normal_half((T, K), 1.0, dt, 47, 1, R + K)
    vals, idx = gpu_compress(w, dt, n, m)
    A = to_dev(act, dt)
    perm = nm_inputs.random_permutation(K, 47, R) if permuted else None
    if perm is None:
        y = nm.nm_spmm(vals, idx, A, K, n, m)
    else:
        y = nm.nm_spmm_perm(vals, idx, A, torch.from_numpy(perm).cuda(), K, n, m)
    torch.cuda.synchronize()
    ref_vals, ref_idx = O.prune_pack(w, n, m)
    yref = O.spmm_ref(ref_vals, ref_idx, K, n, m, act, dt, perm=perm)
    assert_close(y, yref, error_bound(ref_vals, ref_idx, K, n, m, act, dt, perm=perm))


def test_out_tensor_checked():
    R, K, T = 64, 128, 16
    w = nm_inputs.normal_half((R, K), 0.02, "f16", 53, 0, 1)
    act = nm_inputs.normal_half((T, K), 1.0, "f16", 53, 1, 1)
    vals, idx = gpu_compress(w, "f16", 2, 4)
    A = to_dev(act, "f16")
    with pytest.raises(TypeError):  # fp32 output into an fp16 tensor
        nm.nm_spmm(vals, idx, A, K, 2, 4, out=torch.empty((T, R), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):  # too few rows
        nm.nm_spmm(vals, idx, A, K, 2, 4, out=torch.empty((T - 1, R), dtype=torch.float32, device="cuda"))
    y = torch.full((T, R), 7.0, dtype=torch.float32, device="cuda")
    assert nm.nm_spmm(vals, idx, A, K, 2, 4, out=y) is y
    torch.cuda.synchronize()
    assert torch.equal(y, nm.nm_spmm(vals, idx, A, K, 2, 4))


# ---------------------------------------------------------------------------
# every kernel family on the same inputs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,m", nm.PATTERNS)
def test_kernel_families_agree(n, m):
    R, K, T = 512, 1024, 256
    log(f"kernel families {n}:{m}")
    w = nm_inputs.normal_half((R, K), 0.02, "bf16", 49, 0, m)
    act = nm_inputs.normal_half((T, K), 1.0, "bf16", 49, 1, m)
    vals, idx = gpu_compress(w, "bf16", n, m)
    A = to_dev(act, "bf16")
    outs = {v: nm.nm_spmm(vals, idx, A, K, n, m, variant=v) for v in (1, 2, 3, 5, 6)}
    y_few = nm.nm_spmm(vals, idx, A[:16].contiguous(), K, n, m, variant=4)
    y_few_ref = nm.nm_spmm(vals, idx, A[:16].contiguous(), K, n, m, variant=1)
    torch.cuda.synchronize()
    # families that add the K steps in order from zero give identical bits
    # (a family that does not take the shape falls back to the choice by
    # shape).  For 1:4 / 1:8 that choice, and families 3, 5 and 6, is the LDS
    # kernel that sums even and odd K steps apart and then adds the two.
    assert torch.equal(outs[1], outs[2])
    if n == 2:
        assert all(torch.equal(outs[1], outs[v]) for v in (3, 5, 6))
    else:
        assert all(torch.equal(outs[6], outs[v]) for v in (3, 5))
    ref_vals, ref_idx = O.prune_pack(w, n, m)
    yref = O.spmm_ref(ref_vals, ref_idx, K, n, m, act, "bf16")
    bound = error_bound(ref_vals, ref_idx, K, n, m, act, "bf16")
    assert_close(outs[1], yref, bound)
    assert_close(outs[6], yref, bound)
    # the few-token family splits K: same product within the summation bound
    assert_close(y_few, yref[:, :16], error_bound(ref_vals, ref_idx, K, n, m, act[:16], "bf16"))
    assert_close(y_few_ref, yref[:, :16])


# ---------------------------------------------------------------------------
# prefill kernel with more tiles than compute units: each workgroup walks
# several tiles and starts a tile's loads during the one before it
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("R,K,T,out", [(2200, 256, 3900, "f32"), (2200, 384, 3900, "f32"),
                                       (2200, 640, 3900, "f32"), (2200, 768, 3900, "half"),
                                       (2205, 256, 3900, "half"),
                                       (2200, 1408, 3900, "f32"), (4100, 256, 4000, "f32")])
def test_lds_tile_walk(R, K, T, out):
    log(f"lds tile walk R={R} K={K} T={T} out={out}")
    dt = "bf16"
    w = nm_inputs.normal_half((R, K), 0.02, dt, 50, 0, R + K + T)
    act = nm_inputs.normal_half((T, K), 1.0, dt, 50, 1, R + K + T)
    vals, idx = gpu_compress(w, dt, 2, 4)
    A = to_dev(act, dt)
    od = torch.bfloat16 if out == "half" else torch.float32
    y = nm.nm_spmm(vals, idx, A, K, 2, 4, out_dtype=od, variant=3)
    y_gen = nm.nm_spmm(vals, idx, A, K, 2, 4, out_dtype=od, variant=1)
    torch.cuda.synchronize()
    # both add the K steps in order from zero
    assert torch.equal(y, y_gen)
    ref_vals, ref_idx = O.prune_pack(w, 2, 4)
    yref = O.spmm_ref(ref_vals, ref_idx, K, 2, 4, act, dt)
    assert_close(y, yref, error_bound(ref_vals, ref_idx, K, 2, 4, act, dt),
                 **({"out_half": dt} if out == "half" else {}))


# ---------------------------------------------------------------------------
# 1:4 / 1:8 through LDS: 128 x 64 tiles; index bits in 16-step blocks (a
# partial last block when K / 64 is not a multiple of 16); ragged rows and
# tokens; more tiles than two per compute unit (walked)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,m", [(1, 4), (1, 8)])
@pytest.mark.parametrize("R,K,T,dt,out", [(4096, 4096, 512, "f16", "f32"), (300, 768, 100, "bf16", "f32"),
                                          (130, 256, 64, "f16", "half"), (1000, 1280, 1000, "bf16", "half"),
                                          (2432, 512, 1000, "bf16", "f32"), (2200, 512, 3900, "f16", "f32")])
def test_lds_nm(R, K, T, dt, out, n, m):
    log(f"lds 1:4/1:8 {n}:{m} R={R} K={K} T={T} {dt} out={out}")
    w = nm_inputs.normal_half((R, K), 0.02, dt, 52, 0, R + K + T + m)
    act = nm_inputs.normal_half((T, K), 1.0, dt, 52, 1, R + K + T + m)
    vals, idx = gpu_compress(w, dt, n, m)
    A = to_dev(act, dt)
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    od = tdt if out == "half" else torch.float32
    y = nm.nm_spmm(vals, idx, A, K, n, m, out_dtype=od, variant=6)
    y_pipe = nm.nm_spmm(vals, idx, A, K, n, m, out_dtype=od, variant=2)
    y_again = nm.nm_spmm(vals, idx, A, K, n, m, out_dtype=od, variant=6)
    torch.cuda.synchronize()
    # the same widened operands; the LDS kernel sums even and odd K steps
    # apart and adds the two, so it matches the pipelined kernel to rounding,
    # and itself bit for bit
    assert torch.equal(y, y_again)
    ref_vals, ref_idx = O.prune_pack(w, n, m)
    yref = O.spmm_ref(ref_vals, ref_idx, K, n, m, act, dt)
    bound = error_bound(ref_vals, ref_idx, K, n, m, act, dt)
    kw = {"out_half": dt} if out == "half" else {}
    assert_close(y, yref, bound, **kw)
    assert_close(y_pipe, yref, bound, **kw)


# ---------------------------------------------------------------------------
# few-token kernel for tall weights: one workgroup per CU owns 1..8 blocks of
# 16 rows (the even split, last block partial; with 256 CUs the last three
# shapes have three, as the 11008-row decode layer does); K slices past the
# last step in some waves; the index map read inside the kernel
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("R,K,T,dt,permuted", [(4096, 4096, 1, "bf16", False),
                                               (6000, 4096, 16, "bf16", False),
                                               (20000, 4096, 5, "f16", False),
                                               (33000, 2176, 16, "bf16", False),
                                               (5000, 2176, 7, "f16", False),
                                               (6000, 4096, 9, "f16", True), (10000, 4096, 3, "bf16", False),
                                               (11008, 2176, 16, "f16", False), (11008, 4096, 2, "bf16", True)])
def test_decode_stream(R, K, T, dt, permuted):
    log(f"decode stream R={R} K={K} T={T} {dt} perm={permuted}")
    w = nm_inputs.normal_half((R, K), 0.02, dt, 51, 0, R + K + T)
    act = nm_inputs.normal_half((T, K), 1.0, dt, 51, 1, R + K + T)
    vals, idx = gpu_compress(w, dt, 2, 4)
    A = to_dev(act, dt)
    perm = nm_inputs.random_permutation(K, 51, R) if permuted else None
    if perm is None:
        y = nm.nm_spmm(vals, idx, A, K, 2, 4, variant=4)
    else:
        y = nm.nm_spmm_perm(vals, idx, A, torch.from_numpy(perm).cuda(), K, 2, 4, variant=4, workspace=None)
    torch.cuda.synchronize()
    ref_vals, ref_idx = O.prune_pack(w, 2, 4)
    yref = O.spmm_ref(ref_vals, ref_idx, K, 2, 4, act, dt, perm=perm)
    assert_close(y, yref, error_bound(ref_vals, ref_idx, K, 2, 4, act, dt, perm=perm))


# ---------------------------------------------------------------------------
# INT8 2:4: packed values and indices, the decompressed weight and the int32
# product, all bit for bit (the product is exact); ragged rows, tokens and K
# tails (K a multiple of 32 but not of the 128-wide step), T = 1, extremes
# ---------------------------------------------------------------------------

def _i8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("R,K,T", [(1, 32, 1), (7, 96, 5), (130, 160, 129), (300, 4128, 70),
                                   (1000, 1024, 3), (257, 2048, 300),
                                   # whole 256 x 128 tiles, K % 128 == 0: the LDS-staged kernel,
                                   # 1, 2, 3, 4 and 9 K steps (the ring's tail cases)
                                   (256, 128, 128), (256, 256, 256), (512, 384, 128),
                                   (256, 512, 384), (768, 1152, 256)])
def test_i8_bit_exact(R, K, T):
    log(f"int8 2:4 R={R} K={K} T={T}")
    w = nm_inputs.normal_i8((R, K), 32.0, 61, 0, R + K + T)
    act = nm_inputs.normal_i8((T, K), 32.0, 61, 1, R + K + T)
    vals, idx = nm.nm_compress(_i8(w), 2, 4)
    dense = nm.nm_decompress(vals, idx, K, 2, 4)
    y = nm.nm_spmm(vals, idx, _i8(act), K, 2, 4)
    torch.cuda.synchronize()
    ref_vals, ref_idx = O.prune_pack_i8(w, 2, 4)
    assert vals.dtype == torch.int8 and y.dtype == torch.int32
    assert np.array_equal(vals.cpu().numpy(), ref_vals)
    assert np.array_equal(idx.cpu().numpy().view(np.uint32), ref_idx)
    assert np.array_equal(dense.cpu().numpy(), O.decompress_i8(ref_vals, ref_idx, K, 2, 4))
    yref = O.spmm_ref_i8(ref_vals, ref_idx, K, 2, 4, act)
    assert np.array_equal(y.cpu().numpy().T.astype(np.int64), yref)
    y1 = nm.nm_spmm(vals, idx, _i8(act), K, 2, 4, variant=1)  # the register-operand kernel
    torch.cuda.synchronize()
    assert torch.equal(y1, y)


def test_i8_extremes():
    log("int8 2:4 extremes")
    R, K, T = 64, 4096, 32
    # every weight and activation -128: each group keeps positions 0 and 1,
    # every product is 2^14 and the sums reach K/2 * 2^14 = 2^25
    w = np.full((R, K), -128, np.int8)
    act = np.full((T, K), -128, np.int8)
    vals, idx = nm.nm_compress(_i8(w), 2, 4)
    y = nm.nm_spmm(vals, idx, _i8(act), K, 2, 4)
    torch.cuda.synchronize()
    assert np.all(idx.cpu().numpy().view(np.uint32) == 0x44444444)
    assert np.all(y.cpu().numpy() == (K // 2) * 128 * 128)
    # ties of +/-x: the lower position wins; zeros rows give zeros
    w2 = np.tile(np.array([3, -3, 3, -3, 0, 0, 0, 0, -128, 127, -127, 128 - 1], np.int8), (R, K // 12 + 1))[:, :K]
    w2 = np.ascontiguousarray(w2[:, :K])
    vals2, idx2 = nm.nm_compress(_i8(w2), 2, 4)
    rv, ri = O.prune_pack_i8(w2, 2, 4)
    assert np.array_equal(vals2.cpu().numpy(), rv)
    assert np.array_equal(idx2.cpu().numpy().view(np.uint32), ri)


def test_i8_workload_sampled():
    wl = nm_inputs.WORKLOADS[6]
    T = wl.Ts[0]
    log(f"int8 workload {wl.R}x{wl.K}x{T}")
    w = wl.weights()
    act = wl.activations(T)
    vals, idx = nm.nm_compress(_i8(w), 2, 4)
    y = nm.nm_spmm(vals, idx, _i8(act), wl.K, 2, 4)
    torch.cuda.synchronize()
    ref_vals, ref_idx = O.prune_pack_i8(w, 2, 4)
    assert np.array_equal(vals.cpu().numpy(), ref_vals)
    assert np.array_equal(idx.cpu().numpy().view(np.uint32), ref_idx)
    rows = np.sort(np.random.default_rng(5).choice(wl.R, 48, replace=False))
    yref = O.spmm_ref_i8(ref_vals[rows], ref_idx[rows], wl.K, 2, 4, act)
    assert np.array_equal(y.cpu().numpy()[:, rows].T.astype(np.int64), yref)


# ---------------------------------------------------------------------------
# FP8 (OCP E4M3) 2:4: packed bytes bit-exact, Y against the exact product
# ---------------------------------------------------------------------------

def _f8(bits):
    return torch.from_numpy(np.ascontiguousarray(bits)).cuda().view(torch.float8_e4m3fn)


def _abs_sum_bound(y, yref, ref_vals, ref_idx, K, act, frac=2.0 ** -12):
    wa = np.abs(O.fp8_to_f64(O.decompress_fp8(ref_vals, ref_idx, K, 2, 4)))
    xa = np.abs(O.fp8_to_f64(act)).T
    scale = wa @ xa  # [R, T]
    err = np.abs(y.float().cpu().numpy().astype(np.float64).T - yref)
    worst = float(np.max(err / np.maximum(scale, 1e-30)))
    log(f"fp8 worst |error| / sum|products| = {worst:.3e}")
    assert worst <= frac, f"error {worst:.3e} of sum|products| > {frac:.3e}"


def _f8_case(w, act, K, cross_check=True):
    vals, idx = nm.nm_compress(_f8(w), 2, 4)
    dense = nm.nm_decompress(vals, idx, K, 2, 4)
    y = nm.nm_spmm(vals, idx, _f8(act), K, 2, 4)
    torch.cuda.synchronize()
    ref_vals, ref_idx = O.prune_pack_fp8(w, 2, 4)
    assert vals.dtype == torch.float8_e4m3fn and y.dtype == torch.float32
    assert np.array_equal(vals.view(torch.uint8).cpu().numpy(), ref_vals)
    assert np.array_equal(idx.cpu().numpy().view(np.uint32), ref_idx)
    assert np.array_equal(dense.view(torch.uint8).cpu().numpy(), O.decompress_fp8(ref_vals, ref_idx, K, 2, 4))
    yref = O.spmm_ref_fp8(ref_vals, ref_idx, K, 2, 4, act)
    # the stated 1e-2 bound on the floored relative error, and each element's
    # error against the sum of |products| (the hardware's fp8 accumulation is
    # coarser than fp32 where the sum cancels; a wrong index or operand gives
    # errors of the order of that sum)
    assert_close(y, yref, tol=1e-2)
    _abs_sum_bound(y, yref, ref_vals, ref_idx, K, act)
    if cross_check:
        # the register-operand kernel: the same MFMA sequence per tile
        y1 = nm.nm_spmm(vals, idx, _f8(act), K, 2, 4, variant=1)
        torch.cuda.synchronize()
        assert torch.equal(y1, y)
    return y, yref


@pytest.mark.parametrize("R,K,T", [(1, 32, 1), (7, 96, 5), (130, 160, 129), (300, 4128, 70),
                                   (257, 2048, 300),
                                   # the LDS-staged kernel: 1, 2, 3, 4 and 9 K steps
                                   (256, 128, 128), (256, 256, 256), (512, 384, 128),
                                   (256, 512, 384), (768, 1152, 256)])
def test_fp8_pack_and_product(R, K, T):
    log(f"fp8 2:4 R={R} K={K} T={T}")
    w = nm_inputs.normal_fp8((R, K), 1.0, 71, 0, R + K + T)
    act = nm_inputs.normal_fp8((T, K), 1.0, 71, 1, R + K + T)
    _f8_case(w, act, K)


def test_fp8_extremes():
    log("fp8 2:4 extremes")
    R, K, T = 64, 4096, 32
    # every weight -448 and every activation 448: positions 0 and 1 kept, each
    # product -200704 = -49 * 2^12, sums -49 * 2^12 * K/2, exact in fp32
    w = np.full((R, K), 0xFE, np.uint8)   # -448
    act = np.full((T, K), 0x7E, np.uint8)  # 448
    vals, idx = nm.nm_compress(_f8(w), 2, 4)
    y = nm.nm_spmm(vals, idx, _f8(act), K, 2, 4)
    torch.cuda.synchronize()
    assert np.all(idx.cpu().numpy().view(np.uint32) == 0x44444444)
    assert np.all(y.cpu().numpy() == -200704.0 * (K // 2))
    # +x / -x tie (lower position wins), zeros of both signs, the smallest subnormal
    pat = np.array([0x38, 0xB8, 0x38, 0xB8, 0x00, 0x80, 0x00, 0x80, 0x01, 0x81, 0x00, 0x02], np.uint8)
    w2 = np.ascontiguousarray(np.tile(pat, (R, K // 12 + 1))[:, :K])
    vals2, idx2 = nm.nm_compress(_f8(w2), 2, 4)
    rv, ri = O.prune_pack_fp8(w2, 2, 4)
    torch.cuda.synchronize()
    assert np.array_equal(vals2.view(torch.uint8).cpu().numpy(), rv)
    assert np.array_equal(idx2.cpu().numpy().view(np.uint32), ri)


def test_fp8_workload_sampled():
    wl = nm_inputs.WORKLOADS[7]
    T = wl.Ts[0]
    log(f"fp8 workload {wl.R}x{wl.K}x{T}")
    w = wl.weights()
    act = wl.activations(T)
    vals, idx = nm.nm_compress(_f8(w), 2, 4)
    y = nm.nm_spmm(vals, idx, _f8(act), wl.K, 2, 4)
    torch.cuda.synchronize()
    ref_vals, ref_idx = O.prune_pack_fp8(w, 2, 4)
    assert np.array_equal(vals.view(torch.uint8).cpu().numpy(), ref_vals)
    assert np.array_equal(idx.cpu().numpy().view(np.uint32), ref_idx)
    rows = np.sort(np.random.default_rng(7).choice(wl.R, 48, replace=False))
    yref = O.spmm_ref_fp8(ref_vals[rows], ref_idx[rows], wl.K, 2, 4, act)
    assert_close(y[:, rows], yref, tol=1e-2)
    _abs_sum_bound(y[:, rows], yref, ref_vals[rows], ref_idx[rows], wl.K, act)


def test_fp8_small_magnitudes():
    # scale 2^-7: most inputs are E4M3 subnormals (below 2^-6)
    log("fp8 2:4 subnormal inputs")
    R, K, T = 256, 512, 128
    w = nm_inputs.normal_fp8((R, K), 2.0 ** -7, 72, 0)
    act = nm_inputs.normal_fp8((T, K), 1.0, 72, 1)
    _f8_case(w, act, K, cross_check=False)


def test_fp8_nan_inputs():
    # S.1111.111 is E4M3's NaN; its key (0x7F) is the largest, so a group
    # holding one keeps it, and every output of that row is NaN
    log("fp8 2:4 NaN weights")
    R, K, T = 256, 256, 128
    w = nm_inputs.normal_fp8((R, K), 1.0, 73, 0)
    act = nm_inputs.normal_fp8((T, K), 1.0, 73, 1)
    nan_rows = np.array([3, 100, 255])
    w[nan_rows, [5, 130, 255]] = np.array([0x7F, 0xFF, 0x7F], np.uint8)
    vals, idx = nm.nm_compress(_f8(w), 2, 4)
    y = nm.nm_spmm(vals, idx, _f8(act), K, 2, 4)
    torch.cuda.synchronize()
    ref_vals, ref_idx = O.prune_pack_fp8(w, 2, 4)
    assert np.array_equal(vals.view(torch.uint8).cpu().numpy(), ref_vals)
    assert np.array_equal(idx.cpu().numpy().view(np.uint32), ref_idx)
    yv = y.cpu().numpy()
    assert np.all(np.isnan(yv[:, nan_rows]))
    rest = np.setdiff1d(np.arange(R), nan_rows)
    yref = O.spmm_ref_fp8(ref_vals[rest], ref_idx[rest], K, 2, 4, act)
    assert_close(y[:, rest], yref, tol=1e-2)
