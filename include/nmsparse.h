/*
 * nmsparse.h -- N:M structured weight sparsity on AMD Instinct MI355X (gfx950).
 *
 * A C ABI over plain pointers and sizes.  Every device pointer is HIP device
 * memory owned by the caller; the library allocates nothing on these paths
 * and keeps no state between calls.  Streams are passed as `void*` holding a
 * hipStream_t (NULL = the legacy default stream).
 *
 * Notation.  W is R x K (rows = output features, K = the reduction axis).
 * An N:M pattern keeps N of every M consecutive weights along a row of W;
 * S = K*N/M survivors per row; b = ceil(log2 M) index bits per survivor.
 *
 * Sources.  "M:N sparsity on NVIDIA tensor cores" (COE-592 lecture 04-2):
 * the opening section defines the pattern (groups along rows, survivor
 * positions per group) and the survivors:block notation; section "Where this
 * sits among the three case studies" gives the storage format (survivors
 * pushed left, small per-survivor indices), the product rule (only the weight
 * operand is compressed; sparse times dense is dense) and the shape rule (the
 * reduction dimension a multiple of 16 for 16-bit types, other layers stay
 * dense); section "The recipe" gives the pruning rule (keep the largest
 * magnitudes).  "SHUFFLESPARSE" technical summary, section 2 and its item on
 * inference efficiency: y = (W Pi) x with the hardened permutation applied as
 * a precomputed index map on the input reads.
 *
 * Error behaviour.  Every entry point validates its arguments on the host
 * before any HIP call and returns a status; on failure nothing is enqueued
 * and nm_last_error() describes the problem.  NM_OK means the work was
 * enqueued on `stream` (asynchronous, stream-ordered); device-side faults
 * surface at the caller's next synchronisation.  No exception or abort
 * crosses this boundary.  Results are bitwise reproducible (no atomics).
 */
#ifndef NMSPARSE_H
#define NMSPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NM_OK = 0,
  NM_ERR_NULL = 1,         /* a required pointer is NULL                          */
  NM_ERR_SHAPE = 2,        /* R, K or T out of range; K % 16 (K % 32 for 8-bit W) or K % M non-zero */
  NM_ERR_UNSUPPORTED = 3,  /* (n, m) pair or dtype combination not provided       */
  NM_ERR_STRIDE = 4,       /* leading dimension smaller than the row width        */
  NM_ERR_ALIAS = 5,        /* output overlaps an input                            */
  NM_ERR_HIP = 6,          /* a HIP call failed (launch error, no device, ...)    */
  NM_ERR_ALIGN = 7         /* pointer or leading dimension misaligned (see below) */
} nm_status;

typedef enum { NM_F16 = 0, NM_BF16 = 1, NM_F32 = 2, NM_I8 = 3, NM_I32 = 4, NM_FP8 = 5 } nm_dtype;

/*
 * INT8 weights (NM_I8).  The 2:4 pattern is also offered for 8-bit integer
 * weights; the index stays 2 bits per stored value, so a group of four costs
 * 2*8 + 2*2 = 20 bits (37.5% below dense), and the reduction length must be a
 * multiple of 32 (COE-592 lecture 04-2, "M:N sparsity on NVIDIA tensor cores":
 * opening section, and section "Where this sits among the three case
 * studies").  With dtype NM_I8 every entry point below takes only (n, m) =
 * (2, 4) (else NM_ERR_UNSUPPORTED) and K % 32 == 0 (else NM_ERR_SHAPE); values
 * are one byte each; magnitude is |w| as an integer (-128 ranks above 127,
 * equal magnitudes go to the lower position); act is int8 and Y is int32
 * (out_dtype NM_I32, the only one), the exact integer product; leading
 * dimensions of int8 matrices (ldw, ldx) must be multiples of 16.
 * nm_spmm_perm does not take NM_I8 (NM_ERR_UNSUPPORTED).
 *
 * FP8 weights (NM_FP8, OCP E4M3: sign, 4 exponent bits with bias 7, 3
 * mantissa bits, no infinities, S.1111.111 is NaN).  The pages name 16-bit
 * and INT8 2:4 types only; an 8-bit float takes the one-byte layout and every
 * rule of NM_I8 above (2:4 only, K % 32, ldw and ldx multiples of 16, no
 * nm_spmm_perm), with these differences: magnitude is compared on the stored
 * pattern with the sign bit cleared (bits & 0x7F, so +x and -x tie, equal keys
 * going to the lower position), act is E4M3 and Y is fp32 (out_dtype NM_F32,
 * the only one).  The hardware's fp8 sparse multiply-accumulate sums with
 * somewhat less than fp32 precision (relative error near 1e-4 of the result
 * at K = 2048); NaN inputs give NaN outputs.
 */

/* Version of this ABI (major * 100 + minor): 101 adds NM_I8 / NM_I32,
 * 102 adds NM_FP8. */
int nm_version(void);

/* Short fixed text for a status code (never NULL). */
const char* nm_status_string(int status);

/* Detail for the last failing call on this thread (empty string if none). */
const char* nm_last_error(void);

/*
 * Sizes of the packed format.  Pure host arithmetic, no device access.
 *   values_bytes  = R * S * 2            (values [R, S], same type as W; R * S for 8-bit W)
 *   idx_row_words = ceil(S * b / 32)     (uint32 words per row)
 *   idx_bytes     = R * idx_row_words * 4
 * Any output pointer may be NULL.  Same validation as nm_compress.
 *
 * Packed format (the canonical one every entry point reads and writes):
 *   values[r, g*N + j]  the j-th survivor of group g of row r, survivors of a
 *                       group in ascending position order, bits copied
 *                       unchanged from W;
 *   idx row r           an LSB-first bitstream: the in-group position (0..M-1)
 *                       of survivor s = g*N + j sits in bits [s*b, s*b + b);
 *                       stream bit i is bit (i % 32) of word (i / 32); words
 *                       are little-endian uint32, the tail is zero-padded.
 * With 2:4, one group of four 16-bit weights costs 2*16 + 2*2 = 36 bits (8-bit: 20)
 * (+ per-row padding to a whole word when S*b is not a multiple of 32).
 */
nm_status nm_packed_sizes(int64_t R, int64_t K, int n, int m, int dtype,
                          size_t* values_bytes, size_t* idx_bytes, int64_t* idx_row_words);

/*
 * Prune + pack (magnitude top-N of every M along the rows of W).
 *   W       device, [R, K] row-major, leading dimension ldw >= K (elements),
 *           dtype NM_F16, NM_BF16, NM_I8 or NM_FP8 (see above).
 *   values  device, [R, S] contiguous, same dtype (written).
 *   idx     device, [R, idx_row_words] uint32 contiguous (written, padding
 *           bits zero).
 * Selection: magnitude is compared on the stored 16-bit pattern with the sign
 * bit cleared (bits & 0x7FFF), so +0/-0 tie and +x/-x tie; the N largest keys
 * of a group are kept, equal keys going to the lower position.  Exactly N
 * slots are stored per group even when the group holds fewer non-zeros.
 * Supported (n, m): (2, 4), (1, 4), (1, 8).  K % 16 == 0 and K % m == 0.
 * Alignment: W, values and idx 16-byte aligned; ldw % 8 == 0.
 */
nm_status nm_compress(const void* W, int64_t R, int64_t K, int64_t ldw, int dtype, int n, int m,
                      void* values, uint32_t* idx, void* stream);

/*
 * Decompress: dense W_nm [R, K] (leading dimension ldw) with the survivors
 * back in place and zeros elsewhere.  Same format rules as nm_compress.
 */
nm_status nm_decompress(const void* values, const uint32_t* idx, int64_t R, int64_t K, int n,
                        int m, int dtype, void* W_out, int64_t ldw, void* stream);

/*
 * Sparse GEMM  Y = W_nm X,  X = act^T.
 *   values, idx  packed W (see nm_packed_sizes), dtype NM_F16, NM_BF16, NM_I8 or
 *                NM_FP8.
 *   act          device, [T, K] row-major (each token's K features contiguous),
 *                leading dimension ldx >= K, same dtype as values.
 *   Y            device, [T, R] row-major, leading dimension ldy >= R, i.e. the
 *                transpose of Y = W_nm X (the layout of a linear layer's output);
 *                out_dtype NM_F32 (default) or the input dtype (RNE rounded);
 *                NM_I32 for NM_I8 (exact); NM_F32 only for NM_FP8.
 *   Y[t, r] = sum_k W_nm[r, k] * act[t, k], products and sums in fp32.
 * Shapes: R >= 1, T >= 0 (T == 0 enqueues nothing), K >= 16, K % 16 == 0,
 * K % m == 0.  Alignment: every pointer 16-byte aligned, ldx % 8 == 0 (ldy
 * is free).  Y must not overlap values, idx or act (NM_ERR_ALIAS).
 */
nm_status nm_spmm(const void* values, const uint32_t* idx, int64_t R, int64_t K, int n, int m,
                  int dtype, const void* act, int64_t T, int64_t ldx, void* Y, int64_t ldy,
                  int out_dtype, void* stream);

/*
 * Permuted sparse GEMM  y = (W Pi) x:  Y[t, r] = sum_k W_nm[r, k] * act[t, perm[k]]
 * (ShuffleSparse, inference with a learned input-channel permutation).
 *   perm  device int32 [K], a permutation of 0..K-1 (precondition, not checked
 *         on the hot path; an out-of-range entry gives wrong values for its
 *         column, never an out-of-bounds access).
 * All other arguments as nm_spmm.  By default (nm_set_variant 0) the
 * permutation is applied as an index map while X is read by a gather pass
 * that writes X' = act[:, perm] (T * K * 2 bytes) to scratch memory, followed
 * by the plain GEMM on X'.  The library keeps one scratch buffer per (device,
 * stream), grown to the largest T * K * 2 seen on that stream and held until
 * the process ends; growing it synchronises that stream.  Variants 1 and 3
 * gather inside the GEMM kernel instead (no scratch).  NM_ERR_HIP if the
 * scratch cannot be allocated.
 */
nm_status nm_spmm_perm(const void* values, const uint32_t* idx, int64_t R, int64_t K, int n, int m,
                       int dtype, const void* act, int64_t T, int64_t ldx, const int32_t* perm,
                       void* Y, int64_t ldy, int out_dtype, void* stream);

/*
 * Host-side check that perm is a permutation of 0..K-1 (copies perm to the
 * host and synchronises `stream`).  NM_ERR_SHAPE if it is not.  Debug aid.
 */
nm_status nm_check_perm(const int32_t* perm, int64_t K, void* stream);

/*
 * Kernel family for nm_spmm / nm_spmm_perm, process-wide (ablations, tests).
 *   0  choose by shape (default)
 *   1  generic tiled kernel (LDS-staged operands, any shape)
 *   2  register-prefetch pipelined kernel (K % 64 == 0, T >= 64, R >= 128)
 *   3  all-LDS direct-load kernels (2:4; K % 128 == 0; the permuted one also
 *      K <= 768)
 *   4  few-token kernel (T <= 16, K <= 4096)
 *   5  all-LDS direct-load kernel with 256 x 256 tiles (2:4; K % 128 == 0,
 *      T >= 256, R >= 256)
 *   6  all-LDS direct-load kernel with 128 x 64 tiles (1:4 and 1:8;
 *      K % 256 == 0, T >= 64, R >= 128)
 * For 8-bit weights there are two: the LDS-staged kernel (whole 256 x 128 tiles,
 * K % 128 == 0) and, for variant 1 or any other shape, a kernel that loads
 * its operands straight into registers.
 * A forced family that does not take the shape falls back to the choice by
 * shape.  Every family computes the same product; all but 4 add the K steps
 * in the same order and give the same bits.  NM_ERR_UNSUPPORTED outside 0..6.
 */
nm_status nm_set_variant(int variant);

#ifdef __cplusplus
}
#endif

#endif /* NMSPARSE_H */
