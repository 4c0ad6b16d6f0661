/*
 * nmsparse.h -- N:M structured weight sparsity on AMD Instinct MI355X (gfx950).
 *
 * A C ABI over plain pointers and sizes.  Every device pointer is HIP device
 * memory owned by the caller; no entry point allocates device or host memory,
 * synchronises the caller's stream (nm_check_perm excepted, a debug aid) or
 * keeps state between calls beyond read-only caches of device properties
 * (CU count, LDS limit).  Streams are passed as `void*` holding a hipStream_t
 * (NULL = the legacy default stream).
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
 * 102 adds NM_FP8; 200 replaces the process-wide nm_set_variant by the
 * per-call nm_spmm_variant and gives nm_spmm_perm a caller-owned workspace in
 * place of memory the library allocated; 201 adds the hybrid tiles
 * (nm_hybrid_*), the training products (nm_spmm_dx, nm_spmm_dw) and the
 * block / diagonal structures (nm_block_*, nm_diag_*). */
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
 * (SHUFFLESPARSE technical summary, section 2, and the inference-efficiency
 * item of its technical components: the hardened permutation is a
 * precomputed index map applied while the GEMM reads its input).
 *   perm       device int32 [K], a permutation of 0..K-1 (precondition, not
 *              checked on the hot path; an entry outside [0, K) is clamped into
 *              the row, so it gives a wrong value for its column, never an
 *              out-of-bounds access).
 *   workspace  device memory owned by the caller, or NULL; workspace_bytes its
 *              size.  With at least nm_spmm_perm_workspace_size() bytes, one
 *              gather pass writes X' = act[:, perm] there and the fastest
 *              unpermuted kernel multiplies X' (the workspace is overwritten;
 *              calls that share a workspace must be ordered on one stream).
 *              Otherwise the kernel applies the map as it reads act: the few-
 *              token kernel (T <= 16), the resident-tile kernel (2:4,
 *              K % 256 == 0, K <= 4096: each tile of tokens is staged through
 *              the map once, in LDS, and every weight row streams past it) or
 *              the generic kernel (correct, slower).  Nothing is allocated.
 *              16-byte aligned; must not overlap any other argument
 *              (NM_ERR_ALIAS).
 * All other arguments as nm_spmm.
 */
nm_status nm_spmm_perm(const void* values, const uint32_t* idx, int64_t R, int64_t K, int n, int m,
                       int dtype, const void* act, int64_t T, int64_t ldx, const int32_t* perm,
                       void* Y, int64_t ldy, int out_dtype, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * Workspace bytes nm_spmm_perm uses for its gather pass on this shape (T * K *
 * 2 for 16-bit weights with K % 8 == 0, K <= 65536 and T > 16; 0 when the shape
 * always applies the map inside the kernel).  Pure host arithmetic; same
 * format checks as nm_packed_sizes.
 */
nm_status nm_spmm_perm_workspace_size(int64_t R, int64_t K, int64_t T, int n, int m, int dtype,
                                      size_t* bytes);

/*
 * nm_spmm_perm for callers that cannot allocate memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * product, with the gather pass's workspace taken from a device array the
 * library holds on each GPU it runs on, 32 MiB (33554432 bytes), from first
 * use until the process ends.  Shapes whose workspace (nm_spmm_perm_workspace_size)
 * exceeds 32 MiB are refused with NM_ERR_SHAPE before anything is enqueued;
 * shapes with no gather pass (T <= 16, ...) use no workspace.  Every call on
 * one GPU shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from different threads) race and give wrong results;
 * calls ordered on one stream are safe.  Allocates nothing and synchronises
 * nothing; arguments and errors as nm_spmm_perm.
 */
nm_status nm_spmm_perm_static(const void* values, const uint32_t* idx, int64_t R, int64_t K, int n,
                              int m, int dtype, const void* act, int64_t T, int64_t ldx,
                              const int32_t* perm, void* Y, int64_t ldy, int out_dtype, void* stream);

/*
 * Host-side check that perm is a permutation of 0..K-1 (copies perm to the
 * host and synchronises `stream`).  NM_ERR_SHAPE if it is not.  Debug aid.
 */
nm_status nm_check_perm(const int32_t* perm, int64_t K, void* stream);

/*
 * nm_spmm (perm NULL; workspace ignored) or nm_spmm_perm (perm non-NULL) with
 * the kernel family named by the call (tests and ablations; no state is kept;
 * with a large enough workspace the named family multiplies the gathered X'):
 *   0  choose by shape (what nm_spmm / nm_spmm_perm do)
 *   1  generic tiled kernel (LDS-staged operands, any shape, any map)
 *   2  register-prefetch pipelined kernel (K % 64 == 0, T >= 64, R >= 128;
 *      not permuted)
 *   3  all-LDS direct-load kernel with 256 x 128 tiles (2:4; K % 128 == 0,
 *      T >= 128, R >= 256; not permuted)
 *   4  few-token kernel (T <= 16, K <= 4096)
 *   5  resident-tile kernel (2:4; K % 256 == 0, K <= 4096)
 *   6  all-LDS direct-load kernel with 128 x 64 tiles (1:4 and 1:8;
 *      K % 256 == 0, T >= 64, R >= 128; not permuted)
 * For 8-bit weights there are two: the LDS-staged kernel (whole 256 x 128 tiles,
 * K % 128 == 0) and, for variant 1 or any other shape, a kernel that loads
 * its operands straight into registers.
 * A named family that does not take the shape falls back to the choice by
 * shape.  Every family computes the same product; all but 4 and 6 add the
 * 64-wide K steps in the same order and give the same bits (4 splits K over
 * waves, 6 sums the even and the odd K steps apart and then adds the two:
 * the same result within the fp32 summation bound, and the same bits on
 * every run).
 * NM_ERR_UNSUPPORTED outside 0..6.
 */
nm_status nm_spmm_variant(const void* values, const uint32_t* idx, int64_t R, int64_t K, int n, int m,
                          int dtype, const void* act, int64_t T, int64_t ldx, const int32_t* perm,
                          void* Y, int64_t ldy, int out_dtype, void* workspace, size_t workspace_bytes,
                          int variant, void* stream);

/*
 * Training-side products of an N:M layer.  Source: COE-592 lecture 04-2,
 * "M:N sparsity on NVIDIA tensor cores", section "The recipe", step 3 (the
 * pruned network is retrained with the zeros held fixed, so the pattern
 * survives), and the RNM-TD3 abstract of thelatestinai.com's "Structured
 * Sparsity" cards (row-wise N:M sparsity kept throughout training).  With the
 * forward product Yt[t, r] = sum_k W_nm[r, k] act[t, k] (nm_spmm) and
 * G = dL/dYt, the gradient of the output in Yt's layout:
 *
 * nm_spmm_dx: dX[t, k] = sum_r G[t, r] W_nm[r, k]  (dX = G W_nm, the gradient
 *   of act).
 *   values, idx  packed W (nm_compress), NM_F16 or NM_BF16, patterns as nm_spmm.
 *   G            device [T, R] row-major, ldg >= R, ldg % 8 == 0, dtype of W.
 *   dX           device [T, K] row-major, lddx >= K; out_dtype NM_F32 or the
 *                input dtype (RNE rounded).  Overwritten; with R == 0 it is
 *                filled with zeros.
 *   The reduction runs over R, across W's rows, so the N:M groups give the
 *   matrix cores nothing to skip: the product runs at the dense rate and reads
 *   the packed weights.  Sums in fp32.
 *
 * nm_spmm_dw: dW[r, s] = sum_t G[t, r] act[t, k(r, s)], the gradient of every
 *   stored survivor s of row r (k(r, s) the column it came from), in the
 *   packed values' layout [R, S] (S = K*n/m), contiguous.  Dropped weights are
 *   held at zero and get no gradient; a stored slot that holds a zero is a
 *   weight like any other and gets its gradient.
 *   idx          the packed W's index words (the values are not read).
 *   G            [T, R], ldg as above;  act  [T, K], ldx >= K, ldx % 8 == 0.
 *   dW           device [R, S], out_dtype NM_F32 or the input dtype.
 *                Overwritten; with T == 0 it is filled with zeros.
 *
 * Both: R % 8 == 0 and K % 32 == 0 besides nm_spmm's format rules
 * (NM_ERR_SHAPE); every pointer 16-byte aligned; the output must not overlap
 * an input (NM_ERR_ALIAS); stream-ordered, nothing allocated or synchronised.
 * NM_ERR_UNSUPPORTED for 8-bit weights; NM_ERR_SHAPE for a packed W or index
 * array of 4 GiB or more, a 128-token block of G of 4 GiB or more (dX), or G
 * or act of 4 GiB or more (dW).
 */
nm_status nm_spmm_dx(const void* values, const uint32_t* idx, int64_t R, int64_t K, int n, int m, int dtype,
                     const void* G, int64_t T, int64_t ldg, void* dX, int64_t lddx, int out_dtype, void* stream);
nm_status nm_spmm_dw(const uint32_t* idx, int64_t R, int64_t K, int n, int m, int dtype, const void* G, int64_t T,
                     int64_t ldg, const void* act, int64_t ldx, void* dW, int out_dtype, void* stream);

/*
 * Hybrid dense / 2:4 weight tiles.  Source: thelatestinai.com "Structured
 * Sparsity" topic cards, the PATCH abstract: the weight matrix is cut into
 * tiles and each tile is either kept dense or made 2:4 sparse (the choice is
 * a learned mask, an input here), so the zero fraction can be set anywhere
 * between 0 and 50%; a 2:4 tile is pruned with the nm_compress rule.
 *
 * Tiles are tile_rows x tile_cols blocks on a regular grid (both positive
 * multiples of 64; tile_cols divides K; at most 8192 tile-columns; the last
 * tile-row may be shorter when tile_rows does not divide R).  RB = ceil(R /
 * tile_rows) tile-rows, KB = K / tile_cols tile-columns.
 *   flags[b*KB + j]  host uint8: 1 keeps tile (b, j) dense, 0 makes it 2:4.
 * Packed layout: a row stores its tiles in column order, a dense tile as its
 * tile_cols values (bits unchanged), a 2:4 tile as its tile_cols/2 survivors
 * (the nm_compress format on the tile's columns).  Within every block of 16
 * columns a dense tile stores the values at positions 0 and 1 of the block's
 * four groups of four, then those at positions 2 and 3 (block columns 0 1 4 5
 * 8 9 12 13, then 2 3 6 7 10 11 14 15), the operand order of the two fixed-
 * position 2:4 products a dense step takes.  The row's index bytes are
 * the 2:4 tiles' LSB-first 2-bit streams, tile_cols/8 bytes each, in the
 * same order.  The rows of tile-row b share one length, Lv[b] values and
 * Li[b] index bytes; rows follow each other and tile-rows follow each other,
 * in `values` (dtype of W) and in `idx` (bytes).
 *
 * nm_hybrid_layout (host only, no device access) writes the layout tables:
 *   tile_meta  [RB*KB*2] int64: per tile, the offset of its first value in
 *              the first row of its tile-row (elements into values) and of its
 *              first index byte (bytes into idx), or -1 for a dense tile;
 *   row_meta   [RB*4] int64: per tile-row, Lv, Li and the offsets of its
 *              first value and first index byte;
 *   values_count, idx_bytes  the packed sizes (elements, bytes); the index
 *              array is zero-padded to a multiple of 16 bytes.
 * Any output may be NULL (a size query).  NM_ERR_SHAPE for a bad grid, a flag
 * other than 0 or 1, or packed values or index bytes of 2 GiB or more.
 *
 * nm_hybrid_compress packs W (device, [R, K] row-major, ldw >= K, ldw % 8 ==
 * 0; NM_F16 or NM_BF16) into values / idx (device, caller-allocated with the
 * sizes above); tile_meta / row_meta are the tables of nm_hybrid_layout for
 * the same flags, copied to the device by the caller (8-byte aligned).  idx
 * may be NULL when idx_bytes is 0 (every tile dense).
 *
 * nm_hybrid_spmm computes Y[t, r] = sum_k W_hat[r, k] act[t, k] (fp32
 * accumulation) where W_hat is W with every 2:4 tile pruned: act [T, K]
 * (K <= ldx <= 2^22, ldx % 8 == 0), Y [T, R] (ldy >= R), out_dtype NM_F32 or the
 * input dtype.  On a dense tile each K step runs dense MFMAs, on a 2:4 tile
 * the sparse MFMA.  Layout tables that do not match the packed arrays give
 * wrong values, but every weight access stays inside values_count /
 * idx_bytes.  Same pointer, alignment and alias rules as nm_spmm; nothing is
 * allocated and the stream is not synchronised.
 */
nm_status nm_hybrid_layout(int64_t R, int64_t K, int64_t tile_rows, int64_t tile_cols, const uint8_t* flags,
                           int64_t* tile_meta, int64_t* row_meta, int64_t* values_count, int64_t* idx_bytes);

nm_status nm_hybrid_compress(const void* W, int64_t R, int64_t K, int64_t ldw, int dtype, int64_t tile_rows,
                             int64_t tile_cols, const int64_t* tile_meta, const int64_t* row_meta,
                             int64_t values_count, int64_t idx_bytes, void* values, uint8_t* idx, void* stream);

nm_status nm_hybrid_spmm(const void* values, const uint8_t* idx, const int64_t* tile_meta, const int64_t* row_meta,
                         int64_t R, int64_t K, int64_t tile_rows, int64_t tile_cols, int64_t values_count,
                         int64_t idx_bytes, int dtype, const void* act, int64_t T, int64_t ldx, void* Y,
                         int64_t ldy, int out_dtype, void* stream);

/*
 * The column permutation on two other host structures.  Source: searcharxiv
 * author page, the SHUFFLESPARSE abstract (one learned permutation applied the
 * same way to block, N:M and diagonal structures) and the DynaDiag abstract
 * (a diagonal pattern); gist.science "Technische Samenvatting: SHUFFLESPARSE",
 * section "2. Methodologie" (y = (W Pi) x, W following a fixed structured
 * pattern) and the item "Efficiëntie bij Inferentie" (the hardened Pi as a
 * precomputed index map on the structured kernel's input reads).  The pages
 * name the structures only; the geometry and storage below are this
 * library's.  Both products read act through perm the way nm_spmm_perm does,
 * Y[t, r] = sum_k W[r, k] act[t, perm[k]] (perm NULL: act as it is; an entry
 * outside [0, K) reads column K - 1), with fp32 accumulation; 16-bit weights
 * (NM_F16, NM_BF16) and activations of the same type; Y [T, R] row-major,
 * ldy >= R, out_dtype NM_F32 or the input dtype (RNE).  Every pointer 16-byte
 * aligned, ldx and ldw multiples of 8, outputs not overlapping inputs
 * (NM_ERR_ALIAS); stream-ordered, nothing allocated or synchronised.  act of
 * 4 GiB or more is NM_ERR_SHAPE.
 *
 * Block-sparse: W [R, K] (R and K multiples of 32) cut into 32 x 32 blocks,
 * each kept whole or dropped.  Stored as block-sparse rows:
 *   row_ptr  int32 [R/32 + 1]: the kept blocks of block-row b are entries
 *            row_ptr[b] .. row_ptr[b+1]-1;
 *   col      int32 [nnzb]: their block-columns, ascending within a row;
 *   values   [nnzb][32][32]: each kept block row-major, bits of W unchanged.
 * nm_block_structure (host only, no device access) builds row_ptr and col
 *   from mask[(R/32) * (K/32)] (host uint8, 1 keeps block (b, c) at
 *   b*(K/32) + c); any output may be NULL (a size query); NM_ERR_SHAPE for a
 *   bad shape or a mask entry other than 0 or 1.
 * nm_block_compress copies the kept blocks of W (device, [R, K], ldw >= K)
 *   into values (device, nnzb*2048 bytes); row_ptr and col on the device.
 * nm_block_spmm: Y[t, r] = sum over kept blocks (r/32, c) of
 *   sum_j values[blk][r%32][j] * act[t, perm[32c + j]]; act [T, K], ldx >= K;
 *   perm int32 [K] or NULL.  Runs the kept blocks on the dense matrix cores.
 * Entries of row_ptr or col outside their range are clamped on the device: a
 * malformed structure gives wrong values but no access outside the arrays.
 *
 * Diagonal-sparse: W [R, K] non-zero only on D wrap-around diagonals with
 * distinct offsets o_d in [0, K) (offsets int32 [D], any order; others are
 * reduced mod K, and a repeated offset adds its diagonal twice): row r of
 * diagonal d sits at column (r + o_d) mod K.  Stored as values [D][R],
 * values[d][r] = W[r, (r + o_d) mod K].  K % 8 == 0, K <= 1792, 0 <= D <= K,
 * values below 4 GiB.
 * nm_diag_compress gathers values from W (device, [R, K], ldw >= K).
 * nm_diag_spmm: Y[t, r] = sum_d values[d][r] * act[t, perm[(r + o_d) mod K]].
 *   Every row reads a different activation column per diagonal, so the
 *   product runs on the vector ALUs (fp32 FMA), not the matrix cores.
 */
nm_status nm_block_structure(int64_t R, int64_t K, const uint8_t* mask, int32_t* row_ptr, int32_t* col,
                             int64_t* nnzb);
nm_status nm_block_compress(const void* W, int64_t R, int64_t K, int64_t ldw, int dtype, const int32_t* row_ptr,
                            const int32_t* col, int64_t nnzb, void* values, void* stream);
nm_status nm_block_spmm(const void* values, const int32_t* row_ptr, const int32_t* col, int64_t nnzb, int64_t R,
                        int64_t K, int dtype, const void* act, int64_t T, int64_t ldx, const int32_t* perm,
                        void* Y, int64_t ldy, int out_dtype, void* stream);
nm_status nm_diag_compress(const void* W, int64_t R, int64_t K, int64_t ldw, int dtype, const int32_t* offsets,
                           int64_t D, void* values, void* stream);
nm_status nm_diag_spmm(const void* values, const int32_t* offsets, int64_t D, int64_t R, int64_t K, int dtype,
                       const void* act, int64_t T, int64_t ldx, const int32_t* perm, void* Y, int64_t ldy,
                       int out_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NMSPARSE_H */
