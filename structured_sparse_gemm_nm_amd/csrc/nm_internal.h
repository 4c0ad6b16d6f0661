// Internal declarations shared by the host API and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "nmsparse.h"

namespace nm {

enum { NM_VARIANT_AUTO = 0, NM_VARIANT_GENERIC = 1, NM_VARIANT_PIPE = 2, NM_VARIANT_LDS = 3,
       NM_VARIANT_DECODE = 4, NM_VARIANT_WIDE = 5, NM_VARIANT_LDS_NM = 6, NM_VARIANT_MAX = 6 };

// Launchers (defined next to their kernels).  Arguments are already
// validated; each returns the hipError_t of its launch.
hipError_t launch_prune_pack(const uint16_t* W, int64_t R, int64_t K, int64_t ldw, int n, int m,
                             uint16_t* values, uint32_t* idx, int64_t idx_row_words,
                             hipStream_t s);

hipError_t launch_decompress(const uint16_t* values, const uint32_t* idx, int64_t R, int64_t K,
                             int n, int m, int64_t idx_row_words, uint16_t* W, int64_t ldw,
                             hipStream_t s);

// 8-bit 2:4 (nm_int8.hip): prune + pack, decompress (leading dimensions in
// bytes, multiples of 16; K % 32 == 0).  f8: FP8 E4M3 keys (bits & 0x7F)
// instead of int8 |w|; decompress moves bytes and serves both.
hipError_t launch_prune_pack_i8(const uint8_t* W, int64_t R, int64_t K, int64_t ldw, uint8_t* values,
                                uint32_t* idx, int64_t idx_row_words, bool f8, hipStream_t s);
hipError_t launch_decompress_i8(const uint8_t* values, const uint32_t* idx, int64_t R, int64_t K,
                                int64_t idx_row_words, uint8_t* W, int64_t ldw, hipStream_t s);

struct SpmmArgs {
  const uint16_t* values;
  const uint32_t* idx;
  int64_t R, K;
  int n, m;
  int dtype;             // NM_F16 / NM_BF16 / NM_I8 / NM_FP8 (the last two: bytes)
  const uint16_t* act;   // [T, K], ldx (elements)
  int64_t T, ldx;
  const int32_t* perm;   // nullptr: identity
  void* Y;               // [T, R], ldy
  int64_t ldy;
  int out_dtype;         // NM_F32 or dtype
  int64_t idx_row_words;
  int variant;           // NM_VARIANT_* (0 = choose by shape)
};

hipError_t launch_spmm(const SpmmArgs& a, hipStream_t s);
// 8-bit 2:4 GEMM (nm_int8.hip): Y int32 for NM_I8, fp32 for NM_FP8.
hipError_t launch_spmm_i8(const SpmmArgs& a, hipStream_t s);

// Pipelined large-tile kernel (nm_spmm_pipe.hip) and the shapes it takes.
bool spmm_pipe_applies(const SpmmArgs& a);
hipError_t launch_spmm_pipe(const SpmmArgs& a, hipStream_t s);

// Few-token kernel (nm_spmm_decode.hip) and the shapes it takes.
bool spmm_decode_applies(const SpmmArgs& a);
hipError_t launch_spmm_decode(const SpmmArgs& a, hipStream_t s);

// Permuted 2:4 kernel gathering from LDS (nm_spmm_perm.hip) and its shapes.
bool spmm_perm_lds_applies(const SpmmArgs& a);
hipError_t launch_spmm_perm_lds(const SpmmArgs& a, hipStream_t s);

// All-LDS 2:4 kernel (nm_spmm_lds.hip) and the shapes it takes.
bool spmm_lds_applies(const SpmmArgs& a);
hipError_t launch_spmm_lds(const SpmmArgs& a, hipStream_t s);

// All-LDS 1:4 / 1:8 kernel with 128 x 64 tiles (nm_spmm_lds_nm.hip) and the
// shapes it takes.
bool spmm_lds_nm_applies(const SpmmArgs& a);
hipError_t launch_spmm_lds_nm(const SpmmArgs& a, hipStream_t s);

// Permuted GEMM as a gather pass into stream-ordered scratch followed by the
// plain GEMM (nm_permute.hip), and the shapes it takes.
bool spmm_perm_gather_applies(const SpmmArgs& a);
hipError_t launch_spmm_perm_gather(const SpmmArgs& a, hipStream_t s);

// 256 x 256-tile 2:4 kernel (nm_spmm_wide.hip) and the shapes it takes.
bool spmm_wide_applies(const SpmmArgs& a);
hipError_t launch_spmm_wide(const SpmmArgs& a, hipStream_t s);

// Device properties and per-kernel launch set-up, kept per device and safe to
// call from several host threads (nm_api.cpp).
int device_cu_count();                 // CUs of the current device (256 if the query fails)
int device_max_lds();                  // its largest workgroup LDS allocation (0 if the query fails)
// Allow kern up to `bytes` of dynamic LDS on the current device (done once per
// device and kernel).
hipError_t ensure_lds_limit(const void* kern, int bytes);

inline int index_bits(int m) {
  int b = 0;
  while ((1 << b) < m) ++b;
  return b < 1 ? 1 : b;
}

}  // namespace nm
