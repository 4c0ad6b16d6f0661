// Internal declarations shared by the host API and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "nmsparse.h"

namespace nm {

enum { NM_VARIANT_AUTO = 0, NM_VARIANT_GENERIC = 1, NM_VARIANT_PIPE = 2, NM_VARIANT_LDS = 3,
       NM_VARIANT_DECODE = 4, NM_VARIANT_RESIDENT = 5, NM_VARIANT_LDS_NM = 6, NM_VARIANT_MAX = 6 };

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
  void* workspace;       // permuted product: caller memory for X' = act[:, perm], or null
  size_t workspace_bytes;
};

hipError_t launch_spmm(const SpmmArgs& a, hipStream_t s);
// Training-side products (nm_train.hip): dX = G W_nm and the packed dW.
struct TrainArgs {
  const uint16_t* values;  // packed W (dX only)
  size_t values_bytes;
  const uint32_t* idx;     // index words of the packed W
  size_t idx_bytes;
  int64_t R, K;
  int n, m;
  int dtype;               // NM_F16 / NM_BF16
  int64_t idx_row_words;
  const uint16_t* G;       // [T, R], ldg: gradient of the forward output
  int64_t T, ldg;
  const uint16_t* act;     // [T, K], ldx (dW only)
  int64_t ldx;
  void* out;               // dX [T, K] (ldo) or dW [R, S] (contiguous)
  int64_t ldo;
  int out_dtype;           // NM_F32 or dtype
};
hipError_t launch_spmm_dx(const TrainArgs& a, hipStream_t s);
hipError_t launch_spmm_dw(const TrainArgs& a, hipStream_t s);

// 8-bit 2:4 GEMM (nm_int8.hip): Y int32 for NM_I8, fp32 for NM_FP8.
hipError_t launch_spmm_i8(const SpmmArgs& a, hipStream_t s);

// Pipelined large-tile kernel (nm_spmm_pipe.hip) and the shapes it takes.
bool spmm_pipe_applies(const SpmmArgs& a);
hipError_t launch_spmm_pipe(const SpmmArgs& a, hipStream_t s);

// Few-token kernel (nm_spmm_decode.hip) and the shapes it takes.
bool spmm_decode_applies(const SpmmArgs& a);
hipError_t launch_spmm_decode(const SpmmArgs& a, hipStream_t s);

// Permuted product as a gather pass X' = act[:, perm] into the caller's
// workspace followed by the plain GEMM on X' (nm_permute.hip): the bytes it
// needs (0 when the shape does not take it), and the launch.
size_t spmm_perm_gather_bytes(int64_t T, int64_t K, int dtype);
hipError_t launch_spmm_perm_gather(const SpmmArgs& a, void* workspace, hipStream_t s);

// The file-scope device array nm_spmm_perm_static uses as its workspace
// (nm_permute.hip): its size, and its address on the current device.
constexpr size_t kStaticWorkspaceBytes = size_t(32) << 20;
hipError_t static_workspace(void** ptr);

// 2:4 kernel with the token tile resident in LDS, plain or through the index
// map (nm_spmm_resident.hip), and the shapes it takes.
bool spmm_resident_applies(const SpmmArgs& a);
hipError_t launch_spmm_resident(const SpmmArgs& a, hipStream_t s);

// All-LDS 2:4 kernel (nm_spmm_lds.hip) and the shapes it takes.
bool spmm_lds_applies(const SpmmArgs& a);
hipError_t launch_spmm_lds(const SpmmArgs& a, hipStream_t s);

// All-LDS 1:4 / 1:8 kernel with 128 x 64 tiles (nm_spmm_lds_nm.hip) and the
// shapes it takes.
bool spmm_lds_nm_applies(const SpmmArgs& a);
hipError_t launch_spmm_lds_nm(const SpmmArgs& a, hipStream_t s);

// Hybrid dense / 2:4 weight tiles (nm_hybrid.hip): pack and product.  The
// layout tables are device arrays as nm_hybrid_layout writes them; values_bytes
// and idx_bytes bound every weight access (both below 2^32).
struct HybridArgs {
  const uint16_t* values = nullptr;   // product: packed weights
  const uint8_t* idx = nullptr;
  const int64_t* tile_meta = nullptr;
  const int64_t* row_meta = nullptr;
  int64_t R = 0, K = 0, tile_rows = 0, tile_cols = 0;
  int dtype = 0;
  uint64_t values_bytes = 0, idx_bytes = 0;
  const uint16_t* act = nullptr;      // product: activations and output
  int64_t T = 0, ldx = 0;
  void* Y = nullptr;
  int64_t ldy = 0;
  int out_dtype = 0;
  const uint16_t* W = nullptr;        // pack: dense weights and packed outputs
  int64_t ldw = 0;
  uint16_t* values_out = nullptr;
  uint8_t* idx_out = nullptr;
};
constexpr int64_t kHybridMaxTileCols = 8192;  // tile-columns per row the product takes
hipError_t launch_hybrid_pack(const HybridArgs& a, hipStream_t s);
hipError_t launch_hybrid_spmm(const HybridArgs& a, hipStream_t s);

// The column permutation on block-sparse and diagonal-sparse weights
// (nm_hosts.hip).  values_bytes and act_bytes bound the weight and activation
// reads (both below 2^32); row_ptr / col entries are clamped into range on the
// device, so a malformed structure gives wrong sums but no stray access.
struct HostArgs {
  bool diagonal = false;
  const uint16_t* values = nullptr;
  uint64_t values_bytes = 0;
  const int32_t* row_ptr = nullptr;   // block
  const int32_t* col = nullptr;
  const int32_t* offsets = nullptr;   // diagonal
  int64_t nnz = 0;                    // kept blocks, or diagonals
  int64_t R = 0, K = 0;
  int dtype = 0;
  const uint16_t* act = nullptr;
  uint64_t act_bytes = 0;
  int64_t ldx = 0, T = 0;
  const int32_t* perm = nullptr;      // NULL: act read as it is
  void* out = nullptr;
  int64_t ldy = 0;
  int out_dtype = 0;
};
constexpr int64_t kDiagMaxK = 1792;   // the diagonal product stages 80 bytes per column (and the offsets) in LDS
hipError_t launch_block_pack(const uint16_t* W, int64_t ldw, int64_t R, int64_t K, const int32_t* row_ptr,
                             const int32_t* col, int64_t nnzb, uint16_t* values, hipStream_t s);
hipError_t launch_diag_pack(const uint16_t* W, int64_t ldw, int64_t R, int64_t K, const int32_t* offsets, int64_t D,
                            uint16_t* values, hipStream_t s);
hipError_t launch_host_spmm(const HostArgs& a, hipStream_t s);

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
