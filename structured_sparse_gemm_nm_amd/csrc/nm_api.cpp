// C ABI of the N:M sparse library: argument validation and dispatch.
//
// Every check runs on the host before the first HIP call, so argument errors
// never touch the device and can be tested without a GPU.
#include <cstdio>
#include <cstdarg>
#include <map>
#include <mutex>
#include <set>
#include <string>
#include <utility>
#include <vector>

#include "nm_internal.h"

namespace {

thread_local std::string g_last_error;

constexpr int64_t kMaxK = int64_t(1) << 24;
constexpr int64_t kMaxRT = int64_t(1) << 30;
constexpr int64_t kMaxElems = int64_t(1) << 40;

nm_status fail(nm_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = std::string(nm_status_string(st)) + ": " + buf;
  return st;
}

nm_status ok() {
  g_last_error.clear();
  return NM_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// One-byte weight types (INT8, FP8 E4M3).
bool byte_type(int dtype) { return dtype == NM_I8 || dtype == NM_FP8; }

bool supported_pattern(int n, int m) {
  return (n == 2 && m == 4) || (n == 1 && m == 4) || (n == 1 && m == 8);
}

// Checks shared by every entry point that names a packed weight.
nm_status check_format(int64_t R, int64_t K, int n, int m, int dtype) {
  if (dtype != NM_F16 && dtype != NM_BF16 && dtype != NM_I8 && dtype != NM_FP8)
    return fail(NM_ERR_UNSUPPORTED, "weight dtype %d is not NM_F16, NM_BF16, NM_I8 or NM_FP8", dtype);
  if (!supported_pattern(n, m))
    return fail(NM_ERR_UNSUPPORTED, "pattern %d:%d is not one of 2:4, 1:4, 1:8", n, m);
  if (byte_type(dtype) && !(n == 2 && m == 4))
    return fail(NM_ERR_UNSUPPORTED, "8-bit weights take the 2:4 pattern only");
  if (R < 0 || R > kMaxRT) return fail(NM_ERR_SHAPE, "R = %lld out of range", (long long)R);
  if (K < 16 || K > kMaxK) return fail(NM_ERR_SHAPE, "K = %lld out of range [16, 2^24]", (long long)K);
  if (K % 16) return fail(NM_ERR_SHAPE, "K = %lld is not a multiple of 16", (long long)K);
  if (byte_type(dtype) && K % 32)
    return fail(NM_ERR_SHAPE, "K = %lld is not a multiple of 32 (8-bit weights)", (long long)K);
  if (K % m) return fail(NM_ERR_SHAPE, "K = %lld is not a multiple of m = %d", (long long)K, m);
  if (R * K > kMaxElems) return fail(NM_ERR_SHAPE, "R*K too large");
  return NM_OK;
}

struct Sizes {
  int64_t S, words;
  size_t values_bytes, idx_bytes;
};

// Bytes per element of a storage type.
size_t elt_bytes(int dtype) { return byte_type(dtype) ? 1 : dtype == NM_F32 || dtype == NM_I32 ? 4 : 2; }

// Leading dimensions (elements) keep every row 16-byte aligned.
int64_t ld_quantum(int dtype) { return byte_type(dtype) ? 16 : 8; }

Sizes sizes_of(int64_t R, int64_t K, int n, int m, int dtype) {
  Sizes z;
  z.S = K / m * n;
  z.words = (z.S * nm::index_bits(m) + 31) / 32;
  z.values_bytes = size_t(R) * size_t(z.S) * elt_bytes(dtype);
  z.idx_bytes = size_t(R) * size_t(z.words) * 4;
  return z;
}

// Byte extent of a row-major [rows, cols] matrix with leading dimension ld.
size_t extent(int64_t rows, int64_t cols, int64_t ld, size_t elt) {
  if (rows <= 0 || cols <= 0) return 0;
  return (size_t(rows - 1) * size_t(ld) + size_t(cols)) * elt;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

nm_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(NM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Tile grid of the hybrid layout: tiles of tile_rows x tile_cols, both
// positive multiples of 64, tile_cols dividing K, at most kHybridMaxTileCols
// tile-columns; R up to 2^30, K up to 2^24.
nm_status check_hybrid_grid(int64_t R, int64_t K, int64_t tile_rows, int64_t tile_cols) {
  if (R < 0 || R > kMaxRT) return fail(NM_ERR_SHAPE, "R = %lld out of range", (long long)R);
  if (K < 64 || K > kMaxK) return fail(NM_ERR_SHAPE, "K = %lld out of range [64, 2^24]", (long long)K);
  if (tile_rows < 64 || tile_rows % 64 || tile_rows > kMaxRT)
    return fail(NM_ERR_SHAPE, "tile_rows = %lld is not a positive multiple of 64", (long long)tile_rows);
  if (tile_cols < 64 || tile_cols % 64 || K % tile_cols)
    return fail(NM_ERR_SHAPE, "tile_cols = %lld is not a multiple of 64 dividing K = %lld",
                (long long)tile_cols, (long long)K);
  if (K / tile_cols > nm::kHybridMaxTileCols)
    return fail(NM_ERR_SHAPE, "K / tile_cols = %lld tile-columns exceeds %lld", (long long)(K / tile_cols),
                (long long)nm::kHybridMaxTileCols);
  return NM_OK;
}

// Sizes of the packed hybrid arrays: the kernels address them with 32-bit
// byte offsets and use offsets from 2^31 up as "outside".
nm_status check_hybrid_totals(int64_t values_count, int64_t idx_bytes) {
  if (values_count < 0 || idx_bytes < 0) return fail(NM_ERR_SHAPE, "negative packed size");
  if (values_count * 2 >= (int64_t(1) << 31) || idx_bytes >= (int64_t(1) << 31))
    return fail(NM_ERR_SHAPE, "packed hybrid weight of %lld values / %lld index bytes reaches 2 GiB",
                (long long)values_count, (long long)idx_bytes);
  return NM_OK;
}

bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

nm_status spmm_common(const void* values, const uint32_t* idx, int64_t R, int64_t K, int n, int m,
                      int dtype, const void* act, int64_t T, int64_t ldx, const int32_t* perm,
                      bool want_perm, void* Y, int64_t ldy, int out_dtype, void* workspace,
                      size_t workspace_bytes, int variant, void* stream, bool static_ws = false) {
  nm_status st = check_format(R, K, n, m, dtype);
  if (st != NM_OK) return st;
  if (variant < 0 || variant > nm::NM_VARIANT_MAX)
    return fail(NM_ERR_UNSUPPORTED, "kernel family %d is not 0..%d", variant, int(nm::NM_VARIANT_MAX));
  if (T < 0 || T > kMaxRT) return fail(NM_ERR_SHAPE, "T = %lld out of range", (long long)T);
  if (dtype == NM_I8 || dtype == NM_FP8) {
    const int want = dtype == NM_I8 ? NM_I32 : NM_F32;
    if (out_dtype != want)
      return fail(NM_ERR_UNSUPPORTED, "%s weights give an %s output", dtype == NM_I8 ? "int8" : "fp8",
                  dtype == NM_I8 ? "NM_I32" : "NM_F32");
    if (want_perm) return fail(NM_ERR_UNSUPPORTED, "nm_spmm_perm does not take 8-bit weights");
  } else if (out_dtype != NM_F32 && out_dtype != dtype) {
    return fail(NM_ERR_UNSUPPORTED, "out_dtype %d must be NM_F32 or the input dtype", out_dtype);
  }
  if (ldx < K) return fail(NM_ERR_STRIDE, "ldx = %lld < K = %lld", (long long)ldx, (long long)K);
  if (ldy < R) return fail(NM_ERR_STRIDE, "ldy = %lld < R = %lld", (long long)ldy, (long long)R);
  // bounded before any product of sizes below, so no int64 product overflows
  if (ldx > kMaxElems || ldy > kMaxElems)
    return fail(NM_ERR_SHAPE, "leading dimension above 2^40 elements");
  if (R == 0 || T == 0) return ok();  // empty product: nothing to enqueue
  if (!values || !idx || !act || !Y || (want_perm && !perm))
    return fail(NM_ERR_NULL, "values, idx, act, Y%s must be non-NULL", want_perm ? ", perm" : "");
  if (ldx % ld_quantum(dtype))
    return fail(NM_ERR_ALIGN, "ldx = %lld is not a multiple of %lld", (long long)ldx,
                (long long)ld_quantum(dtype));
  if (!aligned16(values) || !aligned16(idx) || !aligned16(act) || !aligned16(Y) ||
      (want_perm && !aligned16(perm)))
    return fail(NM_ERR_ALIGN, "device pointers must be 16-byte aligned");
  if (T * ldx > kMaxElems || T * ldy > kMaxElems) return fail(NM_ERR_SHAPE, "T*ld too large");
  Sizes z = sizes_of(R, K, n, m, dtype);
  size_t ybytes = extent(T, R, ldy, elt_bytes(out_dtype));
  const size_t abytes = extent(T, K, ldx, elt_bytes(dtype));
  if (overlaps(Y, ybytes, values, z.values_bytes) || overlaps(Y, ybytes, idx, z.idx_bytes) ||
      overlaps(Y, ybytes, act, abytes) || (want_perm && overlaps(Y, ybytes, perm, size_t(K) * 4)))
    return fail(NM_ERR_ALIAS, "Y overlaps an input");
  if (static_ws) {
    // the library's own array: a size it cannot hold is refused (before any
    // HIP call); its address is looked up only once validation has passed
    const size_t need = nm::spmm_perm_gather_bytes(T, K, dtype);
    if (need > nm::kStaticWorkspaceBytes)
      return fail(NM_ERR_SHAPE, "T*K*2 = %zu bytes exceeds the static workspace (%zu bytes)", need,
                  nm::kStaticWorkspaceBytes);
    workspace = nullptr;
    workspace_bytes = 0;
    if (need > 0) {
      const hipError_t e = nm::static_workspace(&workspace);
      if (e != hipSuccess) return hip_status(e, "static workspace address");
      workspace_bytes = nm::kStaticWorkspaceBytes;
    }
  } else if (workspace_bytes == 0) {
    workspace = nullptr;
  }
  if (workspace && !static_ws) {
    if (!aligned16(workspace)) return fail(NM_ERR_ALIGN, "workspace must be 16-byte aligned");
    if (overlaps(workspace, workspace_bytes, Y, ybytes) || overlaps(workspace, workspace_bytes, act, abytes) ||
        overlaps(workspace, workspace_bytes, values, z.values_bytes) ||
        overlaps(workspace, workspace_bytes, idx, z.idx_bytes) ||
        (want_perm && overlaps(workspace, workspace_bytes, perm, size_t(K) * 4)))
      return fail(NM_ERR_ALIAS, "workspace overlaps an argument");
  }

  nm::SpmmArgs a;
  a.values = static_cast<const uint16_t*>(values);
  a.idx = idx;
  a.R = R;
  a.K = K;
  a.n = n;
  a.m = m;
  a.dtype = dtype;
  a.act = static_cast<const uint16_t*>(act);
  a.T = T;
  a.ldx = ldx;
  a.perm = want_perm ? perm : nullptr;
  a.Y = Y;
  a.ldy = ldy;
  a.out_dtype = out_dtype;
  a.idx_row_words = z.words;
  a.variant = variant;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  return hip_status(nm::launch_spmm(a, static_cast<hipStream_t>(stream)), "nm_spmm launch");
}

}  // namespace

namespace nm {
namespace {

std::mutex g_dev_mu;

int cached_attr(std::map<int, int>& cache, hipDeviceAttribute_t attr, int fallback) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fallback;
  std::lock_guard<std::mutex> g(g_dev_mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int v = 0;
  if (hipDeviceGetAttribute(&v, attr, dev) != hipSuccess || v <= 0) v = fallback;
  cache[dev] = v;
  return v;
}

}  // namespace

int device_cu_count() {
  static std::map<int, int> cache;
  return cached_attr(cache, hipDeviceAttributeMultiprocessorCount, 256);
}

int device_max_lds() {
  static std::map<int, int> cache;
  return cached_attr(cache, hipDeviceAttributeMaxSharedMemoryPerBlock, 0);
}

hipError_t ensure_lds_limit(const void* kern, int bytes) {
  static std::set<std::pair<int, const void*>> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> g(g_dev_mu);
  if (done.count({dev, kern})) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.insert({dev, kern});
  return e;
}

}  // namespace nm

extern "C" {

int nm_version(void) { return 201; }

const char* nm_status_string(int status) {
  switch (status) {
    case NM_OK: return "NM_OK";
    case NM_ERR_NULL: return "NM_ERR_NULL";
    case NM_ERR_SHAPE: return "NM_ERR_SHAPE";
    case NM_ERR_UNSUPPORTED: return "NM_ERR_UNSUPPORTED";
    case NM_ERR_STRIDE: return "NM_ERR_STRIDE";
    case NM_ERR_ALIAS: return "NM_ERR_ALIAS";
    case NM_ERR_HIP: return "NM_ERR_HIP";
    case NM_ERR_ALIGN: return "NM_ERR_ALIGN";
    default: return "NM_ERR_UNKNOWN";
  }
}

const char* nm_last_error(void) { return g_last_error.c_str(); }

nm_status nm_packed_sizes(int64_t R, int64_t K, int n, int m, int dtype, size_t* values_bytes,
                          size_t* idx_bytes, int64_t* idx_row_words) {
  nm_status st = check_format(R, K, n, m, dtype);
  if (st != NM_OK) return st;
  Sizes z = sizes_of(R, K, n, m, dtype);
  if (values_bytes) *values_bytes = z.values_bytes;
  if (idx_bytes) *idx_bytes = z.idx_bytes;
  if (idx_row_words) *idx_row_words = z.words;
  return ok();
}

nm_status nm_compress(const void* W, int64_t R, int64_t K, int64_t ldw, int dtype, int n, int m,
                      void* values, uint32_t* idx, void* stream) {
  nm_status st = check_format(R, K, n, m, dtype);
  if (st != NM_OK) return st;
  if (ldw < K) return fail(NM_ERR_STRIDE, "ldw = %lld < K = %lld", (long long)ldw, (long long)K);
  if (ldw > kMaxElems) return fail(NM_ERR_SHAPE, "ldw above 2^40 elements");
  if (R == 0) return ok();
  if (!W || !values || !idx) return fail(NM_ERR_NULL, "W, values and idx must be non-NULL");
  if (ldw % ld_quantum(dtype))
    return fail(NM_ERR_ALIGN, "ldw = %lld is not a multiple of %lld", (long long)ldw,
                (long long)ld_quantum(dtype));
  if (!aligned16(W) || !aligned16(values) || !aligned16(idx))
    return fail(NM_ERR_ALIGN, "device pointers must be 16-byte aligned");
  if (R * ldw > kMaxElems) return fail(NM_ERR_SHAPE, "R*ldw too large");
  Sizes z = sizes_of(R, K, n, m, dtype);
  size_t wbytes = extent(R, K, ldw, elt_bytes(dtype));
  if (overlaps(values, z.values_bytes, W, wbytes) || overlaps(idx, z.idx_bytes, W, wbytes) ||
      overlaps(values, z.values_bytes, idx, z.idx_bytes))
    return fail(NM_ERR_ALIAS, "outputs overlap each other or W");
  if (byte_type(dtype))
    return hip_status(nm::launch_prune_pack_i8(static_cast<const uint8_t*>(W), R, K, ldw,
                                               static_cast<uint8_t*>(values), idx, z.words,
                                               dtype == NM_FP8, static_cast<hipStream_t>(stream)),
                      "nm_compress launch");
  return hip_status(nm::launch_prune_pack(static_cast<const uint16_t*>(W), R, K, ldw, n, m,
                                          static_cast<uint16_t*>(values), idx, z.words,
                                          static_cast<hipStream_t>(stream)),
                    "nm_compress launch");
}

nm_status nm_decompress(const void* values, const uint32_t* idx, int64_t R, int64_t K, int n,
                        int m, int dtype, void* W_out, int64_t ldw, void* stream) {
  nm_status st = check_format(R, K, n, m, dtype);
  if (st != NM_OK) return st;
  if (ldw < K) return fail(NM_ERR_STRIDE, "ldw = %lld < K = %lld", (long long)ldw, (long long)K);
  if (ldw > kMaxElems) return fail(NM_ERR_SHAPE, "ldw above 2^40 elements");
  if (R == 0) return ok();
  if (!W_out || !values || !idx) return fail(NM_ERR_NULL, "values, idx and W_out must be non-NULL");
  if (ldw % ld_quantum(dtype))
    return fail(NM_ERR_ALIGN, "ldw = %lld is not a multiple of %lld", (long long)ldw,
                (long long)ld_quantum(dtype));
  if (!aligned16(W_out) || !aligned16(values) || !aligned16(idx))
    return fail(NM_ERR_ALIGN, "device pointers must be 16-byte aligned");
  if (R * ldw > kMaxElems) return fail(NM_ERR_SHAPE, "R*ldw too large");
  Sizes z = sizes_of(R, K, n, m, dtype);
  size_t wbytes = extent(R, K, ldw, elt_bytes(dtype));
  if (overlaps(W_out, wbytes, values, z.values_bytes) || overlaps(W_out, wbytes, idx, z.idx_bytes))
    return fail(NM_ERR_ALIAS, "W_out overlaps an input");
  if (byte_type(dtype))
    return hip_status(nm::launch_decompress_i8(static_cast<const uint8_t*>(values), idx, R, K, z.words,
                                               static_cast<uint8_t*>(W_out), ldw,
                                               static_cast<hipStream_t>(stream)),
                      "nm_decompress launch");
  return hip_status(nm::launch_decompress(static_cast<const uint16_t*>(values), idx, R, K, n, m,
                                          z.words, static_cast<uint16_t*>(W_out), ldw,
                                          static_cast<hipStream_t>(stream)),
                    "nm_decompress launch");
}

nm_status nm_spmm(const void* values, const uint32_t* idx, int64_t R, int64_t K, int n, int m,
                  int dtype, const void* act, int64_t T, int64_t ldx, void* Y, int64_t ldy,
                  int out_dtype, void* stream) {
  return spmm_common(values, idx, R, K, n, m, dtype, act, T, ldx, nullptr, false, Y, ldy,
                     out_dtype, nullptr, 0, 0, stream);
}

nm_status nm_spmm_perm_workspace_size(int64_t R, int64_t K, int64_t T, int n, int m, int dtype,
                                      size_t* bytes) {
  nm_status st = check_format(R, K, n, m, dtype);
  if (st != NM_OK) return st;
  if (T < 0 || T > kMaxRT) return fail(NM_ERR_SHAPE, "T = %lld out of range", (long long)T);
  if (!bytes) return fail(NM_ERR_NULL, "bytes must be non-NULL");
  *bytes = R == 0 ? 0 : nm::spmm_perm_gather_bytes(T, K, dtype);
  return ok();
}

nm_status nm_spmm_perm(const void* values, const uint32_t* idx, int64_t R, int64_t K, int n, int m,
                       int dtype, const void* act, int64_t T, int64_t ldx, const int32_t* perm,
                       void* Y, int64_t ldy, int out_dtype, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return spmm_common(values, idx, R, K, n, m, dtype, act, T, ldx, perm, true, Y, ldy, out_dtype,
                     workspace, workspace_bytes, 0, stream);
}

nm_status nm_spmm_perm_static(const void* values, const uint32_t* idx, int64_t R, int64_t K, int n,
                              int m, int dtype, const void* act, int64_t T, int64_t ldx,
                              const int32_t* perm, void* Y, int64_t ldy, int out_dtype, void* stream) {
  return spmm_common(values, idx, R, K, n, m, dtype, act, T, ldx, perm, true, Y, ldy, out_dtype,
                     nullptr, 0, 0, stream, true);
}

nm_status nm_spmm_variant(const void* values, const uint32_t* idx, int64_t R, int64_t K, int n, int m,
                          int dtype, const void* act, int64_t T, int64_t ldx, const int32_t* perm,
                          void* Y, int64_t ldy, int out_dtype, void* workspace, size_t workspace_bytes,
                          int variant, void* stream) {
  return spmm_common(values, idx, R, K, n, m, dtype, act, T, ldx, perm, perm != nullptr, Y, ldy,
                     out_dtype, workspace, workspace_bytes, variant, stream);
}

nm_status nm_check_perm(const int32_t* perm, int64_t K, void* stream) {
  if (K < 1 || K > kMaxK) return fail(NM_ERR_SHAPE, "K = %lld out of range", (long long)K);
  if (!perm) return fail(NM_ERR_NULL, "perm must be non-NULL");
  std::vector<int32_t> host(static_cast<size_t>(K));
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(host.data(), perm, size_t(K) * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e, "nm_check_perm copy");
  std::vector<char> seen(static_cast<size_t>(K), 0);
  for (int64_t k = 0; k < K; ++k) {
    int32_t p = host[size_t(k)];
    if (p < 0 || p >= K || seen[size_t(p)])
      return fail(NM_ERR_SHAPE, "perm[%lld] = %d breaks the permutation", (long long)k, p);
    seen[size_t(p)] = 1;
  }
  return ok();
}


// Shared checks of the training-side products: format, 16-bit types, output
// dtype, T and the G operand [T, R] (ldg).
static nm_status check_train(int64_t R, int64_t K, int n, int m, int dtype, int64_t T, int64_t ldg,
                             int out_dtype) {
  nm_status st = check_format(R, K, n, m, dtype);
  if (st != NM_OK) return st;
  if (dtype != NM_F16 && dtype != NM_BF16)
    return fail(NM_ERR_UNSUPPORTED, "training products take fp16 or bf16 weights");
  // whole 16-byte pieces of G's rows and whole 32-column segments of W's rows
  if (R % 8 || K % 32)
    return fail(NM_ERR_SHAPE, "training products need R %% 8 == 0 and K %% 32 == 0 (R = %lld, K = %lld)",
                (long long)R, (long long)K);
  if (out_dtype != NM_F32 && out_dtype != dtype)
    return fail(NM_ERR_UNSUPPORTED, "out_dtype %d must be NM_F32 or the input dtype", out_dtype);
  if (T < 0 || T > kMaxRT) return fail(NM_ERR_SHAPE, "T = %lld out of range", (long long)T);
  if (ldg < R) return fail(NM_ERR_STRIDE, "ldg = %lld < R = %lld", (long long)ldg, (long long)R);
  if (ldg > kMaxElems) return fail(NM_ERR_SHAPE, "ldg above 2^40 elements");
  return NM_OK;
}

nm_status nm_spmm_dx(const void* values, const uint32_t* idx, int64_t R, int64_t K, int n, int m, int dtype,
                     const void* G, int64_t T, int64_t ldg, void* dX, int64_t lddx, int out_dtype, void* stream) {
  nm_status st = check_train(R, K, n, m, dtype, T, ldg, out_dtype);
  if (st != NM_OK) return st;
  if (lddx < K) return fail(NM_ERR_STRIDE, "lddx = %lld < K = %lld", (long long)lddx, (long long)K);
  if (lddx > kMaxElems) return fail(NM_ERR_SHAPE, "lddx above 2^40 elements");
  if (T == 0) return ok();  // empty dX: nothing to enqueue (R == 0 writes zeros)
  if (!dX || (R > 0 && (!values || !idx || !G)))
    return fail(NM_ERR_NULL, "values, idx, G and dX must be non-NULL");
  if (ldg % 8) return fail(NM_ERR_ALIGN, "ldg = %lld is not a multiple of 8", (long long)ldg);
  if (!aligned16(values) || !aligned16(idx) || !aligned16(G) || !aligned16(dX))
    return fail(NM_ERR_ALIGN, "device pointers must be 16-byte aligned");
  if (T * ldg > kMaxElems || T * lddx > kMaxElems) return fail(NM_ERR_SHAPE, "T*ld too large");
  Sizes z = sizes_of(R, K, n, m, dtype);
  // the kernel's per-lane byte offsets are 32-bit: the packed arrays and a
  // 128-token block of G
  if (z.values_bytes >= (size_t(1) << 32) || z.idx_bytes >= (size_t(1) << 32) || 128 * ldg * 2 >= (int64_t(1) << 32))
    return fail(NM_ERR_SHAPE, "packed W of 4 GiB or more, or ldg of 2^24 or more");
  const size_t xbytes = extent(T, K, lddx, elt_bytes(out_dtype));
  const size_t gbytes = extent(T, R, ldg, 2);
  if (overlaps(dX, xbytes, values, z.values_bytes) || overlaps(dX, xbytes, idx, z.idx_bytes) ||
      overlaps(dX, xbytes, G, gbytes))
    return fail(NM_ERR_ALIAS, "dX overlaps an input");
  nm::TrainArgs a{};
  a.values = static_cast<const uint16_t*>(values);
  a.values_bytes = z.values_bytes;
  a.idx = idx;
  a.idx_bytes = z.idx_bytes;
  a.R = R;
  a.K = K;
  a.n = n;
  a.m = m;
  a.dtype = dtype;
  a.idx_row_words = z.words;
  a.G = static_cast<const uint16_t*>(G);
  a.T = T;
  a.ldg = ldg;
  a.out = dX;
  a.ldo = lddx;
  a.out_dtype = out_dtype;
  return hip_status(nm::launch_spmm_dx(a, static_cast<hipStream_t>(stream)), "nm_spmm_dx launch");
}

nm_status nm_spmm_dw(const uint32_t* idx, int64_t R, int64_t K, int n, int m, int dtype, const void* G, int64_t T,
                     int64_t ldg, const void* act, int64_t ldx, void* dW, int out_dtype, void* stream) {
  nm_status st = check_train(R, K, n, m, dtype, T, ldg, out_dtype);
  if (st != NM_OK) return st;
  if (ldx < K) return fail(NM_ERR_STRIDE, "ldx = %lld < K = %lld", (long long)ldx, (long long)K);
  if (ldx > kMaxElems) return fail(NM_ERR_SHAPE, "ldx above 2^40 elements");
  if (R == 0) return ok();  // no weights, no gradient (T == 0 writes zeros)
  if (!idx || !dW || (T > 0 && (!G || !act)))
    return fail(NM_ERR_NULL, "idx, G, act and dW must be non-NULL");
  if (ldg % 8 || ldx % 8) return fail(NM_ERR_ALIGN, "ldg and ldx must be multiples of 8");
  if (!aligned16(idx) || !aligned16(G) || !aligned16(act) || !aligned16(dW))
    return fail(NM_ERR_ALIGN, "device pointers must be 16-byte aligned");
  if (T * ldg > kMaxElems || T * ldx > kMaxElems) return fail(NM_ERR_SHAPE, "T*ld too large");
  // per-lane byte offsets are 32-bit: every token row of G and act
  if (T * ldg * 2 >= (int64_t(1) << 32) || T * ldx * 2 >= (int64_t(1) << 32))
    return fail(NM_ERR_SHAPE, "G or act of 4 GiB or more");
  Sizes z = sizes_of(R, K, n, m, dtype);
  if (z.idx_bytes >= (size_t(1) << 32)) return fail(NM_ERR_SHAPE, "index words of 4 GiB or more");
  const size_t wbytes = size_t(R) * size_t(z.S) * elt_bytes(out_dtype);
  const size_t gbytes = extent(T, R, ldg, 2), abytes = extent(T, K, ldx, 2);
  if (overlaps(dW, wbytes, idx, z.idx_bytes) || overlaps(dW, wbytes, G, gbytes) || overlaps(dW, wbytes, act, abytes))
    return fail(NM_ERR_ALIAS, "dW overlaps an input");
  nm::TrainArgs a{};
  a.idx = idx;
  a.idx_bytes = z.idx_bytes;
  a.R = R;
  a.K = K;
  a.n = n;
  a.m = m;
  a.dtype = dtype;
  a.idx_row_words = z.words;
  a.G = static_cast<const uint16_t*>(G);
  a.T = T;
  a.ldg = ldg;
  a.act = static_cast<const uint16_t*>(act);
  a.ldx = ldx;
  a.out = dW;
  a.out_dtype = out_dtype;
  return hip_status(nm::launch_spmm_dw(a, static_cast<hipStream_t>(stream)), "nm_spmm_dw launch");
}

nm_status nm_hybrid_layout(int64_t R, int64_t K, int64_t tile_rows, int64_t tile_cols, const uint8_t* flags,
                           int64_t* tile_meta, int64_t* row_meta, int64_t* values_count, int64_t* idx_bytes) {
  nm_status st = check_hybrid_grid(R, K, tile_rows, tile_cols);
  if (st != NM_OK) return st;
  const int64_t RB = (R + tile_rows - 1) / tile_rows, KB = K / tile_cols;
  if (R > 0 && !flags) return fail(NM_ERR_NULL, "flags must be non-NULL");
  for (int64_t t = 0; t < RB * KB; ++t)
    if (flags[t] > 1)
      return fail(NM_ERR_SHAPE, "flag %lld is %d: flags are 0 (2:4) or 1 (dense)", (long long)t, int(flags[t]));
  int64_t vbase = 0, ibase = 0;
  for (int64_t b = 0; b < RB; ++b) {
    int64_t v = 0, i = 0;  // position along the first row of tile-row b
    for (int64_t j = 0; j < KB; ++j) {
      const bool dense = flags[b * KB + j] != 0;
      if (tile_meta) {
        tile_meta[(b * KB + j) * 2] = vbase + v;
        tile_meta[(b * KB + j) * 2 + 1] = dense ? -1 : ibase + i;
      }
      v += dense ? tile_cols : tile_cols / 2;
      i += dense ? 0 : tile_cols / 8;
    }
    if (row_meta) {
      row_meta[b * 4] = v;
      row_meta[b * 4 + 1] = i;
      row_meta[b * 4 + 2] = vbase;
      row_meta[b * 4 + 3] = ibase;
    }
    const int64_t rows = (b + 1) * tile_rows <= R ? tile_rows : R - b * tile_rows;
    vbase += rows * v;
    ibase += rows * i;
  }
  ibase = (ibase + 15) / 16 * 16;  // whole 16-byte blocks (zero padding)
  st = check_hybrid_totals(vbase, ibase);
  if (st != NM_OK) return st;
  if (values_count) *values_count = vbase;
  if (idx_bytes) *idx_bytes = ibase;
  return ok();
}

nm_status nm_hybrid_compress(const void* W, int64_t R, int64_t K, int64_t ldw, int dtype, int64_t tile_rows,
                             int64_t tile_cols, const int64_t* tile_meta, const int64_t* row_meta,
                             int64_t values_count, int64_t idx_bytes, void* values, uint8_t* idx, void* stream) {
  if (dtype != NM_F16 && dtype != NM_BF16)
    return fail(NM_ERR_UNSUPPORTED, "hybrid tiles take NM_F16 or NM_BF16 weights, not dtype %d", dtype);
  nm_status st = check_hybrid_grid(R, K, tile_rows, tile_cols);
  if (st != NM_OK) return st;
  st = check_hybrid_totals(values_count, idx_bytes);
  if (st != NM_OK) return st;
  if (ldw < K) return fail(NM_ERR_STRIDE, "ldw = %lld < K = %lld", (long long)ldw, (long long)K);
  if (ldw > kMaxElems) return fail(NM_ERR_SHAPE, "ldw above 2^40 elements");
  if (R == 0) return ok();
  if (!W || !values || !tile_meta || !row_meta || (idx_bytes > 0 && !idx))
    return fail(NM_ERR_NULL, "W, values, tile_meta, row_meta (and idx with 2:4 tiles) must be non-NULL");
  if (ldw % 8) return fail(NM_ERR_ALIGN, "ldw = %lld is not a multiple of 8", (long long)ldw);
  if (!aligned16(W) || !aligned16(values) || (idx && !aligned16(idx)) || !aligned8(tile_meta) ||
      !aligned8(row_meta))
    return fail(NM_ERR_ALIGN, "W, values and idx must be 16-byte aligned, the layout tables 8-byte aligned");
  if (R * ldw > kMaxElems) return fail(NM_ERR_SHAPE, "R*ldw too large");
  const int64_t RB = (R + tile_rows - 1) / tile_rows, KB = K / tile_cols;
  const size_t wbytes = extent(R, K, ldw, 2), vbytes = size_t(values_count) * 2, ib = size_t(idx_bytes);
  const size_t tmb = size_t(RB * KB) * 16, rmb = size_t(RB) * 32;
  if (overlaps(values, vbytes, W, wbytes) || overlaps(idx, ib, W, wbytes) || overlaps(values, vbytes, idx, ib) ||
      overlaps(values, vbytes, tile_meta, tmb) || overlaps(values, vbytes, row_meta, rmb) ||
      overlaps(idx, ib, tile_meta, tmb) || overlaps(idx, ib, row_meta, rmb))
    return fail(NM_ERR_ALIAS, "outputs overlap each other, W or the layout tables");
  nm::HybridArgs a;
  a.W = static_cast<const uint16_t*>(W);
  a.ldw = ldw;
  a.R = R;
  a.K = K;
  a.tile_rows = tile_rows;
  a.tile_cols = tile_cols;
  a.dtype = dtype;
  a.tile_meta = tile_meta;
  a.row_meta = row_meta;
  a.values_out = static_cast<uint16_t*>(values);
  a.idx_out = idx;
  a.values_bytes = vbytes;
  a.idx_bytes = ib;
  return hip_status(nm::launch_hybrid_pack(a, static_cast<hipStream_t>(stream)), "nm_hybrid_compress launch");
}

nm_status nm_hybrid_spmm(const void* values, const uint8_t* idx, const int64_t* tile_meta, const int64_t* row_meta,
                         int64_t R, int64_t K, int64_t tile_rows, int64_t tile_cols, int64_t values_count,
                         int64_t idx_bytes, int dtype, const void* act, int64_t T, int64_t ldx, void* Y,
                         int64_t ldy, int out_dtype, void* stream) {
  if (dtype != NM_F16 && dtype != NM_BF16)
    return fail(NM_ERR_UNSUPPORTED, "hybrid tiles take NM_F16 or NM_BF16 weights, not dtype %d", dtype);
  if (out_dtype != NM_F32 && out_dtype != dtype)
    return fail(NM_ERR_UNSUPPORTED, "out_dtype %d must be NM_F32 or the input dtype", out_dtype);
  nm_status st = check_hybrid_grid(R, K, tile_rows, tile_cols);
  if (st != NM_OK) return st;
  st = check_hybrid_totals(values_count, idx_bytes);
  if (st != NM_OK) return st;
  if (T < 0 || T > kMaxRT) return fail(NM_ERR_SHAPE, "T = %lld out of range", (long long)T);
  if (ldx < K) return fail(NM_ERR_STRIDE, "ldx = %lld < K = %lld", (long long)ldx, (long long)K);
  if (ldy < R) return fail(NM_ERR_STRIDE, "ldy = %lld < R = %lld", (long long)ldy, (long long)R);
  if (ldx > kMaxElems || ldy > kMaxElems) return fail(NM_ERR_SHAPE, "leading dimension above 2^40 elements");
  if (ldx > (int64_t(1) << 22))
    return fail(NM_ERR_SHAPE, "ldx = %lld above 2^22 (a token tile's offsets are 31-bit)", (long long)ldx);
  if (R == 0 || T == 0) return ok();
  if (!values || !tile_meta || !row_meta || !act || !Y || (idx_bytes > 0 && !idx))
    return fail(NM_ERR_NULL, "values, tile_meta, row_meta, act, Y (and idx with 2:4 tiles) must be non-NULL");
  if (ldx % 8) return fail(NM_ERR_ALIGN, "ldx = %lld is not a multiple of 8", (long long)ldx);
  if (!aligned16(values) || (idx && !aligned16(idx)) || !aligned16(act) || !aligned16(Y) ||
      !aligned8(tile_meta) || !aligned8(row_meta))
    return fail(NM_ERR_ALIGN, "values, idx, act and Y must be 16-byte aligned, the layout tables 8-byte aligned");
  if (T * ldx > kMaxElems || T * ldy > kMaxElems) return fail(NM_ERR_SHAPE, "T*ld too large");
  const int64_t RB = (R + tile_rows - 1) / tile_rows, KB = K / tile_cols;
  const size_t ybytes = extent(T, R, ldy, elt_bytes(out_dtype)), abytes = extent(T, K, ldx, 2);
  const size_t vbytes = size_t(values_count) * 2, ib = size_t(idx_bytes);
  if (overlaps(Y, ybytes, values, vbytes) || overlaps(Y, ybytes, idx, ib) || overlaps(Y, ybytes, act, abytes) ||
      overlaps(Y, ybytes, tile_meta, size_t(RB * KB) * 16) || overlaps(Y, ybytes, row_meta, size_t(RB) * 32))
    return fail(NM_ERR_ALIAS, "Y overlaps an input");
  nm::HybridArgs a;
  a.values = static_cast<const uint16_t*>(values);
  a.idx = idx;
  a.tile_meta = tile_meta;
  a.row_meta = row_meta;
  a.R = R;
  a.K = K;
  a.tile_rows = tile_rows;
  a.tile_cols = tile_cols;
  a.dtype = dtype;
  a.values_bytes = vbytes;
  a.idx_bytes = ib;
  a.act = static_cast<const uint16_t*>(act);
  a.T = T;
  a.ldx = ldx;
  a.Y = Y;
  a.ldy = ldy;
  a.out_dtype = out_dtype;
  return hip_status(nm::launch_hybrid_spmm(a, static_cast<hipStream_t>(stream)), "nm_hybrid_spmm launch");
}

// ---------------------------------------------------------------------------
// Block-sparse and diagonal-sparse structures with the column permutation
// ---------------------------------------------------------------------------
static nm_status check_block_shape(int64_t R, int64_t K) {
  if (R < 0 || R > kMaxRT || R % 32)
    return fail(NM_ERR_SHAPE, "R = %lld must be a multiple of 32 in [0, 2^30]", (long long)R);
  if (K < 32 || K > kMaxK || K % 32)
    return fail(NM_ERR_SHAPE, "K = %lld must be a multiple of 32 in [32, 2^24]", (long long)K);
  return NM_OK;
}

static nm_status check_host_product(int dtype, int out_dtype, int64_t R, int64_t K, int64_t T, int64_t ldx,
                                    int64_t ldy) {
  if (dtype != NM_F16 && dtype != NM_BF16)
    return fail(NM_ERR_UNSUPPORTED, "block / diagonal products take NM_F16 or NM_BF16, not dtype %d", dtype);
  if (out_dtype != NM_F32 && out_dtype != dtype)
    return fail(NM_ERR_UNSUPPORTED, "out_dtype %d must be NM_F32 or the input dtype", out_dtype);
  if (T < 0 || T > kMaxRT) return fail(NM_ERR_SHAPE, "T = %lld out of range", (long long)T);
  if (ldx < K) return fail(NM_ERR_STRIDE, "ldx = %lld < K = %lld", (long long)ldx, (long long)K);
  if (ldy < R) return fail(NM_ERR_STRIDE, "ldy = %lld < R = %lld", (long long)ldy, (long long)R);
  if (ldx > kMaxElems || ldy > kMaxElems) return fail(NM_ERR_SHAPE, "leading dimension above 2^40 elements");
  if (T * ldx > kMaxElems || T * ldy > kMaxElems) return fail(NM_ERR_SHAPE, "T*ld too large");
  if (int64_t(extent(T, K, ldx, 2)) >= (int64_t(1) << 32))
    return fail(NM_ERR_SHAPE, "act of 4 GiB or more (its reads use 32-bit offsets)");
  return NM_OK;
}

nm_status nm_block_structure(int64_t R, int64_t K, const uint8_t* mask, int32_t* row_ptr, int32_t* col,
                             int64_t* nnzb) {
  nm_status st = check_block_shape(R, K);
  if (st != NM_OK) return st;
  const int64_t RB = R / 32, KB = K / 32;
  if (RB * KB > 0 && !mask) return fail(NM_ERR_NULL, "mask must be non-NULL");
  int64_t n = 0;
  for (int64_t b = 0; b < RB; ++b) {
    if (row_ptr) row_ptr[b] = int32_t(n);
    for (int64_t c = 0; c < KB; ++c) {
      const uint8_t f = mask[b * KB + c];
      if (f > 1) return fail(NM_ERR_SHAPE, "mask[%lld] = %d is neither 0 nor 1", (long long)(b * KB + c), f);
      if (f) {
        if (col) col[n] = int32_t(c);
        ++n;
      }
    }
  }
  if (n > (int64_t(1) << 21)) return fail(NM_ERR_SHAPE, "more than 2^21 kept blocks (values of 4 GiB)");
  if (row_ptr) row_ptr[RB] = int32_t(n);
  if (nnzb) *nnzb = n;
  return ok();
}

nm_status nm_block_compress(const void* W, int64_t R, int64_t K, int64_t ldw, int dtype, const int32_t* row_ptr,
                            const int32_t* col, int64_t nnzb, void* values, void* stream) {
  if (dtype != NM_F16 && dtype != NM_BF16)
    return fail(NM_ERR_UNSUPPORTED, "block structures take NM_F16 or NM_BF16 weights, not dtype %d", dtype);
  nm_status st = check_block_shape(R, K);
  if (st != NM_OK) return st;
  if (nnzb < 0 || nnzb > (R / 32) * (K / 32))
    return fail(NM_ERR_SHAPE, "nnzb = %lld outside [0, blocks of W]", (long long)nnzb);
  if (ldw < K) return fail(NM_ERR_STRIDE, "ldw = %lld < K = %lld", (long long)ldw, (long long)K);
  if (ldw > kMaxElems || R * ldw > kMaxElems) return fail(NM_ERR_SHAPE, "R*ldw too large");
  if (R == 0 || nnzb == 0) return ok();
  if (!W || !row_ptr || !col || !values) return fail(NM_ERR_NULL, "W, row_ptr, col and values must be non-NULL");
  if (ldw % 8) return fail(NM_ERR_ALIGN, "ldw = %lld is not a multiple of 8", (long long)ldw);
  if (!aligned16(W) || !aligned16(values) || !aligned16(row_ptr) || !aligned16(col))
    return fail(NM_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const size_t vbytes = size_t(nnzb) * 2048;
  if (overlaps(values, vbytes, W, extent(R, K, ldw, 2)) || overlaps(values, vbytes, row_ptr, size_t(R / 32 + 1) * 4) ||
      overlaps(values, vbytes, col, size_t(nnzb) * 4))
    return fail(NM_ERR_ALIAS, "values overlaps an input");
  return hip_status(nm::launch_block_pack(static_cast<const uint16_t*>(W), ldw, R, K, row_ptr, col, nnzb,
                                          static_cast<uint16_t*>(values), static_cast<hipStream_t>(stream)),
                    "nm_block_compress launch");
}

nm_status nm_block_spmm(const void* values, const int32_t* row_ptr, const int32_t* col, int64_t nnzb, int64_t R,
                        int64_t K, int dtype, const void* act, int64_t T, int64_t ldx, const int32_t* perm,
                        void* Y, int64_t ldy, int out_dtype, void* stream) {
  nm_status st = check_block_shape(R, K);
  if (st != NM_OK) return st;
  st = check_host_product(dtype, out_dtype, R, K, T, ldx, ldy);
  if (st != NM_OK) return st;
  if (nnzb < 0 || nnzb > (R / 32) * (K / 32))
    return fail(NM_ERR_SHAPE, "nnzb = %lld outside [0, blocks of W]", (long long)nnzb);
  if (R == 0 || T == 0) return ok();
  if (!row_ptr || !act || !Y || (nnzb > 0 && (!values || !col)))
    return fail(NM_ERR_NULL, "row_ptr, act, Y (and values, col with kept blocks) must be non-NULL");
  if (ldx % 8) return fail(NM_ERR_ALIGN, "ldx = %lld is not a multiple of 8", (long long)ldx);
  if ((values && !aligned16(values)) || !aligned16(row_ptr) || (col && !aligned16(col)) || !aligned16(act) ||
      !aligned16(Y) || (perm && !aligned16(perm)))
    return fail(NM_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const size_t ybytes = extent(T, R, ldy, elt_bytes(out_dtype)), abytes = extent(T, K, ldx, 2);
  const size_t vbytes = size_t(nnzb) * 2048;
  if (overlaps(Y, ybytes, values, vbytes) || overlaps(Y, ybytes, act, abytes) ||
      overlaps(Y, ybytes, row_ptr, size_t(R / 32 + 1) * 4) || overlaps(Y, ybytes, col, size_t(nnzb) * 4) ||
      overlaps(Y, ybytes, perm, perm ? size_t(K) * 4 : 0))
    return fail(NM_ERR_ALIAS, "Y overlaps an input");
  nm::HostArgs a;
  a.diagonal = false;
  a.values = static_cast<const uint16_t*>(values);
  a.values_bytes = vbytes;
  a.row_ptr = row_ptr;
  a.col = col;
  a.nnz = nnzb;
  a.R = R;
  a.K = K;
  a.dtype = dtype;
  a.act = static_cast<const uint16_t*>(act);
  a.act_bytes = abytes;
  a.ldx = ldx;
  a.T = T;
  a.perm = perm;
  a.out = Y;
  a.ldy = ldy;
  a.out_dtype = out_dtype;
  return hip_status(nm::launch_host_spmm(a, static_cast<hipStream_t>(stream)), "nm_block_spmm launch");
}

static nm_status check_diag_shape(int64_t R, int64_t K, int64_t D) {
  if (R < 0 || R > kMaxRT) return fail(NM_ERR_SHAPE, "R = %lld out of range", (long long)R);
  if (K < 8 || K > nm::kDiagMaxK || K % 8)
    return fail(NM_ERR_SHAPE, "K = %lld must be a multiple of 8 in [8, %lld]", (long long)K,
                (long long)nm::kDiagMaxK);
  if (D < 0 || D > K) return fail(NM_ERR_SHAPE, "D = %lld outside [0, K]", (long long)D);
  if (D * R * 2 >= (int64_t(1) << 32)) return fail(NM_ERR_SHAPE, "values of 4 GiB or more (32-bit offsets)");
  return NM_OK;
}

nm_status nm_diag_compress(const void* W, int64_t R, int64_t K, int64_t ldw, int dtype, const int32_t* offsets,
                           int64_t D, void* values, void* stream) {
  if (dtype != NM_F16 && dtype != NM_BF16)
    return fail(NM_ERR_UNSUPPORTED, "diagonal structures take NM_F16 or NM_BF16 weights, not dtype %d", dtype);
  nm_status st = check_diag_shape(R, K, D);
  if (st != NM_OK) return st;
  if (ldw < K) return fail(NM_ERR_STRIDE, "ldw = %lld < K = %lld", (long long)ldw, (long long)K);
  if (ldw > kMaxElems || R * ldw > kMaxElems) return fail(NM_ERR_SHAPE, "R*ldw too large");
  if (R == 0 || D == 0) return ok();
  if (!W || !offsets || !values) return fail(NM_ERR_NULL, "W, offsets and values must be non-NULL");
  if (!aligned16(W) || !aligned16(values) || !aligned16(offsets))
    return fail(NM_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const size_t vbytes = size_t(D) * size_t(R) * 2;
  if (overlaps(values, vbytes, W, extent(R, K, ldw, 2)) || overlaps(values, vbytes, offsets, size_t(D) * 4))
    return fail(NM_ERR_ALIAS, "values overlaps an input");
  return hip_status(nm::launch_diag_pack(static_cast<const uint16_t*>(W), ldw, R, K, offsets, D,
                                         static_cast<uint16_t*>(values), static_cast<hipStream_t>(stream)),
                    "nm_diag_compress launch");
}

nm_status nm_diag_spmm(const void* values, const int32_t* offsets, int64_t D, int64_t R, int64_t K, int dtype,
                       const void* act, int64_t T, int64_t ldx, const int32_t* perm, void* Y, int64_t ldy,
                       int out_dtype, void* stream) {
  nm_status st = check_diag_shape(R, K, D);
  if (st != NM_OK) return st;
  st = check_host_product(dtype, out_dtype, R, K, T, ldx, ldy);
  if (st != NM_OK) return st;
  if (R == 0 || T == 0) return ok();
  if (!act || !Y || (D > 0 && (!values || !offsets)))
    return fail(NM_ERR_NULL, "act, Y (and values, offsets with D > 0) must be non-NULL");
  if (ldx % 8) return fail(NM_ERR_ALIGN, "ldx = %lld is not a multiple of 8", (long long)ldx);
  if ((values && !aligned16(values)) || (offsets && !aligned16(offsets)) || !aligned16(act) || !aligned16(Y) ||
      (perm && !aligned16(perm)))
    return fail(NM_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const size_t ybytes = extent(T, R, ldy, elt_bytes(out_dtype)), abytes = extent(T, K, ldx, 2);
  if (overlaps(Y, ybytes, values, size_t(D) * size_t(R) * 2) || overlaps(Y, ybytes, act, abytes) ||
      overlaps(Y, ybytes, offsets, size_t(D) * 4) || overlaps(Y, ybytes, perm, perm ? size_t(K) * 4 : 0))
    return fail(NM_ERR_ALIAS, "Y overlaps an input");
  nm::HostArgs a;
  a.diagonal = true;
  a.values = static_cast<const uint16_t*>(values);
  a.values_bytes = size_t(D) * size_t(R) * 2;
  a.offsets = offsets;
  a.nnz = D;
  a.R = R;
  a.K = K;
  a.dtype = dtype;
  a.act = static_cast<const uint16_t*>(act);
  a.act_bytes = abytes;
  a.ldx = ldx;
  a.T = T;
  a.perm = perm;
  a.out = Y;
  a.ldy = ldy;
  a.out_dtype = out_dtype;
  return hip_status(nm::launch_host_spmm(a, static_cast<hipStream_t>(stream)), "nm_diag_spmm launch");
}

}  // extern "C"
