// C ABI of the N:M sparse library: argument validation and dispatch.
//
// Every check runs on the host before the first HIP call, so argument errors
// never touch the device and can be tested without a GPU.
#include <atomic>
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
std::atomic<int> g_variant{0};

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

nm_status spmm_common(const void* values, const uint32_t* idx, int64_t R, int64_t K, int n, int m,
                      int dtype, const void* act, int64_t T, int64_t ldx, const int32_t* perm,
                      bool want_perm, void* Y, int64_t ldy, int out_dtype, void* stream) {
  nm_status st = check_format(R, K, n, m, dtype);
  if (st != NM_OK) return st;
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
  if (overlaps(Y, ybytes, values, z.values_bytes) || overlaps(Y, ybytes, idx, z.idx_bytes) ||
      overlaps(Y, ybytes, act, extent(T, K, ldx, elt_bytes(dtype))) ||
      (want_perm && overlaps(Y, ybytes, perm, size_t(K) * 4)))
    return fail(NM_ERR_ALIAS, "Y overlaps an input");

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
  a.variant = g_variant.load(std::memory_order_relaxed);
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

int nm_version(void) { return 102; }

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
                     out_dtype, stream);
}

nm_status nm_spmm_perm(const void* values, const uint32_t* idx, int64_t R, int64_t K, int n, int m,
                       int dtype, const void* act, int64_t T, int64_t ldx, const int32_t* perm,
                       void* Y, int64_t ldy, int out_dtype, void* stream) {
  return spmm_common(values, idx, R, K, n, m, dtype, act, T, ldx, perm, true, Y, ldy, out_dtype,
                     stream);
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

nm_status nm_set_variant(int variant) {
  if (variant < 0 || variant > nm::NM_VARIANT_MAX)
    return fail(NM_ERR_UNSUPPORTED, "variant %d", variant);
  g_variant.store(variant, std::memory_order_relaxed);
  return ok();
}

}  // extern "C"
