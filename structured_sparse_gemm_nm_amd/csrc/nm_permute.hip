// Permuted sparse GEMM through a gather pass: X' = act[:, perm] is written to
// scratch memory owned by the calling stream, then the plain sparse GEMM
// runs on X'.
//
// ShuffleSparse (permutation-aware N:M pruning, inference section) applies the
// learned column permutation to the layer input, so the product is
// Y[t, r] = sum_k W_nm[r, k] * act[t, perm[k]].  Applied inside the GEMM the
// gather is along K, the contiguous axis of each token row, so it cannot use
// 16-byte loads and costs one LDS read per element per row fragment; done
// once per call it is a bandwidth-bound pass (read X, write X') after which
// the GEMM keeps its full-width, conflict-free loads.
//
// The pass: a workgroup stages a block of token rows in LDS with 16-byte
// loads, then each thread builds 8 consecutive output columns (chunk c) from
// 8 LDS reads at perm[c..c+7] and writes them as one 16-byte store.  A thread
// keeps one chunk for every row it handles, so its 8 perm entries are read
// from memory once.  Out-of-range perm entries (a broken precondition) are
// clamped into the row, so they give wrong values, never wrong addresses.
#include "nm_internal.h"

#include <functional>
#include <map>
#include <mutex>

namespace nm {
namespace {

constexpr int kThreads = 256;
constexpr int kRowBytes = 16 * 1024;   // LDS for staged rows per workgroup (several per CU)
constexpr int64_t kMaxK = 65536;       // one row must fit the LDS a workgroup can have

__global__ __launch_bounds__(kThreads) void permute_cols_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, const int32_t* __restrict__ perm, int T, int K,
    int rows_blk, uint16_t* __restrict__ Xp) {
  extern __shared__ __align__(16) uint16_t rowbuf[];
  const int t0 = blockIdx.x * rows_blk;
  const int nr = min(rows_blk, T - t0);
  const int cpr = K >> 3;                 // 8-column chunks per row
  const int total = nr * cpr;
  for (int i = threadIdx.x; i < total; i += kThreads) {
    const int r = i / cpr, c = i - r * cpr;
    *reinterpret_cast<uint4*>(rowbuf + r * K + c * 8) =
        *reinterpret_cast<const uint4*>(X + int64_t(t0 + r) * ldx + c * 8);
  }
  __syncthreads();
  // thread -> (chunk c, first row): chunks c, c + kThreads, ... of the rows
  // r0, r0 + rstep, ... (rstep = kThreads / cpr rows at a time when a row has
  // fewer chunks than threads)
  const uint32_t kmax = uint32_t(K - 1);
  const int rstep = cpr >= kThreads ? 1 : kThreads / cpr;
  const int lanes = cpr >= kThreads ? kThreads : rstep * cpr;
  if (threadIdx.x >= lanes) return;
  const int r0 = cpr >= kThreads ? 0 : threadIdx.x / cpr;
  for (int c = cpr >= kThreads ? threadIdx.x : threadIdx.x - r0 * cpr; c < cpr; c += kThreads) {
    const int4 p0 = *reinterpret_cast<const int4*>(perm + c * 8);
    const int4 p1 = *reinterpret_cast<const int4*>(perm + c * 8 + 4);
    const uint32_t q[8] = {min(uint32_t(p0.x), kmax), min(uint32_t(p0.y), kmax), min(uint32_t(p0.z), kmax),
                           min(uint32_t(p0.w), kmax), min(uint32_t(p1.x), kmax), min(uint32_t(p1.y), kmax),
                           min(uint32_t(p1.z), kmax), min(uint32_t(p1.w), kmax)};
    for (int r = r0; r < nr; r += rstep) {
      const uint16_t* row = rowbuf + r * K;
      uint4 o;
      o.x = uint32_t(row[q[0]]) | (uint32_t(row[q[1]]) << 16);
      o.y = uint32_t(row[q[2]]) | (uint32_t(row[q[3]]) << 16);
      o.z = uint32_t(row[q[4]]) | (uint32_t(row[q[5]]) << 16);
      o.w = uint32_t(row[q[6]]) | (uint32_t(row[q[7]]) << 16);
      *reinterpret_cast<uint4*>(Xp + int64_t(t0 + r) * K + c * 8) = o;
    }
  }
}

// Scratch for X': one buffer per (device, stream), grown to the largest size
// seen and kept until the process ends.  Work on one stream runs in order, so
// a buffer is never used by two calls at once; calls on different streams
// use different buffers.
struct ScratchKey {
  int dev;
  hipStream_t stream;
  bool operator<(const ScratchKey& o) const {
    return dev != o.dev ? dev < o.dev : std::less<hipStream_t>()(stream, o.stream);
  }
};
struct Scratch {
  void* ptr = nullptr;
  size_t bytes = 0;
};

hipError_t stream_scratch(int dev, hipStream_t s, size_t bytes, void** out) {
  static std::mutex mu;
  static std::map<ScratchKey, Scratch> cache;
  std::lock_guard<std::mutex> g(mu);
  Scratch& sc = cache[ScratchKey{dev, s}];
  if (sc.bytes < bytes) {
    // a smaller buffer may still be read by queued work on this stream
    if (sc.ptr) {
      hipError_t e = hipStreamSynchronize(s);
      if (e == hipSuccess) e = hipFree(sc.ptr);
      sc.ptr = nullptr;
      sc.bytes = 0;
      if (e != hipSuccess) return e;
    }
    hipError_t e = hipMalloc(&sc.ptr, bytes);
    if (e != hipSuccess) {
      sc.ptr = nullptr;
      return e;
    }
    sc.bytes = bytes;
  }
  *out = sc.ptr;
  return hipSuccess;
}

}  // namespace

bool spmm_perm_gather_applies(const SpmmArgs& a) {
  return a.perm != nullptr && (a.K % 8) == 0 && a.K <= kMaxK && a.T > 0;
}

hipError_t launch_spmm_perm_gather(const SpmmArgs& a, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  void* xp = nullptr;
  if ((e = stream_scratch(dev, s, size_t(a.T) * size_t(a.K) * 2, &xp)) != hipSuccess) return e;

  const int K = int(a.K);
  int rows_blk = kRowBytes / (K * 2);
  if (rows_blk < 1) rows_blk = 1;
  if (rows_blk > 64) rows_blk = 64;
  const int64_t blocks = (a.T + rows_blk - 1) / rows_blk;
  const size_t lds = size_t(rows_blk) * size_t(K) * 2;
  static bool attr_set = false;
  if (!attr_set) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(permute_cols_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(kMaxK * 2));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(permute_cols_kernel, dim3(unsigned(blocks)), dim3(kThreads), lds, s, a.act, a.ldx,
                     a.perm, int(a.T), K, rows_blk, static_cast<uint16_t*>(xp));
  e = hipGetLastError();
  if (e == hipSuccess) {
    SpmmArgs b = a;
    b.act = static_cast<const uint16_t*>(xp);
    b.ldx = a.K;
    b.perm = nullptr;
    e = launch_spmm(b, s);
  }
  return e;
}

}  // namespace nm
