// Permuted sparse GEMM through a gather pass: X' = act[:, perm] is written to
// a workspace the caller provides, then the plain sparse GEMM runs on X'.
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
// Rows of up to 8192 columns go through a persistent variant: each workgroup
// walks row blocks with two LDS buffers, and the direct global->LDS loads of
// its next block land while it gathers and stores the current one, so the
// pass reads and writes HBM at the same time (a workgroup per block would put
// every workgroup in the same phase: all loading, then all storing).
#include "nm_device.h"
#include "nm_internal.h"

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
    const uint32_t q[8] = {umin(uint32_t(p0.x), kmax), umin(uint32_t(p0.y), kmax), umin(uint32_t(p0.z), kmax),
                           umin(uint32_t(p0.w), kmax), umin(uint32_t(p1.x), kmax), umin(uint32_t(p1.y), kmax),
                           umin(uint32_t(p1.z), kmax), umin(uint32_t(p1.w), kmax)};
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

constexpr int kDbMaxK = 8192;  // the persistent variant: a row fits a 16 KB buffer

// Blocks of rows_blk token rows (rows_blk * K * 2 <= kRowBytes); workgroup w
// takes blocks w, w + grid, ...  Each thread issues 4 direct loads per block
// (slots tid + 256 j of the block's kRowBytes / 16 slots; slots past the
// block's rows reread its last row into LDS nothing reads), so the wait
// counts are fixed: loads complete in order, and stores only make a counted
// wait stricter.
__global__ __launch_bounds__(kThreads) void permute_cols_db_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, const int32_t* __restrict__ perm, int T, int K,
    int rows_blk, int nblocks, uint16_t* __restrict__ Xp) {
  extern __shared__ __align__(16) unsigned char smem[];  // [2][kRowBytes]
  const int tid = threadIdx.x;
  const int cpr = K >> 3;  // 8-column (16-byte) chunks per row
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(X), (short)0, -1, 0x00020000);
  // this thread's 4 load slots: (row within the block, chunk)
  int lr[4], lc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int slot = tid + j * kThreads;
    lr[j] = min(slot / cpr, rows_blk - 1);
    lc[j] = slot - (slot / cpr) * cpr;
  }
  // first slot of this wave's part of each load (scalar: it feeds M0)
  const int wave_base = __builtin_amdgcn_readfirstlane(tid >> 6) * 64;
  auto issue = [&](int b, int buf) {
    const int t0 = b * rows_blk;
    const int nr = min(rows_blk, T - t0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = t0 + min(lr[j], nr - 1);
      const uint32_t off = uint32_t(t) * uint32_t(ldx) * 2u + uint32_t(lc[j]) * 16u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (lds_byte*)(smem + buf * kRowBytes + (wave_base + j * kThreads) * 16), 16, int(off), 0, 0, 0);
    }
  };

  // gather roles, as in permute_cols_kernel
  const uint32_t kmax = uint32_t(K - 1);
  const int rstep = cpr >= kThreads ? 1 : kThreads / cpr;
  const int lanes = cpr >= kThreads ? kThreads : rstep * cpr;
  const int r0 = cpr >= kThreads ? 0 : tid / cpr;
  const int c0 = cpr >= kThreads ? tid : tid - r0 * cpr;
  const bool gathers = tid < lanes;
  // one chunk per thread when a row has fewer chunks than threads: its perm
  // entries stay in registers across blocks
  uint32_t q[8];
  auto load_perm = [&](int c) {
    const int4 p0 = *reinterpret_cast<const int4*>(perm + c * 8);
    const int4 p1 = *reinterpret_cast<const int4*>(perm + c * 8 + 4);
    q[0] = umin(uint32_t(p0.x), kmax); q[1] = umin(uint32_t(p0.y), kmax);
    q[2] = umin(uint32_t(p0.z), kmax); q[3] = umin(uint32_t(p0.w), kmax);
    q[4] = umin(uint32_t(p1.x), kmax); q[5] = umin(uint32_t(p1.y), kmax);
    q[6] = umin(uint32_t(p1.z), kmax); q[7] = umin(uint32_t(p1.w), kmax);
  };
  if (gathers && cpr < kThreads) load_perm(c0);

  int it = 0;
  for (int b = blockIdx.x; b < nblocks; b += gridDim.x, ++it) {
    const int buf = it & 1;
    if (it == 0) issue(b, buf);
    barrier_no_fence();  // every thread is done gathering from the other buffer
    if (b + int(gridDim.x) < nblocks) {
      issue(b + gridDim.x, buf ^ 1);
      wait_vmcnt<4>();   // block b has landed (the next block's 4 loads may remain)
    } else {
      wait_vmcnt<0>();
    }
    barrier_no_fence();  // block b is visible to every thread
    if (!gathers) continue;
    const int t0 = b * rows_blk;
    const int nr = min(rows_blk, T - t0);
    const uint16_t* blk = reinterpret_cast<const uint16_t*>(smem + buf * kRowBytes);
    for (int c = c0; c < cpr; c += kThreads) {
      if (cpr >= kThreads) load_perm(c);
      for (int r = r0; r < nr; r += rstep) {
        const uint16_t* row = blk + r * K;
        uint4 o;
        o.x = uint32_t(row[q[0]]) | (uint32_t(row[q[1]]) << 16);
        o.y = uint32_t(row[q[2]]) | (uint32_t(row[q[3]]) << 16);
        o.z = uint32_t(row[q[4]]) | (uint32_t(row[q[5]]) << 16);
        o.w = uint32_t(row[q[6]]) | (uint32_t(row[q[7]]) << 16);
        *reinterpret_cast<uint4*>(Xp + int64_t(t0 + r) * K + c * 8) = o;
      }
    }
  }
}

}  // namespace

// The allocation-free entry point's workspace: one array per GPU, held until
// the process ends.  Host code never uses the array's name as an address (on
// the host it is only a stand-in): the device address comes from
// hipGetSymbolAddress, once per device with that device current.
static __device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

hipError_t static_workspace(void** ptr) {
  static std::mutex mu;
  static std::map<int, void*> addr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> g(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    it = addr.emplace(dev, p).first;
  }
  *ptr = it->second;
  return hipSuccess;
}

// The gather pass takes 16-bit activations with K % 8 == 0 (16-byte chunks)
// and K <= 65536; few tokens (T <= 16) gather inside the few-token kernel.
size_t spmm_perm_gather_bytes(int64_t T, int64_t K, int dtype) {
  const bool applies = (K % 8) == 0 && K <= kMaxK && T > 16 && (dtype == NM_F16 || dtype == NM_BF16);
  return applies ? size_t(T) * size_t(K) * 2 : 0;
}

hipError_t launch_spmm_perm_gather(const SpmmArgs& a, void* xp, hipStream_t s) {
  hipError_t e = hipSuccess;
  const int K = int(a.K);
  int rows_blk = kRowBytes / (K * 2);
  if (rows_blk < 1) rows_blk = 1;
  if (rows_blk > 64) rows_blk = 64;
  const int64_t blocks = (a.T + rows_blk - 1) / rows_blk;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (K <= kDbMaxK && int64_t(a.T) * a.ldx * 2 <= int64_t(0xFFFFFFFFu)) {
    const int cus = device_cu_count();
    // four workgroups per CU (32 KB of LDS each; measured: 8.9 us for the
    // 3072 x 768 x 12608 layer's 38.7 MB, against 9.2 with two and 10.0 for
    // one workgroup per block)
    const int64_t grid = blocks < int64_t(4) * cus ? blocks : int64_t(4) * cus;
    hipLaunchKernelGGL(permute_cols_db_kernel, dim3(unsigned(grid)), dim3(kThreads), 2 * kRowBytes, s, a.act,
                       a.ldx, a.perm, int(a.T), K, rows_blk, int(blocks), static_cast<uint16_t*>(xp));
  } else {
    const size_t lds = size_t(rows_blk) * size_t(K) * 2;
    if ((e = ensure_lds_limit(reinterpret_cast<const void*>(permute_cols_kernel), int(kMaxK * 2))) != hipSuccess)
      return e;
    hipLaunchKernelGGL(permute_cols_kernel, dim3(unsigned(blocks)), dim3(kThreads), lds, s, a.act, a.ldx,
                       a.perm, int(a.T), K, rows_blk, static_cast<uint16_t*>(xp));
  }
  e = hipGetLastError();
  if (e == hipSuccess) {
    SpmmArgs b = a;
    b.act = static_cast<const uint16_t*>(xp);
    b.ldx = a.K;
    b.perm = nullptr;
    b.workspace = nullptr;
    b.workspace_bytes = 0;
    e = launch_spmm(b, s);
  }
  return e;
}

}  // namespace nm
