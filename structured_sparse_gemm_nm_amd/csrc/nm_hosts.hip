// The column permutation on two other host structures, block-sparse and
// diagonal-sparse weights, on gfx950.
//
// Sources: searcharxiv.com author page, the SHUFFLESPARSE abstract (one
// permutation primitive for block, N:M and diagonal structures) and the
// DynaDiag abstract (a diagonal pattern); gist.science "Technische
// Samenvatting: SHUFFLESPARSE", section "2. Methodologie" (y = (W Pi) x) and
// the item "Efficiëntie bij Inferentie" (the hardened Pi is an index map
// through which the structured kernel reads its input).  Both products take
// the map on their activation reads, Y^T[t, r] = sum_k W[r, k] act[t, perm[k]]
// (perm NULL reads act as it is; an entry outside [0, K) reads column K - 1).
// Storage (the pages name the structures only):
//   block     32 x 32 blocks in block-sparse rows: row_ptr[R/32 + 1],
//             col[nnzb] (block-columns), values[nnzb][32][32] row-major;
//   diagonal  wrap-around diagonals: offsets[D], values[D][R], weight
//             values[d][r] at column (r + offsets[d]) mod K.
#include "nm_device.h"
#include "nm_internal.h"

namespace nm {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// D = C + A x B on v_mfma_f32_16x16x32: lane (i, q) holds A[i][8q..8q+7] and
// B[8q..8q+7][i]; D rows 4q..4q+3 of column i.
template <int DT>
__device__ inline f32x4 mfma32(const u32x4& a, const u32x4& b, const f32x4& c) {
  if constexpr (DT == NM_F16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b),
                                                  c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8_t, a), __builtin_bit_cast(bf8_t, b), c,
                                                   0, 0, 0);
  }
}

template <int DT>
__device__ inline float half_to_f32(uint32_t h) {
  if constexpr (DT == NM_F16) {
    return float(__builtin_bit_cast(_Float16, uint16_t(h)));
  } else {
    return __builtin_bit_cast(float, h << 16);
  }
}

// XCD-aware order of a 1-D grid: the hardware deals workgroups to the 8 XCDs
// round robin, so workgroup p runs on XCD p % 8; when the grid is a multiple
// of 8 each XCD is given a contiguous run of logical tiles instead.
__device__ inline int xcd_tile(int p, int grid) {
  return (grid & 7) == 0 ? (p & 7) * (grid >> 3) + (p >> 3) : p;
}

// ---------------------------------------------------------------------------
// Block pack: the kept blocks of W copied to values[nnzb][32][32].  One
// workgroup per block-row; each thread copies one 16-byte piece of a block
// (a block is 128 pieces, two blocks per pass).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void block_pack_kernel(const uint16_t* __restrict__ W, int64_t ldw, int KB,
                                                         const int32_t* __restrict__ row_ptr,
                                                         const int32_t* __restrict__ col, int nnzb,
                                                         uint16_t* __restrict__ values) {
  const int b = blockIdx.x;
  const int begin = min(max(row_ptr[b], 0), nnzb);
  const int end = min(max(row_ptr[b + 1], begin), nnzb);
  const int piece = threadIdx.x & 127;
  const int row = piece >> 2, part = piece & 3;
  for (int blk = begin + (threadIdx.x >> 7); blk < end; blk += 2) {
    const int c = min(max(col[blk], 0), KB - 1);
    const u32x4 v = *reinterpret_cast<const u32x4*>(W + (int64_t(32) * b + row) * ldw + 32 * c + 8 * part);
    *reinterpret_cast<u32x4*>(values + (int64_t(blk) * 32 + row) * 32 + 8 * part) = v;
  }
}

// ---------------------------------------------------------------------------
// Block product.  A workgroup owns one block-row (32 rows) and 256 tokens;
// wave w the tokens 64w .. 64w+63 (2 x 4 fragments of 16 x 16).  For each
// kept block of the row (block-column c) the wave multiplies the block (K
// step of 32) with its tokens' 32 activations of the block's columns, on
// v_mfma_f32_16x16x32: an A lane (row i, quarter q) loads the 16 bytes of
// row i, columns 8q .. 8q+7 of the block; a B lane (token i, quarter q) the
// activations of columns 32c + 8q .. 8q+7 of its token, one 16-byte load, or
// with the map eight 2-byte loads at perm[32c + 8q + e].  No LDS: every
// operand byte is used by one lane only, so staging would not save reads.
// ---------------------------------------------------------------------------
constexpr int kBlkTok = 256;

template <int DT, int OUT, bool MAP>
__global__ __launch_bounds__(256) void block_spmm_kernel(const uint16_t* __restrict__ values, uint32_t values_bytes,
                                                         const int32_t* __restrict__ row_ptr,
                                                         const int32_t* __restrict__ col, int nnzb, int RB, int K,
                                                         const uint16_t* __restrict__ act, uint32_t act_bytes,
                                                         int64_t ldx, int T, const int32_t* __restrict__ perm,
                                                         void* __restrict__ Y, int64_t ldy) {
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int br = tile % RB, T0 = (tile / RB) * kBlkTok;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const int KB = K / 32;
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(values, values_bytes);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(act, act_bytes);

  // the token rows this lane reads (rows past T reread row T - 1; their
  // outputs are dropped)
  uint32_t trow[4];
#pragma unroll
  for (int ft = 0; ft < 4; ++ft) {
    const int t = min(T0 + wave * 64 + ft * 16 + li, T - 1);
    trow[ft] = uint32_t(t) * uint32_t(ldx) * 2u;
  }

  f32x4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int begin = __builtin_amdgcn_readfirstlane(min(max(row_ptr[br], 0), nnzb));
  const int end = __builtin_amdgcn_readfirstlane(min(max(row_ptr[br + 1], begin), nnzb));
  for (int blk = begin; blk < end; ++blk) {
    const int c = __builtin_amdgcn_readfirstlane(min(max(col[blk], 0), KB - 1));
    u32x4 a[2], b[4];
#pragma unroll
    for (int fr = 0; fr < 2; ++fr)
      a[fr] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rv, uint32_t(((blk * 32 + fr * 16 + li) * 32 + 8 * lq) * 2), 0, 0));
    const int k0 = 32 * c + 8 * lq;
    if constexpr (MAP) {
      // the 8 source columns of this lane's quarter, clamped into [0, K)
      const u32x4 p0 = *reinterpret_cast<const u32x4*>(perm + k0);
      const u32x4 p1 = *reinterpret_cast<const u32x4*>(perm + k0 + 4);
      uint32_t src[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        src[e] = umin(p0[e], uint32_t(K - 1)) * 2u;
        src[4 + e] = umin(p1[e], uint32_t(K - 1)) * 2u;
      }
#pragma unroll
      for (int ft = 0; ft < 4; ++ft) {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = __builtin_amdgcn_raw_buffer_load_b16(ra, trow[ft] + src[e], 0, 0);
        b[ft] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
      }
    } else {
#pragma unroll
      for (int ft = 0; ft < 4; ++ft)
        b[ft] = __builtin_bit_cast(u32x4,
                                   __builtin_amdgcn_raw_buffer_load_b128(ra, trow[ft] + uint32_t(k0) * 2u, 0, 0));
    }
#pragma unroll
    for (int fr = 0; fr < 2; ++fr)
#pragma unroll
      for (int ft = 0; ft < 4; ++ft) acc[fr][ft] = mfma32<DT>(a[fr], b[ft], acc[fr][ft]);
  }

  // epilogue: lane (token li, quarter q) holds rows 4q .. 4q+3 of each
  // fragment: 4 consecutive entries of Y^T's row t
  const bool vec_ok = (ldy & 3) == 0;
#pragma unroll
  for (int ft = 0; ft < 4; ++ft) {
    const int t = T0 + wave * 64 + ft * 16 + li;
    if (t >= T) continue;
#pragma unroll
    for (int fr = 0; fr < 2; ++fr) {
      const int r = br * 32 + fr * 16 + lq * 4;
      const f32x4 v = acc[fr][ft];
      if constexpr (OUT == NM_F32) {
        float* y = static_cast<float*>(Y) + int64_t(t) * ldy + r;
        if (vec_ok) {
          *reinterpret_cast<f32x4*>(y) = v;
        } else {
          for (int e = 0; e < 4; ++e) y[e] = v[e];
        }
      } else {
        uint16_t* y = static_cast<uint16_t*>(Y) + int64_t(t) * ldy + r;
        const uint32_t p0 = pack_half2<DT>(v[0], v[1]), p1 = pack_half2<DT>(v[2], v[3]);
        if (vec_ok) {
          *reinterpret_cast<u32x2*>(y) = u32x2{p0, p1};
        } else {
          const uint16_t hh[4] = {uint16_t(p0), uint16_t(p0 >> 16), uint16_t(p1), uint16_t(p1 >> 16)};
          for (int e = 0; e < 4; ++e) y[e] = hh[e];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Diagonal pack: values[d][r] = W[r][(r + o_d) mod K], one thread per entry.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void diag_pack_kernel(const uint16_t* __restrict__ W, int64_t ldw, int R, int K,
                                                        const int32_t* __restrict__ offsets, int D,
                                                        uint16_t* __restrict__ values) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= int64_t(D) * R) return;
  const int d = int(i / R), r = int(i - int64_t(d) * R);
  const int o = ((offsets[d] % K) + K) % K;
  const int c = (r % K + o) % K;
  values[i] = W[int64_t(r) * ldw + c];
}

// ---------------------------------------------------------------------------
// Diagonal product.  Each output row needs, for every diagonal, one
// activation column per token (a different one for every row), so the product
// is not a tile contraction: it runs on the vector ALUs.  A workgroup owns
// 256 rows (a thread each) and 32 tokens.  It first stages the 32 tokens'
// activations in LDS column by column, xs[k][t] = act[T0 + t][perm[k]] (the
// map is applied here, once per element, so the loop below reads plain
// columns; 64 bytes per column, K <= 2048), then thread r walks the
// diagonals: column c = (r + o_d) mod K, its 32 activations in four 16-byte
// LDS reads, 32 fp32 FMAs with values[d][r].
// ---------------------------------------------------------------------------
constexpr int kDiagTok = 32;

template <int DT, int OUT, bool MAP>
__global__ __launch_bounds__(256) void diag_spmm_kernel(const uint16_t* __restrict__ values,
                                                        const int32_t* __restrict__ offsets, int D, int R, int K,
                                                        const uint16_t* __restrict__ act, uint32_t act_bytes,
                                                        int64_t ldx, int T, const int32_t* __restrict__ perm,
                                                        void* __restrict__ Y, int64_t ldy, int tilesR) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int R0 = (tile % tilesR) * 256, T0 = (tile / tilesR) * kDiagTok;
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(act, act_bytes);

  // ---- stage: a thread fills 8 consecutive columns of one token (lane
  // order: token fastest, so the 32 lanes of a column group write its 64
  // contiguous bytes); tokens past T are zeros
  const int groups = kDiagTok * (K / 8);
  for (int g = tid; g < groups; g += 256) {
    const int t = g % kDiagTok, k8 = (g / kDiagTok) * 8;
    const bool live = T0 + t < T;
    const uint32_t rowoff = uint32_t(min(T0 + t, T - 1)) * uint32_t(ldx) * 2u;
    uint32_t h[8];
    if constexpr (MAP) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        h[e] = live ? __builtin_amdgcn_raw_buffer_load_b16(ra, rowoff + umin(uint32_t(perm[k8 + e]), uint32_t(K - 1)) * 2u, 0, 0)
                    : 0u;
    } else {
      const u32x4 v = live ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                           ra, rowoff + uint32_t(k8) * 2u, 0, 0))
                           : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[2 * e] = v[e] & 0xFFFFu;
        h[2 * e + 1] = v[e] >> 16;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *reinterpret_cast<uint16_t*>(smem + (k8 + e) * (kDiagTok * 2) + t * 2) = uint16_t(h[e]);
  }
  __syncthreads();

  const int r = R0 + tid;
  if (r >= R) return;
  const int rk = r % K;
  float acc[kDiagTok];
#pragma unroll
  for (int j = 0; j < kDiagTok; ++j) acc[j] = 0.f;
  for (int d = 0; d < D; ++d) {
    const int o = __builtin_amdgcn_readfirstlane(((offsets[d] % K) + K) % K);
    int c = rk + o;
    c -= c >= K ? K : 0;
    const float w = half_to_f32<DT>(values[int64_t(d) * R + r]);
    const u32x4* xs = reinterpret_cast<const u32x4*>(smem + c * (kDiagTok * 2));
#pragma unroll
    for (int q = 0; q < kDiagTok / 8; ++q) {
      const u32x4 x = xs[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[8 * q + 2 * e] = __builtin_fmaf(w, half_to_f32<DT>(x[e] & 0xFFFFu), acc[8 * q + 2 * e]);
        acc[8 * q + 2 * e + 1] = __builtin_fmaf(w, half_to_f32<DT>(x[e] >> 16), acc[8 * q + 2 * e + 1]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kDiagTok; ++j) {
    const int t = T0 + j;
    if (t >= T) break;
    if constexpr (OUT == NM_F32) {
      static_cast<float*>(Y)[int64_t(t) * ldy + r] = acc[j];
    } else {
      static_cast<uint16_t*>(Y)[int64_t(t) * ldy + r] = to_half_bits<DT>(acc[j]);
    }
  }
}

template <int DT, int OUT, bool MAP>
hipError_t launch_block_cfg(const HostArgs& a, hipStream_t s) {
  const int64_t RB = a.R / 32, tilesT = (a.T + kBlkTok - 1) / kBlkTok;
  if (RB * tilesT > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((block_spmm_kernel<DT, OUT, MAP>), dim3(unsigned(RB * tilesT)), dim3(256), 0, s, a.values,
                     uint32_t(a.values_bytes), a.row_ptr, a.col, int(a.nnz), int(RB), int(a.K), a.act,
                     uint32_t(a.act_bytes), a.ldx, int(a.T), a.perm, a.out, a.ldy);
  return hipGetLastError();
}

template <int DT, int OUT, bool MAP>
hipError_t launch_diag_cfg(const HostArgs& a, hipStream_t s) {
  const int64_t tilesR = (a.R + 255) / 256, tilesT = (a.T + kDiagTok - 1) / kDiagTok;
  if (tilesR * tilesT > 0x7FFFFFFF) return hipErrorInvalidValue;
  const size_t lds = size_t(a.K) * kDiagTok * 2;
  auto kern = diag_spmm_kernel<DT, OUT, MAP>;
  if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), lds); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(unsigned(tilesR * tilesT)), dim3(256), lds, s, a.values, a.offsets, int(a.nnz),
                     int(a.R), int(a.K), a.act, uint32_t(a.act_bytes), a.ldx, int(a.T), a.perm, a.out, a.ldy,
                     int(tilesR));
  return hipGetLastError();
}

template <int DT, int OUT>
hipError_t launch_host_map(const HostArgs& a, hipStream_t s) {
  if (a.diagonal)
    return a.perm ? launch_diag_cfg<DT, OUT, true>(a, s) : launch_diag_cfg<DT, OUT, false>(a, s);
  return a.perm ? launch_block_cfg<DT, OUT, true>(a, s) : launch_block_cfg<DT, OUT, false>(a, s);
}

template <int DT>
hipError_t launch_host_out(const HostArgs& a, hipStream_t s) {
  return a.out_dtype == NM_F32 ? launch_host_map<DT, NM_F32>(a, s) : launch_host_map<DT, DT>(a, s);
}

}  // namespace

hipError_t launch_block_pack(const uint16_t* W, int64_t ldw, int64_t R, int64_t K, const int32_t* row_ptr,
                             const int32_t* col, int64_t nnzb, uint16_t* values, hipStream_t s) {
  if (R == 0) return hipSuccess;
  hipLaunchKernelGGL(block_pack_kernel, dim3(unsigned(R / 32)), dim3(256), 0, s, W, ldw, int(K / 32), row_ptr, col,
                     int(nnzb), values);
  return hipGetLastError();
}

hipError_t launch_diag_pack(const uint16_t* W, int64_t ldw, int64_t R, int64_t K, const int32_t* offsets, int64_t D,
                            uint16_t* values, hipStream_t s) {
  const int64_t n = D * R;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(diag_pack_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, W, ldw, int(R), int(K),
                     offsets, int(D), values);
  return hipGetLastError();
}

hipError_t launch_host_spmm(const HostArgs& a, hipStream_t s) {
  if (a.T == 0 || a.R == 0) return hipSuccess;
  return a.dtype == NM_F16 ? launch_host_out<NM_F16>(a, s) : launch_host_out<NM_BF16>(a, s);
}

}  // namespace nm
