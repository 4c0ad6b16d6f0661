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

#include <type_traits>

namespace nm {
namespace {


// c + a.lo * b.lo + a.hi * b.hi on two packed 16-bit values (v_dot2_f32_*).
template <int DT>
__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  if constexpr (DT == NM_F16) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
  } else {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, a), __builtin_bit_cast(b2, b), c, false);
  }
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
// Block product, direct (K above 2048, where a token tile's staged row would
// not fit LDS).  A workgroup owns one block-row (32 rows) and 256 tokens;
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
// Block product, staged: one workgroup per 32 tokens and every block-row.
// The tile's activations are staged once in LDS as read through the map,
// xs[t][j] = act[T0 + t][perm[j]] (rows of 2K + 16 bytes: the 16-byte B
// operand reads of 16 consecutive tokens fall in distinct banks when K is a
// multiple of 128; the map itself is copied to LDS behind the tile first), so
// a kept block's B operands are plain 16-byte LDS reads
// whatever the map.  (Gathering per block instead drags every cache line of
// each token row in for every block, since a block's 32 mapped columns spread
// over the whole row.)  Wave w then walks block-rows w, w + 4, ...: for each
// kept block its two 16-row A fragments straight from global memory (the next
// block's loaded while the current one is multiplied), its two 16-token B
// fragments from LDS, four MFMAs; the block-row's 32 x 32 outputs go out
// before the next block-row.  K <= 2048 (LDS); larger K takes the direct
// kernel above.
// ---------------------------------------------------------------------------
constexpr int kStTok = 32;
constexpr int64_t kBlockStagedMaxK = 2048;
constexpr int kGatherLdsMaxK = 1024;   // the map applied by gathering within LDS up to this K

__host__ __device__ constexpr int staged_pitch(int K) { return 2 * K + 16; }

template <int DT, int OUT, bool MAP>
__global__ __launch_bounds__(256) void block_spmm_staged_kernel(
    const uint16_t* __restrict__ values, uint32_t values_bytes, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col, int nnzb, int RB, int K, const uint16_t* __restrict__ act, uint32_t act_bytes,
    int64_t ldx, int T, const int32_t* __restrict__ perm, void* __restrict__ Y, int64_t ldy) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int T0 = blockIdx.x * kStTok;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const int KB = K / 32, pitch = staged_pitch(K);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(values, values_bytes);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(act, act_bytes);

  // ---- stage: item = 8 columns of one token, consecutive lanes along the
  // row (one token row's reads stay within its cache lines); tokens past T
  // are zeros.  With the map, K <= 1024: the rows are staged as they are
  // (16-byte loads), then every thread gathers its items' mapped columns from
  // LDS into registers and writes them back after a barrier; larger K gathers
  // 2-byte pieces from global memory.  The map is copied to LDS (behind the
  // tile) first, and four items' loads are in flight at a time.
  const int per_row = K / 8, items = kStTok * per_row;
  const int32_t* pl = reinterpret_cast<const int32_t*>(smem + kStTok * pitch);
  auto stage = [&](auto gather_c) {
    constexpr bool GATHER = decltype(gather_c)::value;
    constexpr int kU = 4;
    for (int it0 = tid; it0 < items; it0 += 256 * kU) {
      u32x4 v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int it = min(it0 + 256 * u, items - 1);
        const int t = it / per_row, j8 = (it - t * per_row) * 8;
        const bool live = T0 + t < T;
        const uint32_t rowoff = uint32_t(min(T0 + t, T - 1)) * uint32_t(ldx) * 2u;
        if constexpr (GATHER) {
          uint32_t h[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            h[e] = live ? __builtin_amdgcn_raw_buffer_load_b16(
                              ra, rowoff + umin(uint32_t(pl[j8 + e]), uint32_t(K - 1)) * 2u, 0, 0)
                        : 0u;
          v[u] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        } else {
          v[u] = live ? __builtin_bit_cast(
                            u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, rowoff + uint32_t(j8) * 2u, 0, 0))
                      : u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int it = it0 + 256 * u;
        if (it < items) {
          const int t = it / per_row, j8 = (it - t * per_row) * 8;
          *reinterpret_cast<u32x4*>(smem + t * pitch + j8 * 2) = v[u];
        }
      }
    }
  };
  if constexpr (MAP) {
    for (int k = tid * 4; k < K; k += 1024)
      *reinterpret_cast<u32x4*>(smem + kStTok * pitch + k * 4) = *reinterpret_cast<const u32x4*>(perm + k);
    __syncthreads();
    if (K <= kGatherLdsMaxK) {
      stage(std::false_type{});
      __syncthreads();
      constexpr int kItems = kStTok * (kGatherLdsMaxK / 8) / 256;   // items per thread, at most
      u32x4 v[kItems];
#pragma unroll
      for (int u = 0; u < kItems; ++u) {
        const int it = tid + 256 * u;
        if (it < items) {
          const int t = it / per_row, j8 = (it - t * per_row) * 8;
          const unsigned char* row = smem + t * pitch;
          uint32_t h[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            h[e] = *reinterpret_cast<const uint16_t*>(row + umin(uint32_t(pl[j8 + e]), uint32_t(K - 1)) * 2u);
          v[u] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        }
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kItems; ++u) {
        const int it = tid + 256 * u;
        if (it < items) {
          const int t = it / per_row, j8 = (it - t * per_row) * 8;
          *reinterpret_cast<u32x4*>(smem + t * pitch + j8 * 2) = v[u];
        }
      }
    } else {
      stage(std::true_type{});
    }
  } else {
    stage(std::false_type{});
  }
  __syncthreads();

  const bool vec_ok = (ldy & 3) == 0;
  for (int br = wave; br < RB; br += 4) {
    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int begin = __builtin_amdgcn_readfirstlane(min(max(row_ptr[br], 0), nnzb));
    const int end = __builtin_amdgcn_readfirstlane(min(max(row_ptr[br + 1], begin), nnzb));
    auto load_a = [&](int blk, u32x4 (&a)[2]) {
#pragma unroll
      for (int fr = 0; fr < 2; ++fr)
        a[fr] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rv, uint32_t(((blk * 32 + fr * 16 + li) * 32 + 8 * lq) * 2), 0, 0));
    };
    u32x4 a[2], an[2];
    if (begin < end) load_a(begin, a);
    for (int blk = begin; blk < end; ++blk) {
      const int c = __builtin_amdgcn_readfirstlane(min(max(col[blk], 0), KB - 1));
      if (blk + 1 < end) load_a(blk + 1, an);
      u32x4 b[2];
#pragma unroll
      for (int ft = 0; ft < 2; ++ft)
        b[ft] = *reinterpret_cast<const u32x4*>(smem + (ft * 16 + li) * pitch + (32 * c + 8 * lq) * 2);
#pragma unroll
      for (int fr = 0; fr < 2; ++fr)
#pragma unroll
        for (int ft = 0; ft < 2; ++ft) acc[fr][ft] = mfma32<DT>(a[fr], b[ft], acc[fr][ft]);
      a[0] = an[0];
      a[1] = an[1];
    }
#pragma unroll
    for (int ft = 0; ft < 2; ++ft) {
      const int t = T0 + ft * 16 + li;
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
// is not a tile contraction: it runs on the vector ALUs.  A workgroup owns 32
// tokens and one part of the rows.  It first stages the 32 tokens'
// activations in LDS column by column, xs[k][t] = act[T0 + t][perm[k]] (the
// map is applied here, once per element and workgroup, so the loop below reads
// plain columns; 80 bytes per column, K <= 1792), then each thread takes one
// unit of G rows: per diagonal the column c = (r + o_d) mod K and its 32
// activations in four 16-byte LDS reads; two diagonals at a time feed v_dot2_f32 (fp32
// accumulation of the pair's exact products).  Rows r and r + K lie on the
// same columns of every diagonal (the diagonals wrap round K), so when R is at
// least G K a unit is the G rows r, r + K, ..., r + (G - 1) K: the LDS reads
// and the byte permutes that pair two diagonals' activations are shared by G
// rows' products (one permute and G v_dot2 per token and diagonal pair).
// ---------------------------------------------------------------------------
constexpr int kDiagTok = 32;
// a column of the staged tile: 64 bytes of tokens and 16 of padding, so the
// 16-byte reads of 16 threads on 16 consecutive columns fall in distinct
// banks (at 64 bytes every fourth column shares banks: 4-way conflicts)
constexpr int kDiagPitch = kDiagTok * 2 + 16;
// workgroup size: G == 1, 8 waves (two workgroups per CU, 4 waves per SIMD);
// G > 1, 4 waves holding G x 32 accumulators each (two workgroups per CU)
constexpr int diag_threads(int G) { return G == 1 ? 512 : 256; }
// largest workgroup LDS with the row buffer for the map: two workgroups per CU
constexpr int kDiagGatherLds = 80 * 1024;
// 16-byte pieces of one 8-token row group a thread loads for the row buffer
constexpr int kGatherPieces = 4;

template <int DT, int OUT, bool MAP, int G>
__global__ __launch_bounds__(diag_threads(G)) void diag_spmm_kernel(const uint16_t* __restrict__ values,
                                                        const int32_t* __restrict__ offsets, int D, int R, int K,
                                                        const uint16_t* __restrict__ act, uint32_t act_bytes,
                                                        int64_t ldx, int T, const int32_t* __restrict__ perm,
                                                        void* __restrict__ Y, int64_t ldy, int parts,
                                                        int lds_gather) {
  constexpr int kThreads = diag_threads(G);
  extern __shared__ __align__(16) unsigned char smem[];
  // workgroup -> (token tile, part): a part is kThreads units of rows, one per
  // thread; the parts of a token tile are consecutive, on one XCD
  const int b = xcd_tile(blockIdx.x, gridDim.x);
  const int tile = b / parts, part = b - tile * parts;
  const int T0 = tile * kDiagTok;
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(act, act_bytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(values, uint32_t(D) * uint32_t(R) * 2u);   // below 4 GiB

  // ---- stage (tokens past T are zeros)
  int32_t* offl = reinterpret_cast<int32_t*>(smem + K * kDiagPitch);
  if constexpr (MAP) {
    if (lds_gather) {
      // through the map, 8 tokens at a time: their rows are copied whole
      // (coalesced 16-byte loads) into a buffer behind the offsets, then each
      // thread gathers whole columns k from it, 8 tokens into one 16-byte
      // write of the tile (at the 80-byte pitch 16 consecutive columns cover
      // all 64 banks once).  The loads of all four row groups are issued
      // first (a thread holds at most kGatherPieces pieces of each: the
      // launcher takes this path only for K <= kGatherPieces * threads), so
      // their latency is paid once.
      uint16_t* raw = reinterpret_cast<uint16_t*>(smem + K * kDiagPitch + ((D * 4 + 15) & ~15));
      const int k8s = K / 8;
      u32x4 rv[kDiagTok / 8][kGatherPieces];
#pragma unroll
      for (int c = 0; c < kDiagTok / 8; ++c)
#pragma unroll
        for (int i = 0; i < kGatherPieces; ++i) {
          const int p = tid + i * kThreads;
          const int tt = p / k8s, k8 = (p - tt * k8s) * 8;
          const int t = T0 + 8 * c + tt;
          const uint32_t rowoff = uint32_t(min(t, T - 1)) * uint32_t(ldx) * 2u;
          rv[c][i] = p < 8 * k8s && t < T
                         ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, rowoff + uint32_t(k8) * 2u, 0, 0))
                         : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
      for (int c = 0; c < kDiagTok / 8; ++c) {
#pragma unroll
        for (int i = 0; i < kGatherPieces; ++i) {
          const int p = tid + i * kThreads;
          if (p < 8 * k8s) {
            const int tt = p / k8s, k8 = (p - tt * k8s) * 8;
            *reinterpret_cast<u32x4*>(raw + tt * K + k8) = rv[c][i];
          }
        }
        __syncthreads();
        for (int k = tid; k < K; k += kThreads) {
          const int pk = int(umin(uint32_t(perm[k]), uint32_t(K - 1)));
          uint32_t h[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) h[e] = raw[e * K + pk];
          *reinterpret_cast<u32x4*>(smem + k * kDiagPitch + 16 * c) =
              u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        }
        __syncthreads();   // the buffer is refilled next
      }
    } else {
      // through the map, gathered from global memory (K too large for the
      // buffer): a thread takes whole columns k, lanes on consecutive columns
      // (the 64 gathers of one load fall in a single token row, a few of its
      // lines), and every token, 8 at a time into one 16-byte write
      for (int k = tid; k < K; k += kThreads) {
        const uint32_t col = umin(uint32_t(perm[k]), uint32_t(K - 1)) * 2u;
#pragma unroll
        for (int i = 0; i < kDiagTok / 8; ++i) {
          uint32_t h[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int t = 8 * i + e;
            const uint32_t rowoff = uint32_t(min(T0 + t, T - 1)) * uint32_t(ldx) * 2u;
            h[e] = T0 + t < T ? uint32_t(__builtin_amdgcn_raw_buffer_load_b16(ra, rowoff + col, 0, 0)) : 0u;
          }
          *reinterpret_cast<u32x4*>(smem + k * kDiagPitch + 16 * i) =
              u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        }
      }
    }
  } else {
    // a thread fills 8 consecutive columns of one token (lane order: token
    // fastest, so the 32 lanes of a column group write its 64 contiguous bytes)
    const int groups = kDiagTok * (K / 8);
    for (int g = tid; g < groups; g += kThreads) {
      const int t = g % kDiagTok, k8 = (g / kDiagTok) * 8;
      const uint32_t rowoff = uint32_t(min(T0 + t, T - 1)) * uint32_t(ldx) * 2u;
      const u32x4 v = T0 + t < T ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       ra, rowoff + uint32_t(k8) * 2u, 0, 0))
                                 : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<uint16_t*>(smem + (k8 + e) * kDiagPitch + t * 2) = uint16_t(v[e >> 1] >> (16 * (e & 1)));
    }
  }
  __syncthreads();

  // the offsets, reduced into [0, K), go to LDS behind the tile
  for (int d = tid; d < D; d += kThreads) offl[d] = ((offsets[d] % K) + K) % K;
  __syncthreads();

  constexpr int kDC = G == 1 ? 16 : 8;   // diagonals whose weights are loaded together
  // unit u: rows q G K + j K + rk (j < G) with q = u div K, rk = u mod K; with
  // G == 1 that is row u.  Rows past R (the last q's) are computed from
  // clamped weight reads and not stored.
  const int units = G == 1 ? R : ((R + G * K - 1) / (G * K)) * K;
  if (const int u = part * kThreads + tid; u < units) {
    const int q = u / K, rk = u - q * K;
    int row[G];
#pragma unroll
    for (int j = 0; j < G; ++j) row[j] = q * G * K + j * K + rk;
    float acc[G][kDiagTok];
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int t = 0; t < kDiagTok; ++t) acc[j][t] = 0.f;
    auto column = [&](int d) {
      const int c = rk + offl[d];
      return reinterpret_cast<const u32x4*>(smem + (c - (c >= K ? K : 0)) * kDiagPitch);
    };
    // two diagonals at a time: per token one byte permute pairs the token's
    // activations on the two diagonals, and each of the G rows takes one
    // v_dot2 on its (w_d, w_d+1): fewer than one VALU operation per
    // multiply-add
    auto pair = [&](int d, const uint32_t (&wp)[G]) {
      const u32x4* x1 = column(d);
      const u32x4* x2 = column(d + 1);
#pragma unroll
      for (int c = 0; c < kDiagTok / 8; ++c) {
        const u32x4 a1 = x1[c], a2 = x2[c];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // v_perm_b32 byte selectors 0-3 take bytes of its second operand,
          // 4-7 of its first: (low halves of a1, a2), then (high halves)
          const uint32_t lo = __builtin_amdgcn_perm(a2[e], a1[e], 0x05040100u);   // token 2i of both
          const uint32_t hi = __builtin_amdgcn_perm(a2[e], a1[e], 0x07060302u);   // token 2i + 1
#pragma unroll
          for (int j = 0; j < G; ++j) {
            acc[j][8 * c + 2 * e] = dot2<DT>(wp[j], lo, acc[j][8 * c + 2 * e]);
            acc[j][8 * c + 2 * e + 1] = dot2<DT>(wp[j], hi, acc[j][8 * c + 2 * e + 1]);
          }
        }
      }
    };
    auto weight = [&](int d, int j) {
      const uint32_t r = uint32_t(min(row[j], R - 1));
      return uint32_t(__builtin_amdgcn_raw_buffer_load_b16(rw, uint32_t(d) * uint32_t(R) * 2u + r * 2u, 0, 0));
    };
    // whole batches of kDC diagonals, their weights loaded before the first is
    // used, then the remaining pairs, then an odd last diagonal: no branch
    // inside a batch, so every accumulator is updated in place
    int d = 0;
    for (; d + kDC <= D; d += kDC) {
      uint32_t wv[G][kDC];
#pragma unroll
      for (int i = 0; i < kDC; ++i)
#pragma unroll
        for (int j = 0; j < G; ++j) wv[j][i] = weight(d + i, j);
#pragma unroll
      for (int i = 0; i < kDC; i += 2) {
        uint32_t wp[G];
#pragma unroll
        for (int j = 0; j < G; ++j) wp[j] = wv[j][i] | (wv[j][i + 1] << 16);
        pair(d + i, wp);
      }
    }
    for (; d + 1 < D; d += 2) {
      uint32_t wp[G];
#pragma unroll
      for (int j = 0; j < G; ++j) wp[j] = weight(d, j) | (weight(d + 1, j) << 16);
      pair(d, wp);
    }
    if (d < D) {
      const u32x4* xs = column(d);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float w = half_to_f32<DT>(weight(d, j));
#pragma unroll
        for (int c = 0; c < kDiagTok / 8; ++c) {
          const u32x4 x = xs[c];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[j][8 * c + 2 * e] = __builtin_fmaf(w, half_to_f32<DT>(x[e] & 0xFFFFu), acc[j][8 * c + 2 * e]);
            acc[j][8 * c + 2 * e + 1] = __builtin_fmaf(w, half_to_f32<DT>(x[e] >> 16), acc[j][8 * c + 2 * e + 1]);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int r = row[j];
      if (r >= R) continue;
#pragma unroll
      for (int t = 0; t < kDiagTok; ++t) {
        if (T0 + t >= T) break;
        if constexpr (OUT == NM_F32) {
          static_cast<float*>(Y)[int64_t(T0 + t) * ldy + r] = acc[j][t];
        } else {
          static_cast<uint16_t*>(Y)[int64_t(T0 + t) * ldy + r] = to_half_bits<DT>(acc[j][t]);
        }
      }
    }
  }
}

template <int DT, int OUT, bool MAP>
hipError_t launch_block_cfg(const HostArgs& a, hipStream_t s) {
  const int64_t RB = a.R / 32;
  if (a.K <= kBlockStagedMaxK) {
    const int64_t tiles = (a.T + kStTok - 1) / kStTok;
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int lds = kStTok * staged_pitch(int(a.K)) + (MAP ? int(a.K) * 4 : 0);
    auto kern = block_spmm_staged_kernel<DT, OUT, MAP>;
    if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), lds); e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(unsigned(tiles)), dim3(256), lds, s, a.values, uint32_t(a.values_bytes), a.row_ptr,
                       a.col, int(a.nnz), int(RB), int(a.K), a.act, uint32_t(a.act_bytes), a.ldx, int(a.T), a.perm,
                       a.out, a.ldy);
    return hipGetLastError();
  }
  const int64_t tilesT = (a.T + kBlkTok - 1) / kBlkTok;
  if (RB * tilesT > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((block_spmm_kernel<DT, OUT, MAP>), dim3(unsigned(RB * tilesT)), dim3(256), 0, s, a.values,
                     uint32_t(a.values_bytes), a.row_ptr, a.col, int(a.nnz), int(RB), int(a.K), a.act,
                     uint32_t(a.act_bytes), a.ldx, int(a.T), a.perm, a.out, a.ldy);
  return hipGetLastError();
}

template <int DT, int OUT, bool MAP>
hipError_t launch_diag_cfg(const HostArgs& a, hipStream_t s) {
  const int64_t tiles = (a.T + kDiagTok - 1) / kDiagTok;
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  // the tile, the offsets, and for the map the buffer of 8 token rows when
  // two workgroups per CU still fit (else the map gathers from global memory)
  const int base = int(a.K) * kDiagPitch + ((int(a.nnz) * 4 + 15) & ~15);
  const int lds_gather = MAP && base + 16 * int(a.K) <= kDiagGatherLds ? 1 : 0;
  // every thread's share of a row group fits its kGatherPieces registers
  static_assert(kDiagGatherLds / (16 + kDiagPitch) <= kGatherPieces * diag_threads(4), "row group pieces");
  const int lds = base + (lds_gather ? 16 * int(a.K) : 0);
  // rows per unit: G rows share their columns only when R >= G K.  A token
  // tile's units are split into parts of one unit per thread, each its own
  // workgroup: several small workgroups per CU balance better than one or two
  // large ones, at the price of staging each tile once per part.
  auto launch = [&](auto kern, int G) {
    const int64_t units = G == 1 ? a.R : ((a.R + G * a.K - 1) / (G * a.K)) * a.K;
    const int64_t parts = (units + diag_threads(G) - 1) / diag_threads(G);
    if (tiles * parts > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), lds); e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(unsigned(tiles * parts)), dim3(diag_threads(G)), lds, s, a.values, a.offsets,
                       int(a.nnz), int(a.R), int(a.K), a.act, uint32_t(a.act_bytes), a.ldx, int(a.T), a.perm, a.out,
                       a.ldy, int(parts), lds_gather);
    return hipGetLastError();
  };
  if (a.R >= 4 * a.K) return launch(diag_spmm_kernel<DT, OUT, MAP, 4>, 4);
  if (a.R >= 2 * a.K) return launch(diag_spmm_kernel<DT, OUT, MAP, 2>, 2);
  return launch(diag_spmm_kernel<DT, OUT, MAP, 1>, 1);
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
