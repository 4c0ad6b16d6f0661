// Permuted 2:4 sparse GEMM, y = (W Pi) x, for prefill shapes with a short
// reduction axis (K <= 768, K % 128 == 0; e.g. a ViT-B/16 MLP fc1).
//
// SHUFFLESPARSE technical summary, section 2, the inference-efficiency item:
// the hardened permutation is a precomputed index map, and the sparse GEMM
// reads its input at the permuted addresses instead of running a separate
// permutation.  Here:  Y^T[t, r] = sum_k W_nm[r, k] * act[t, perm[k]].
//
// A permutation mixes the N:M groups of K, so the dense operand has to be
// gathered element by element.  Gathering 2-byte elements from global memory
// costs one request each; this kernel gathers from LDS instead:
//   * a workgroup owns a 256 x 64 tile of Y^T and, once, copies its 64 tokens'
//     full activation rows into LDS with direct global->LDS loads (whole
//     lines).  16-byte chunk c of token t is stored at chunk c ^ (t & 15) of
//     the token's row, so 16 tokens reading the same permuted column hit 16
//     different bank groups;
//   * perm and the index bits of the tile's 256 rows are copied once too;
//   * packed values stream through a double-buffered one-step LDS stage;
//   * each B fragment element is read from the token rows through perm (one
//     2-byte LDS read per element), packed, and fed to v_smfmac.
// Waves are 2 x 2 (128 rows x 32 tokens each).
#include "nm_internal.h"

namespace nm {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16_t __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_byte;

template <int DT>
__device__ inline f32x4 smfmac(const u32x4& a, const u32x8& b, const f32x4& c, uint32_t idx) {
  if constexpr (DT == NM_F16) {
    return __builtin_amdgcn_smfmac_f32_16x16x64_f16(__builtin_bit_cast(half8_t, a),
                                                    __builtin_bit_cast(half16_t, b), c, int(idx), 0, 0);
  } else {
    return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf8_t, a),
                                                     __builtin_bit_cast(bf16_t, b), c, int(idx), 0, 0);
  }
}

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

template <int DT>
__device__ inline uint16_t to_half_bits(float f) {
  if constexpr (DT == NM_F16) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
  } else {
    return f32_to_bf16_rne(f);
  }
}

__device__ inline void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ inline void wait_all_vm() { __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8)); }

__device__ inline void dma16(const void* src, unsigned char* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_byte*)dst, 16, 0, 0);
}

constexpr int kBR = 256, kBT = 64;
constexpr int kKMax = 768;
constexpr int kXBytes = kBT * kKMax * 2;          // token rows, 96 KB
constexpr int kPermBytes = kKMax * 4 + 1024;      // perm (+ tail of the last copy)
constexpr int kIdxBytes = kBR * (kKMax / 8);      // index bits of the tile's rows
constexpr int kStageA = kBR * 64;                 // one K step of packed values
constexpr int kLds = kXBytes + kPermBytes + kIdxBytes + 2 * kStageA;

template <int DT, int OUT>
__global__ __launch_bounds__(256, 1) void spmm_perm_kernel(
    const uint16_t* __restrict__ values, const uint32_t* __restrict__ idx, int R, int K,
    const uint16_t* __restrict__ act, int T, int64_t ldx, const int32_t* __restrict__ perm,
    void* __restrict__ Y, int64_t ldy, int tilesR, int tilesT) {
  constexpr int FR = 8, FT = 2;
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* xs = smem;
  unsigned char* ps = smem + kXBytes;
  unsigned char* is = ps + kPermBytes;
  unsigned char* as = is + kIdxBytes;  // [2][kStageA]

  // consecutive workgroups share a token tile (its rows stay in L2)
  const int tr = blockIdx.x % tilesR, tt = blockIdx.x / tilesR;
  const int R0 = tr * kBR, T0 = tt * kBT;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wt = wave & 1;
  const int li = lane & 15, lq = lane >> 4;
  const int nsteps = K >> 6;
  const int CH = K >> 3;          // 16-byte chunks per token row
  const int S = K >> 1;
  const int irow = K >> 3;        // index bytes per row
  const int ich = K >> 7;         // 16-byte index chunks per row

  // ---- one-time copies: token rows, perm, index bits
  {
    const int nx = kBT * CH / 64;  // instructions for the token rows (CH % 16 == 0)
    for (int j = wave; j < nx; j += 4) {
      const int slot = j * 64 + lane;
      const int tok = slot / CH;
      const int c = (slot % CH) ^ (tok & 15);
      const int t = min(T0 + tok, T - 1);
      dma16(act + int64_t(t) * ldx + c * 8, xs + j * 1024);
    }
    const int np = (K / 4 + 63) / 64;
    for (int j = wave; j < np; j += 4) {
      int c = j * 64 + lane;
      if (c >= K / 4) c = 0;
      dma16(perm + c * 4, ps + j * 1024);
    }
    const int ni = kBR * ich / 64;
    for (int j = wave; j < ni; j += 4) {
      const int slot = j * 64 + lane;
      const int row = slot / ich;
      const int c = slot % ich;
      const int r = min(R0 + row, R - 1);
      dma16(reinterpret_cast<const unsigned char*>(idx) + int64_t(r) * irow + c * 16, is + j * 1024);
    }
  }
  // packed values of step s: slot (row, quarter q') holds quarter q' ^ ((row >> 2) & 3)
  const uint16_t* asrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int slot = (wave * 4 + j) * 64 + lane;
    const int row = slot >> 2;
    const int q = (slot & 3) ^ ((row >> 2) & 3);
    const int r = min(R0 + row, R - 1);
    asrc[j] = values + int64_t(r) * S + q * 8;
  }
  auto issue_a = [&](int s, int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(asrc[j] + s * 32, as + buf * kStageA + (wave * 4 + j) * 1024);
  };

  f32x4 acc[FR][FT];
#pragma unroll
  for (int i = 0; i < FR; ++i)
#pragma unroll
    for (int j = 0; j < FT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  issue_a(0, 0);
  for (int s = 0; s < nsteps; ++s) {
    wait_all_vm();
    barrier_no_fence();
    if (s + 1 < nsteps) issue_a(s + 1, (s + 1) & 1);
    const unsigned char* sa = as + (s & 1) * kStageA;
    // A fragments
    u32x4 a[FR];
    uint32_t ix[FR];
#pragma unroll
    for (int i = 0; i < FR; ++i) {
      const int row = wr * 128 + i * 16 + li;
      a[i] = *reinterpret_cast<const u32x4*>(sa + (row * 4 + (lq ^ ((row >> 2) & 3))) * 16);
      ix[i] = *reinterpret_cast<const uint16_t*>(is + row * irow + s * 8 + lq * 2);
    }
    // the 16 permuted K positions of this lane: k = 64s + 32h + 8lq + e
    int32_t kp[16];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const i32x4 p0 = *reinterpret_cast<const i32x4*>(ps + (s * 64 + h * 32 + lq * 8) * 4);
      const i32x4 p1 = *reinterpret_cast<const i32x4*>(ps + (s * 64 + h * 32 + lq * 8 + 4) * 4);
      kp[8 * h + 0] = p0[0]; kp[8 * h + 1] = p0[1]; kp[8 * h + 2] = p0[2]; kp[8 * h + 3] = p0[3];
      kp[8 * h + 4] = p1[0]; kp[8 * h + 5] = p1[1]; kp[8 * h + 6] = p1[2]; kp[8 * h + 7] = p1[3];
    }
    // byte offsets inside a token row for this lane (token & 15 == li for every fragment)
    uint32_t off[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) off[e] = uint32_t((((kp[e] >> 3) ^ li) << 4) | ((kp[e] & 7) << 1));
    u32x8 bf[FT];
#pragma unroll
    for (int j = 0; j < FT; ++j) {
      const unsigned char* trow = xs + (wt * 32 + j * 16 + li) * (K * 2);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = *reinterpret_cast<const uint16_t*>(trow + off[2 * e]);
        const uint32_t hi = *reinterpret_cast<const uint16_t*>(trow + off[2 * e + 1]);
        bf[j][e] = lo | (hi << 16);
      }
    }
#pragma unroll
    for (int j = 0; j < FT; ++j)
#pragma unroll
      for (int i = 0; i < FR; ++i) acc[i][j] = smfmac<DT>(a[i], bf[j], acc[i][j], ix[i]);
  }

  // ---- epilogue
  const bool vec_ok = (ldy & 3) == 0;
#pragma unroll
  for (int i = 0; i < FR; ++i) {
    const int r = R0 + wr * 128 + i * 16 + lq * 4;
#pragma unroll
    for (int j = 0; j < FT; ++j) {
      const int t = T0 + wt * 32 + j * 16 + li;
      if (t >= T || r >= R) continue;
      const f32x4 v = acc[i][j];
      if constexpr (OUT == NM_F32) {
        float* y = static_cast<float*>(Y) + int64_t(t) * ldy + r;
        if (vec_ok && r + 3 < R) {
          *reinterpret_cast<f32x4*>(y) = v;
        } else {
          for (int e = 0; e < 4 && r + e < R; ++e) y[e] = v[e];
        }
      } else {
        uint16_t* y = static_cast<uint16_t*>(Y) + int64_t(t) * ldy + r;
        const uint16_t h0 = to_half_bits<DT>(v[0]), h1 = to_half_bits<DT>(v[1]);
        const uint16_t h2 = to_half_bits<DT>(v[2]), h3 = to_half_bits<DT>(v[3]);
        if (vec_ok && r + 3 < R) {
          *reinterpret_cast<uint2*>(y) = make_uint2(uint32_t(h0) | (uint32_t(h1) << 16),
                                                    uint32_t(h2) | (uint32_t(h3) << 16));
        } else {
          const uint16_t hh[4] = {h0, h1, h2, h3};
          for (int e = 0; e < 4 && r + e < R; ++e) y[e] = hh[e];
        }
      }
    }
  }
}

template <int DT, int OUT>
hipError_t launch_perm(const SpmmArgs& a, hipStream_t s) {
  const int tilesR = int((a.R + kBR - 1) / kBR);
  const int tilesT = int((a.T + kBT - 1) / kBT);
  const int64_t ntiles = int64_t(tilesR) * tilesT;
  if (ntiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  auto kern = spmm_perm_kernel<DT, OUT>;
  if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), kLds); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(unsigned(ntiles)), dim3(256), kLds, s, a.values, a.idx, int(a.R),
                     int(a.K), a.act, int(a.T), a.ldx, a.perm, a.Y, a.ldy, tilesR, tilesT);
  return hipGetLastError();
}

}  // namespace

bool spmm_perm_lds_applies(const SpmmArgs& a) {
  if (!(a.perm != nullptr && a.n == 2 && a.m == 4 && a.K % 128 == 0 && a.K <= kKMax &&
        a.T >= 64 && a.R >= 256))
    return false;
  return device_max_lds() >= kLds;
}

hipError_t launch_spmm_perm_lds(const SpmmArgs& a, hipStream_t s) {
  if (a.dtype == NM_F16)
    return a.out_dtype == NM_F32 ? launch_perm<NM_F16, NM_F32>(a, s) : launch_perm<NM_F16, NM_F16>(a, s);
  return a.out_dtype == NM_F32 ? launch_perm<NM_BF16, NM_F32>(a, s) : launch_perm<NM_BF16, NM_BF16>(a, s);
}

}  // namespace nm
