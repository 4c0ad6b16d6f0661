// 2:4 sparse GEMM for prefill shapes with every operand staged through LDS
// by direct global->LDS loads (gfx950 global_load_lds_dwordx4).
//
// Same product as nm_spmm.hip (Y^T[t, r] = sum_k W_nm[r, k] act[t, k] on
// v_smfmac_f32_16x16x64).  What this kernel is organised around is the cost
// of L2 requests: no lane loads fewer than 16 bytes and every instruction
// reads 64- or 128-byte runs.  A direct load deposits lane l's 16 bytes at
// slot base + l of LDS, so the LDS layout is chosen by which global address
// each lane reads:
//
//   packed values  one K step per stage; slot (row, quarter q) at
//                  row*4 + (q ^ ((row >> 2) & 3)): an instruction covers 16 rows
//                  x 64 bytes, and a fragment read by 8 consecutive rows hits
//                  distinct bank groups;
//   activations    one K step per stage; slot (token, chunk c) at
//                  token*8 + (c ^ (token & 7)): 8 tokens x 128 bytes per
//                  instruction;
//   index bits     block = 8 K steps (64 bytes per row); slot (row, chunk) at
//                  row*4 + (chunk ^ ((row >> 2) & 3)).
//
// A workgroup (4 waves) owns a 256 x 128 tile; waves are 2 x 2, each owning
// 128 rows x 64 tokens (8 x 4 fragments: the fragment-read volume per MFMA is
// lowest for this split).  Stages form a 4-deep ring, so three K steps of
// loads are in flight while one is computed; each step waits (counted vmcnt)
// for exactly its own loads and passes one fence-free barrier, which both
// publishes it and retires the slot the step's new loads reuse.
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

__device__ inline void wait_all_vm() {
  // vmcnt(0), expcnt/lgkmcnt untouched (gfx9 encoding)
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
}

__device__ inline void dma16(const void* src, unsigned char* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_byte*)lds_dst, 16, 0, 0);
}

constexpr int kBR = 256;
constexpr int kBT = 128;
constexpr int kNS = 4;                     // one-K-step stages in the ring
constexpr int kStageB = kBT * 128;         // activations, one step
constexpr int kStageA = kBR * 64;          // packed values, one step
constexpr int kBlockI = kBR * 64;          // index bits, 8 steps
constexpr int kLds = kNS * (kStageB + kStageA) + 2 * kBlockI;
constexpr int kPerStep = 8;                // direct loads per wave per step (4 B + 4 A)

template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

template <int DT, int OUT>
__global__ __launch_bounds__(256, 1) void spmm_lds_kernel(
    const uint16_t* __restrict__ values, const uint32_t* __restrict__ idx, int R, int K,
    const uint16_t* __restrict__ act, int T, int64_t ldx, void* __restrict__ Y, int64_t ldy,
    int tilesR, int tilesT, int group_r) {
  constexpr int FR = 8, FT = kBT / 32;
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* bbuf = smem;                              // [kNS][kStageB]
  unsigned char* abuf = smem + kNS * kStageB;              // [kNS][kStageA]
  unsigned char* ibuf = smem + kNS * (kStageB + kStageA);  // [2][kBlockI]

  // ---- tile: XCD-aware remap, then groups of group_r row tiles sharing X
  const int ntiles = tilesR * tilesT;
  int b = blockIdx.x;
  if ((ntiles & 7) == 0) b = (b & 7) * (ntiles >> 3) + (b >> 3);
  const int per_group = group_r * tilesT;
  const int grp = b / per_group;
  const int rem = b - grp * per_group;
  const int rows_in_grp = min(group_r, tilesR - grp * group_r);
  const int tr = grp * group_r + rem % rows_in_grp;
  const int tt = rem / rows_in_grp;
  const int R0 = tr * kBR, T0 = tt * kBT;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lq = lane >> 4;
  const int wr = wave >> 1, wt = wave & 1;
  const int nsteps = K >> 6;                 // K % 128 == 0 on this path
  const int S = K >> 1;                      // packed values per row
  const int irow_bytes = K >> 3;             // index bytes per row (2 bits per survivor)

  // Per-lane source pointers.  Instruction j of a wave fills slots
  // [(wave*4 + j)*64, +64); lane l takes slot base + l.
  // Activations, one step: slot (token, chunk) at token*8 + (c ^ (token & 7)).
  const unsigned char* bsrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int slot = (wave * 4 + j) * 64 + lane;
    const int tok = slot >> 3;
    const int c = (slot & 7) ^ (tok & 7);
    const int t = min(T0 + tok, T - 1);
    bsrc[j] = reinterpret_cast<const unsigned char*>(act + int64_t(t) * ldx + c * 8);
  }
  // Packed values, one step: slot (row, quarter) at row*4 + (q ^ ((row >> 2) & 3)).
  const unsigned char* asrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int slot = (wave * 4 + j) * 64 + lane;
    const int row = slot >> 2;
    const int q = (slot & 3) ^ ((row >> 2) & 3);
    const int r = min(R0 + row, R - 1);
    asrc[j] = reinterpret_cast<const unsigned char*>(values + int64_t(r) * S + q * 8);
  }
  // Index bits, 8 steps: slot (row, chunk) at row*4 + (c ^ ((row >> 2) & 3)).
  const unsigned char* isrc[4];
  int ichunk[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int slot = (wave * 4 + j) * 64 + lane;
    const int row = slot >> 2;
    const int c = (slot & 3) ^ ((row >> 2) & 3);
    const int r = min(R0 + row, R - 1);
    ichunk[j] = c;
    isrc[j] = reinterpret_cast<const unsigned char*>(idx) + int64_t(r) * irow_bytes + c * 16;
  }

  auto issue_step = [&](int s) {
    const int buf = s & (kNS - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dma16(bsrc[j] + int64_t(s) * 128, bbuf + buf * kStageB + (wave * 4 + j) * 1024);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dma16(asrc[j] + int64_t(s) * 64, abuf + buf * kStageA + (wave * 4 + j) * 1024);
  };
  auto issue_index = [&](int q) {
    const int steps_left = nsteps - 8 * q;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // chunk c holds steps 2c, 2c+1 of the block (steps_left is even); past
      // the row's end the lane rereads chunk 0 of the block
      const int back = (2 * ichunk[j] < steps_left) ? 0 : ichunk[j] * 16;
      dma16(isrc[j] + int64_t(q) * 64 - back, ibuf + (q & 1) * kBlockI + (wave * 4 + j) * 1024);
    }
  };

  f32x4 acc[FR][FT];
#pragma unroll
  for (int i = 0; i < FR; ++i)
#pragma unroll
    for (int j = 0; j < FT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- prologue: index block 0, then steps 0 .. kNS-2
  issue_index(0);
#pragma unroll
  for (int p = 0; p < kNS - 1; ++p)
    if (p < nsteps) issue_step(p);

  for (int s = 0; s < nsteps; ++s) {
    // Step s has landed once at most the loads issued after it remain: those
    // of steps s+1, s+2 (an index block issued in between only makes the
    // wait stricter).
    if (s + 2 < nsteps) wait_vmcnt<2 * kPerStep>();
    else if (s + 1 < nsteps) wait_vmcnt<kPerStep>();
    else wait_vmcnt<0>();
    barrier_no_fence();  // publishes step s, retires step s - 1
    if (s + kNS - 1 < nsteps) issue_step(s + kNS - 1);
    if ((s & 7) == 0 && s + 8 < nsteps) issue_index((s >> 3) + 1);

    const unsigned char* sb = bbuf + (s & (kNS - 1)) * kStageB;
    const unsigned char* sa = abuf + (s & (kNS - 1)) * kStageA;
    const unsigned char* si = ibuf + ((s >> 3) & 1) * kBlockI;
    const int u8 = s & 7;
    u32x4 a[FR];
    uint32_t ix[FR];
#pragma unroll
    for (int i = 0; i < FR; ++i) {
      const int row = wr * 128 + i * 16 + li;
      a[i] = *reinterpret_cast<const u32x4*>(sa + (row * 4 + (lq ^ ((row >> 2) & 3))) * 16);
      const int ch = (u8 >> 1) ^ ((row >> 2) & 3);
      ix[i] = *reinterpret_cast<const uint16_t*>(si + row * 64 + ch * 16 + (u8 & 1) * 8 + lq * 2);
    }
    u32x8 bf[FT];
#pragma unroll
    for (int j = 0; j < FT; ++j) {
      const int tok = wt * (kBT / 2) + j * 16 + li;
      const int sw = tok & 7;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(sb + (tok * 8 + (lq ^ sw)) * 16);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(sb + (tok * 8 + ((lq + 4) ^ sw)) * 16);
      bf[j] = u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int j = 0; j < FT; ++j)
#pragma unroll
      for (int i = 0; i < FR; ++i) acc[i][j] = smfmac<DT>(a[i], bf[j], acc[i][j], ix[i]);
    // Schedule: the A reads and the first B fragment, then MFMAs with the
    // remaining B reads spread between them.
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * FR + 2, 0);
    for (int k = 0; k < 2 * FT - 2; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, FR * FT - 2 * (2 * FT - 2), 0);
  }

  // ---- epilogue
  const bool vec_ok = (ldy & 3) == 0;
#pragma unroll
  for (int i = 0; i < FR; ++i) {
    const int r = R0 + wr * 128 + i * 16 + lq * 4;
#pragma unroll
    for (int j = 0; j < FT; ++j) {
      const int t = T0 + wt * (kBT / 2) + j * 16 + li;
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
hipError_t launch_lds(const SpmmArgs& a, hipStream_t s) {
  const int tilesR = int((a.R + kBR - 1) / kBR);
  const int tilesT = int((a.T + kBT - 1) / kBT);
  const int64_t ntiles = int64_t(tilesR) * tilesT;
  if (ntiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int group_r = tilesR < 4 ? tilesR : 4;
  auto kern = spmm_lds_kernel<DT, OUT>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(unsigned(ntiles)), dim3(256), kLds, s, a.values, a.idx, int(a.R),
                     int(a.K), a.act, int(a.T), a.ldx, a.Y, a.ldy, tilesR, tilesT, group_r);
  return hipGetLastError();
}

}  // namespace

bool spmm_lds_applies(const SpmmArgs& a) {
  if (!(a.perm == nullptr && a.n == 2 && a.m == 4 && (a.K % 128) == 0 && a.T >= 128 &&
        a.R >= 256))
    return false;
  // needs a workgroup LDS allocation of kLds bytes
  static int max_lds = -1;
  if (max_lds < 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
      v = 0;
    max_lds = v;
  }
  return max_lds >= kLds;
}

hipError_t launch_spmm_lds(const SpmmArgs& a, hipStream_t s) {
  if (a.dtype == NM_F16)
    return a.out_dtype == NM_F32 ? launch_lds<NM_F16, NM_F32>(a, s) : launch_lds<NM_F16, NM_F16>(a, s);
  return a.out_dtype == NM_F32 ? launch_lds<NM_BF16, NM_F32>(a, s) : launch_lds<NM_BF16, NM_BF16>(a, s);
}

}  // namespace nm
