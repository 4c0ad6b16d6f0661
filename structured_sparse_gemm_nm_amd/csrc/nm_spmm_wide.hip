// 2:4 sparse GEMM with 256 x 256 output tiles (prefill shapes), operands
// staged through LDS by direct buffer->LDS loads.
//
// Same product as nm_spmm.hip (Y^T[t, r] = sum_k W_nm[r, k] act[t, k] on
// v_smfmac_f32_16x16x64).  Per 64-wide K step a workgroup loads 16 KB of
// packed values, 32 KB of activations and 2 KB of index bits and runs 64
// smfmac per wave: 48 KB per 256 x 256 x 64 step against 32 KB per
// 256 x 128 x 64 step for 128-token tiles, i.e. a quarter fewer bytes per
// MFMA through L2, the load path and LDS.  Four waves (2 x 2) each own
// 128 rows x 128 tokens (8 x 8 fragments, 256 fp32 accumulators per lane).
//
// LDS layouts (XOR swizzles picked by measuring the bank-conflict counter for
// these exact reads; all read without conflicts):
//   packed values  one K step per stage, slot (row, quarter q) at
//                  row*4 + (q ^ ((row >> 1) & 3)); a load covers 16 rows x 64 B;
//   activations    one K step per stage, slot (token, chunk c) at
//                  token*8 + (c ^ (token & 7)); 8 tokens x 128 B per load;
//   index bits     block = 4 K steps (32 bytes per row), slot (row, chunk c) at
//                  row*2 + (c ^ ((row >> 3) & 1)); a lane reads its row's 8
//                  bytes of a step and keeps its 2 by a byte permute.
// Stages form a 3-deep ring (2 x 48 KB in flight while one is read); index
// blocks are double-buffered.  The fragment reads of step s+1 are issued
// between the MFMAs of step s (packed values into a second register set,
// activations into the registers a fragment frees once its MFMAs are issued).
// Accumulators live in AGPRs, operands in VGPRs.
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

__device__ inline void wait_lgkm0() {
  // lgkmcnt(0), vmcnt/expcnt untouched (gfx9 encoding)
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14));
}

template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Buffer resource over [base, base + 4 GiB): raw 32-bit data; every offset
// used here is clamped by the caller.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}

// 16 bytes per lane from base + voff + soff into LDS slot lds_dst + lane*16.
__device__ inline void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, unsigned char* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_byte*)lds_dst, 16, int(voff), int(soff), 0, 0);
}

constexpr int kBR = 256;
constexpr int kBT = 256;
constexpr int kNS = 3;                      // one-K-step stages in the ring
constexpr int kStageA = kBR * 64;           // packed values, one step (16 KB)
constexpr int kStageB = kBT * 128;          // activations, one step (32 KB)
constexpr int kBlockI = kBR * 32;           // index bits, 4 steps (8 KB)
constexpr int kLds = kNS * (kStageA + kStageB) + 2 * kBlockI;  // 160 KB
constexpr int kLoadsB = 8, kLoadsA = 4;     // direct loads per wave per step
constexpr int kPerStep = kLoadsB + kLoadsA;

template <int DT, int OUT>
__global__ __launch_bounds__(256, 1) void spmm_wide_kernel(
    const uint16_t* __restrict__ values, const uint32_t* __restrict__ idx, int R, int K,
    const uint16_t* __restrict__ act, int T, int64_t ldx, void* __restrict__ Y, int64_t ldy,
    int tilesR, int tilesT, int group_r) {
  constexpr int FR = 8, FT = 8;
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* abuf = smem;                              // [kNS][kStageA]
  unsigned char* bbuf = smem + kNS * kStageA;              // [kNS][kStageB]
  unsigned char* ibuf = smem + kNS * (kStageA + kStageB);  // [2][kBlockI]

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
  const int nsteps = K >> 6;                 // even: K % 128 == 0 on this path
  const int S = K >> 1;                      // packed values per row
  const int irow_bytes = K >> 3;             // index bytes per row (2 bits per survivor)

  const __amdgpu_buffer_rsrc_t bsrc = make_rsrc(act + int64_t(T0) * ldx);
  const __amdgpu_buffer_rsrc_t asrc = make_rsrc(values + int64_t(R0) * S);
  const __amdgpu_buffer_rsrc_t isrc = make_rsrc(reinterpret_cast<const unsigned char*>(idx) + int64_t(R0) * irow_bytes);
  // Per-lane byte offsets (loop invariant).  Load j of a wave fills slots
  // [(wave*n + j)*64, +64) of its region; lane l takes slot base + l.
  uint32_t boff[kLoadsB];
#pragma unroll
  for (int j = 0; j < kLoadsB; ++j) {
    const int slot = (wave * kLoadsB + j) * 64 + lane;
    const int tok = slot >> 3;
    const int c = (slot & 7) ^ (tok & 7);
    const int t = min(T0 + tok, T - 1) - T0;
    boff[j] = uint32_t(t) * uint32_t(ldx) * 2u + uint32_t(c) * 16u;
  }
  uint32_t aoff[kLoadsA];
#pragma unroll
  for (int j = 0; j < kLoadsA; ++j) {
    const int slot = (wave * kLoadsA + j) * 64 + lane;
    const int row = slot >> 2;
    const int q = (slot & 3) ^ ((row >> 1) & 3);
    const int r = min(R0 + row, R - 1) - R0;
    aoff[j] = uint32_t(r) * uint32_t(S) * 2u + uint32_t(q) * 16u;
  }
  uint32_t ioff[2];
  int ichunk[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int slot = (wave * 2 + j) * 64 + lane;
    const int row = slot >> 1;
    const int c = (slot & 1) ^ ((row >> 3) & 1);
    const int r = min(R0 + row, R - 1) - R0;
    ichunk[j] = c;
    ioff[j] = uint32_t(r) * uint32_t(irow_bytes) + uint32_t(c) * 16u;
  }

  // Load j (0..7 activations, 8..11 packed values) of step src into ring slot buf.
  auto issue_load = [&](int j, int src, int buf) {
    if (j < kLoadsB)
      dma16(bsrc, boff[j], uint32_t(src) * 128u, bbuf + buf * kStageB + (wave * kLoadsB + j) * 1024);
    else
      dma16(asrc, aoff[j - kLoadsB], uint32_t(src) * 64u,
            abuf + buf * kStageA + (wave * kLoadsA + j - kLoadsB) * 1024);
  };
  auto issue_step = [&](int src, int buf) {
#pragma unroll
    for (int j = 0; j < kPerStep; ++j) issue_load(j, src, buf);
  };
  auto issue_index = [&](int q) {
    const int steps_left = nsteps - 4 * q;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // chunk c holds steps 2c, 2c+1 of the block (steps_left is even); past
      // the row's end the lane rereads chunk 0 of the block
      const uint32_t back = (2 * ichunk[j] < steps_left) ? 0u : uint32_t(ichunk[j]) * 16u;
      dma16(isrc, ioff[j] - back, uint32_t(q) * 32u, ibuf + (q & 1) * kBlockI + (wave * 2 + j) * 1024);
    }
  };

  // byte selector: bytes 2*lq, 2*lq+1 of {hi, lo} into bits 0..15, zeros above
  const uint32_t ix_sel = uint32_t(2 * lq) | (uint32_t(2 * lq + 1) << 8) | (0x0C0Cu << 16);
  auto read_a = [&](int slot, int s, int i, u32x4& a, uint2& ix) {
    const unsigned char* sa = abuf + slot * kStageA;
    const unsigned char* si = ibuf + ((s >> 2) & 1) * kBlockI;
    const int row = wr * 128 + i * 16 + li;
    a = *reinterpret_cast<const u32x4*>(sa + (row * 4 + (lq ^ ((row >> 1) & 3))) * 16);
    // (read as uint64_t: through the uint2 struct the compiler cannot tell
    // this from the slots the direct loads are filling and waits for them)
    const int u4 = s & 3;
    const int ch = (u4 >> 1) ^ ((row >> 3) & 1);
    const uint64_t w = *reinterpret_cast<const uint64_t*>(si + row * 32 + ch * 16 + (u4 & 1) * 8);
    ix.x = uint32_t(w);
    ix.y = uint32_t(w >> 32);
  };
  auto read_b = [&](int slot, int j, int h, u32x8& bf) {
    const unsigned char* sb = bbuf + slot * kStageB;
    const int tok = wt * 128 + j * 16 + li;
    const u32x4 v = *reinterpret_cast<const u32x4*>(sb + (tok * 8 + ((lq + 4 * h) ^ (tok & 7))) * 16);
    bf[4 * h + 0] = v[0];
    bf[4 * h + 1] = v[1];
    bf[4 * h + 2] = v[2];
    bf[4 * h + 3] = v[3];
  };

  // 256 accumulators per lane have to live in AGPRs; zeroing them with
  // AGPR writes makes the register allocator keep them there (left to
  // itself it starts them in VGPRs and then shuffles).
  f32x4 acc[FR][FT];
#pragma unroll
  for (int i = 0; i < FR; ++i)
#pragma unroll
    for (int j = 0; j < FT; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float z;
        asm volatile("v_accvgpr_write_b32 %0, 0" : "=a"(z));
        acc[i][j][e] = z;
      }

  // Packed values of step s+1 are read into a second set and copied over at
  // the end of step s (the copies co-issue with MFMAs); each token fragment
  // has one set: fragment k of step s+1 is read into it right after the last
  // MFMA of step s that uses it.
  u32x4 ca[FR], na[FR];
  uint2 xr[FR];   // raw index words of the next step
  u32x8 bf[FT];

  // One step: make step s+1 visible, refill the slot step s used, read step
  // s+1, multiply step s.  Every step issues the same loads (past the last
  // step a slot nothing reads any more is refilled with the last step), so
  // the wait count is fixed and the block has no branch.  Eight chunks, each:
  // the 8 MFMAs of token fragment k, one or two loads and four fragment reads.
  auto body = [&](int s, int slot, int nslot) {
    // step s+1 has landed once at most the loads of step s+2 remain (an
    // index block issued in between only makes the wait stricter)
    wait_vmcnt<kPerStep>();
    wait_lgkm0();        // this wave's reads of step s are done
    barrier_no_fence();  // publishes step s+1; every wave is done reading step s
    if ((s & 3) == 0 && s + 4 < nsteps) issue_index((s >> 2) + 1);
    const int src = min(s + kNS, nsteps - 1);
    uint32_t ik[FR];
#pragma unroll
    for (int i = 0; i < FR; ++i) ik[i] = __builtin_amdgcn_perm(xr[i].y, xr[i].x, ix_sel);
#pragma unroll
    for (int k = 0; k < FT; ++k) {
#pragma unroll
      for (int i = 0; i < FR; ++i) acc[i][k] = smfmac<DT>(ca[i], bf[k], acc[i][k], ik[i]);
      issue_load(k, src, slot);
      if (k < kLoadsA) issue_load(kLoadsB + k, src, slot);
      read_b(nslot, k, 0, bf[k]);
      read_b(nslot, k, 1, bf[k]);
      read_a(nslot, s + 1, k, na[k], xr[k]);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < FR; ++i) ca[i] = na[i];
  };

  // ---- prologue: index block 0 and steps 0, 1; then step 0 into set 0
  issue_index(0);
  issue_step(0, 0);
  issue_step(min(1, nsteps - 1), 1);
  wait_vmcnt<kPerStep>();
  barrier_no_fence();
  issue_step(min(2, nsteps - 1), 2);  // slot 2 is still unused
#pragma unroll
  for (int i = 0; i < FR; ++i) read_a(0, 0, i, ca[i], xr[i]);
#pragma unroll
  for (int j = 0; j < FT; ++j) {
    read_b(0, j, 0, bf[j]);
    read_b(0, j, 1, bf[j]);
  }

  int slot = 0;  // ring slot of step s
  for (int s = 0; s < nsteps; ++s) {
    const int s1 = slot == kNS - 1 ? 0 : slot + 1;
    body(s, slot, s1);
    slot = s1;
  }
  wait_vmcnt<0>();  // no load may still be writing LDS when the workgroup ends

  // ---- epilogue: interior tiles store without any test; edge tiles store
  // element by element under a mask
  const bool interior = (R0 + kBR <= R) && (T0 + kBT <= T) && (ldy & 3) == 0;
  // Accumulators are read out of AGPRs explicitly (so they stay there until
  // here); 24 wait states first cover the last MFMA's write of them.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  auto out4 = [&](const f32x4& a) {
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v[e]) : "a"(a[e]));
    return v;
  };
  const int rl = R0 + wr * 128 + lq * 4;
  const int tl = T0 + wt * 128 + li;
  if (interior) {
#pragma unroll
    for (int i = 0; i < FR; ++i)
#pragma unroll
      for (int j = 0; j < FT; ++j) {
        const f32x4 v = out4(acc[i][j]);
        const int64_t off = int64_t(tl + j * 16) * ldy + rl + i * 16;
        if constexpr (OUT == NM_F32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(Y) + off) = v;
        } else {
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(Y) + off) =
              make_uint2(uint32_t(to_half_bits<DT>(v[0])) | (uint32_t(to_half_bits<DT>(v[1])) << 16),
                         uint32_t(to_half_bits<DT>(v[2])) | (uint32_t(to_half_bits<DT>(v[3])) << 16));
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < FR; ++i)
#pragma unroll
      for (int j = 0; j < FT; ++j) {
        const f32x4 v = out4(acc[i][j]);
        const int t = tl + j * 16, r = rl + i * 16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (t < T && r + e < R) {
            if constexpr (OUT == NM_F32)
              static_cast<float*>(Y)[int64_t(t) * ldy + r + e] = v[e];
            else
              static_cast<uint16_t*>(Y)[int64_t(t) * ldy + r + e] = to_half_bits<DT>(v[e]);
          }
        }
      }
  }
}

template <int DT, int OUT>
hipError_t launch_wide(const SpmmArgs& a, hipStream_t s) {
  const int tilesR = int((a.R + kBR - 1) / kBR);
  const int tilesT = int((a.T + kBT - 1) / kBT);
  const int64_t ntiles = int64_t(tilesR) * tilesT;
  if (ntiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int group_r = tilesR < 4 ? tilesR : 4;
  auto kern = spmm_wide_kernel<DT, OUT>;
  if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), kLds); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(unsigned(ntiles)), dim3(256), kLds, s, a.values, a.idx, int(a.R),
                     int(a.K), a.act, int(a.T), a.ldx, a.Y, a.ldy, tilesR, tilesT, group_r);
  return hipGetLastError();
}

}  // namespace

bool spmm_wide_applies(const SpmmArgs& a) {
  if (!(a.perm == nullptr && a.n == 2 && a.m == 4 && (a.K % 128) == 0 && a.T >= 256 &&
        a.R >= 256))
    return false;
  // per-lane byte offsets within a tile are 32-bit
  const int64_t lim = int64_t(0xFFFFFFFFu);
  if (int64_t(kBT) * a.ldx * 2 > lim || int64_t(kBR) * a.K > lim) return false;
  return device_max_lds() >= kLds;
}

hipError_t launch_spmm_wide(const SpmmArgs& a, hipStream_t s) {
  if (a.dtype == NM_F16)
    return a.out_dtype == NM_F32 ? launch_wide<NM_F16, NM_F32>(a, s) : launch_wide<NM_F16, NM_F16>(a, s);
  return a.out_dtype == NM_F32 ? launch_wide<NM_BF16, NM_F32>(a, s) : launch_wide<NM_BF16, NM_BF16>(a, s);
}

}  // namespace nm
