// Device helpers shared by the gfx950 kernels: operand vector types, the
// sparse and dense MFMA, conversions and output rounding, counted waits and
// direct global->LDS loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nmsparse.h"

namespace nm {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16_t __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) unsigned char lds_byte;

// D = C + A x B on v_smfmac_f32_16x16x64_{f16,bf16}: A is 16 rows x 64 K in
// 2:4 form (8 stored halves per lane), B 64 K x 16 columns (16 halves per
// lane), idx the 16 index bits of the lane's 8 stored values; ABID picks the
// low (0) or high (1) 16-bit half of the index register.
template <int DT, int ABID = 0>
__device__ inline f32x4 smfmac(const u32x4& a, const u32x8& b, const f32x4& c, uint32_t idx) {
  if constexpr (DT == NM_F16) {
    return __builtin_amdgcn_smfmac_f32_16x16x64_f16(__builtin_bit_cast(half8_t, a),
                                                    __builtin_bit_cast(half16_t, b), c, int(idx), 0, ABID);
  } else {
    return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf8_t, a),
                                                     __builtin_bit_cast(bf16_t, b), c, int(idx), 0, ABID);
  }
}

// D = C + A x B on the dense v_mfma_f32_16x16x32_{f16,bf16}: lane (i, q)
// holds A[i][8q..8q+7] and B[8q..8q+7][i]; D rows 4q..4q+3 of column i.
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

// A 16-bit storage value (low 16 bits of h) as fp32.
template <int DT>
__device__ inline float half_to_f32(uint32_t h) {
  if constexpr (DT == NM_F16) {
    return float(__builtin_bit_cast(_Float16, uint16_t(h)));
  } else {
    return __builtin_bit_cast(float, h << 16);
  }
}

// Unsigned minimum (the map clamp: an entry outside [0, K) reads column K-1).
__device__ inline uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }

// fp32 -> the 16-bit storage type DT by the hardware conversions, round to
// nearest even: v_cvt_f16_f32, and for bf16 v_cvt_pk_bf16_f32, whose bits equal
// the integer rounding of the fp32 pattern (add 0x7FFF plus the kept lsb, keep
// the top half; a NaN quieted with its top payload bits) for every input
// checked: 4M random patterns and the halfway, denormal, overflow and
// NaN-payload cases.  One instruction per pair of outputs.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

template <int DT>
__device__ inline uint16_t to_half_bits(float f) {
  if constexpr (DT == NM_F16) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
  } else {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
  }
}

// Two rounded outputs packed into one 32-bit word, the first in the low half.
template <int DT>
__device__ inline uint32_t pack_half2(float lo, float hi) {
  if constexpr (DT == NM_F16) {
    return uint32_t(to_half_bits<DT>(lo)) | (uint32_t(to_half_bits<DT>(hi)) << 16);
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
  }
}

// s_barrier without the fence __syncthreads() adds (which waits for every
// outstanding global load): callers wait for exactly what they need first.
__device__ inline void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// lgkmcnt(0), vmcnt/expcnt untouched (gfx9 encoding): this wave's LDS
// operations are done.
__device__ inline void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14));
}

// vmcnt(N): at most the newest N vector-memory operations of this wave are
// still outstanding (loads and stores retire from the counter in issue order).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Buffer resource over [base, base + 4 GiB): raw 32-bit data (callers keep
// every offset inside their buffers).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}

// Buffer resource over [base, base + bytes): a lane whose offset lies past
// `bytes` reads zeros and touches no memory.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
}

// 16 bytes per lane from base + voff + soff into LDS slot lds_dst + lane*16.
__device__ inline void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, unsigned char* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_byte*)lds_dst, 16, int(voff), int(soff), 0, 0);
}

// XCD-aware order of a 1-D grid: the hardware deals workgroups to the 8 XCDs
// round robin, so workgroup p runs on XCD p % 8.  Of the largest multiple of 8
// workgroups each XCD is given a contiguous run of logical tiles instead; the
// last grid % 8 keep their index.
__device__ inline int xcd_tile(int p, int grid) {
  const int full = grid & ~7;
  return p < full ? (p & 7) * (full >> 3) + (p >> 3) : p;
}

// Logical tile b of a tilesA x tilesB grid, taken in groups of `group` A tiles
// that walk every B tile: a run of consecutive b (one XCD's share) covers a
// rectangle of about group x (run / group) tiles, whose operand bands that
// XCD's L2 holds for all of them.
__device__ inline void grouped_tile(int b, int tilesA, int tilesB, int group, int& ta, int& tb) {
  const int per = group * tilesB;
  const int grp = b / per, rem = b - grp * per;
  const int ga = min(group, tilesA - grp * group);
  ta = grp * group + rem % ga;
  tb = rem / ga;
}

}  // namespace nm
