// Sparse GEMM Y = W_nm X on gfx950 sparse MFMA (v_smfmac_f32_16x16x64_{f16,bf16}).
//
// Product rule: "M:N sparsity on NVIDIA tensor cores" (COE-592 lecture 04-2),
// section "Where this sits among the three case studies": only the weight
// operand is compressed; its indices select which entries of the dense
// operand take part, so a 2:4 row does half the multiplies.  Permuted layer:
// SHUFFLESPARSE technical summary, section 2 and its inference-efficiency
// item -- y = (W Pi) x with Pi applied as a precomputed index map while the
// input is read.
//
// Operand layout of v_smfmac_f32_16x16x64 (measured on gfx950; lane l,
// q = l / 16, i = l % 16):
//   A (sparse, 8 halves): row i, groups 4q..4q+3 of the 64-wide K step, two
//     values per group; value j takes its in-group position from bits
//     [2j, 2j+2) of the lane's 16-bit index half (the immediate selects the
//     low or high half of the 32-bit index register).  This is exactly a
//     16-byte slice of a packed 2:4 row plus the matching 16 bits of its
//     LSB-first index bitstream.
//   B (dense, 16 halves): column i, K = 8q..8q+7 then 32+8q..32+8q+7.
//   D (4 floats): column i, rows 4q..4q+3.
// 1:4 and 1:8 rows are widened in registers to this 2:4 operand: a survivor
// at position p fills one slot of the 4-group that holds p, its partner slot
// gets value 0 with the same position, and 4-groups without a survivor get
// zeros.
//
// Tiling: a workgroup of 256 threads computes a BR x BT tile of Y^T
// (R rows x T tokens); waves are laid out WR x WT.  Each 64-wide K step the
// packed A slice (values + index bits) and the X slice (BT tokens x 64 K,
// gathered through perm when permuted) are staged into LDS, double buffered
// with register prefetch of the next step; each wave then issues
// (BR/WR/16) x (BT/WT/16) smfmac per step.  Accumulation is fp32.
#include "nm_device.h"
#include "nm_internal.h"

namespace nm {
namespace {

// Per-pattern constants for one 64-wide K step of one row.
//   VPS  packed values per step; VB bytes of values a lane takes per step
//   IBS  index bits per step
template <int P>
struct Pat;
template <>
struct Pat<0> {  // 2:4
  static constexpr int N = 2, M = 4, B = 2, VPS = 32, IBS = 64, VEC = 8;  // VEC: halves per load
};
template <>
struct Pat<1> {  // 1:4
  static constexpr int N = 1, M = 4, B = 2, VPS = 16, IBS = 32, VEC = 4;
};
template <>
struct Pat<2> {  // 1:8
  static constexpr int N = 1, M = 8, B = 3, VPS = 8, IBS = 24, VEC = 2;
};

// Widen one lane's slice of a step to the 2:4 smfmac operand.
//   raw: the lane's packed values (VEC halves, low bits first)
//   ib:  the lane's index bits (IBS/4 bits, survivor order)
template <int P>
__device__ inline void widen(const uint32_t* raw, uint32_t ib, u32x4& a, uint32_t& idx16) {
  if constexpr (P == 0) {
    a[0] = raw[0]; a[1] = raw[1]; a[2] = raw[2]; a[3] = raw[3];
    idx16 = ib & 0xFFFFu;
  } else if constexpr (P == 1) {
    // four survivors v0..v3 at 2-bit positions p0..p3: pair j = (v_j, 0), both
    // slots naming p_j.
    a[0] = raw[0] & 0xFFFFu; a[1] = raw[0] >> 16; a[2] = raw[1] & 0xFFFFu; a[3] = raw[1] >> 16;
    uint32_t t = (ib & 0x3u) | ((ib & 0xCu) << 2) | ((ib & 0x30u) << 4) | ((ib & 0xC0u) << 6);
    idx16 = t | (t << 2);
  } else {
    // two survivors, each at a 3-bit position inside a group of 8 that spans
    // two 4-groups: the half holding p gets (v, 0) naming p & 3, the other
    // half gets zeros.
    const uint32_t v0 = raw[0] & 0xFFFFu, v1 = raw[0] >> 16;
    const uint32_t p0 = ib & 7u, p1 = (ib >> 3) & 7u;
    const bool h0 = p0 >= 4, h1 = p1 >= 4;
    a[0] = h0 ? 0u : v0; a[1] = h0 ? v0 : 0u;
    a[2] = h1 ? 0u : v1; a[3] = h1 ? v1 : 0u;
    const uint32_t f0 = (p0 & 3u) * 5u, f1 = (p1 & 3u) * 5u;  // same position in both slots
    idx16 = (h0 ? (f0 << 4) : f0) | (h1 ? (f1 << 12) : (f1 << 8));
  }
}

template <int P, int DT, int OUT, bool PERM, int BR, int BT, int WR, int WT>
struct Cfg {
  using PT = Pat<P>;
  static constexpr int FR = BR / WR / 16;  // A fragments per wave
  static constexpr int FT = BT / WT / 16;  // B fragments per wave
  static_assert(WR * WT == 4, "four waves per workgroup");
  static_assert(FR >= 1 && FT >= 1, "wave tile at least 16 x 16");
  // LDS strides (bytes).  Padding keeps the 16 lanes that share q on distinct banks.
  static constexpr int AV_ROW = PT::VPS * 2;          // packed bytes per row per step
  static constexpr int AV_STRIDE = AV_ROW + 16;
  static constexpr int AI_STRIDE = 8;                 // index bits per row per step, as 64-bit slot
  static constexpr int B_STRIDE = 128 + 16;           // 64 halves + pad
  static constexpr int AV_BYTES = BR * AV_STRIDE;
  static constexpr int AI_BYTES = BR * AI_STRIDE;
  static constexpr int B_BYTES = BT * B_STRIDE;
  static constexpr int BUF_BYTES = AV_BYTES + AI_BYTES + B_BYTES;
  // global -> LDS chunking
  static constexpr int AV_CHUNKS = BR * (PT::VPS / PT::VEC);  // loads of VEC halves
  static constexpr int AV_PER_T = (AV_CHUNKS + 255) / 256;
  static constexpr int B_CHUNKS = BT * 8;                      // 16-byte chunks
  static constexpr int B_PER_T = (B_CHUNKS + 255) / 256;
  static constexpr int AI_PER_T = (BR + 255) / 256;
};

template <int P, int DT, int OUT, bool PERM, int BR, int BT, int WR, int WT>
__global__ __launch_bounds__(256) void spmm_kernel(const uint16_t* __restrict__ values,
                                                   const uint32_t* __restrict__ idx, int R, int K,
                                                   int64_t idx_row_words,
                                                   const uint16_t* __restrict__ act, int T,
                                                   int64_t ldx, const int32_t* __restrict__ perm,
                                                   void* __restrict__ Y, int64_t ldy, int tilesR,
                                                   int tilesT, int group_r) {
  using C = Cfg<P, DT, OUT, PERM, BR, BT, WR, WT>;
  using PT = typename C::PT;
  extern __shared__ __align__(16) unsigned char smem[];

  // ---- tile index: XCD-aware remap, then grouped order (group_r R-tiles share X)
  const int ntiles = tilesR * tilesT;
  int b = blockIdx.x;
  if ((ntiles & 7) == 0) b = (b & 7) * (ntiles >> 3) + (b >> 3);
  const int per_group = group_r * tilesT;
  const int grp = b / per_group;
  const int rem = b - grp * per_group;
  const int rows_in_grp = min(group_r, tilesR - grp * group_r);
  const int tr = grp * group_r + rem % rows_in_grp;
  const int tt = rem / rows_in_grp;
  const int R0 = tr * BR, T0 = tt * BT;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave / WT, wt = wave % WT;
  const int li = lane & 15, lq = lane >> 4;

  const int64_t S = int64_t(K) / PT::M * PT::N;
  const int nsteps = (K + 63) / 64;

  // ---- register staging for one step
  uint32_t av_reg[C::AV_PER_T][PT::VEC / 2];
  uint32_t ai_reg[C::AI_PER_T][2];
  u32x4 b_reg[C::B_PER_T];

  auto load_step = [&](int s) {
    const int k0 = s * 64;
    const int64_t v0 = int64_t(k0) / PT::M * PT::N;       // first packed value of the step
    const int vvalid = (min(K - k0, 64) / PT::M) * PT::N;  // packed values present this step
#pragma unroll
    for (int i = 0; i < C::AV_PER_T; ++i) {
      const int ch = tid + i * 256;
      const int row = ch / (PT::VPS / PT::VEC), c = ch % (PT::VPS / PT::VEC);
      const int gr = R0 + row;
#pragma unroll
      for (int e = 0; e < PT::VEC / 2; ++e) av_reg[i][e] = 0u;
      if (ch < C::AV_CHUNKS && gr < R && c * PT::VEC < vvalid) {
        const uint16_t* src = values + int64_t(gr) * S + v0 + c * PT::VEC;
        if constexpr (PT::VEC == 8) {
          const uint4 t = *reinterpret_cast<const uint4*>(src);
          av_reg[i][0] = t.x; av_reg[i][1] = t.y; av_reg[i][2] = t.z; av_reg[i][3] = t.w;
        } else if constexpr (PT::VEC == 4) {
          const uint2 t = *reinterpret_cast<const uint2*>(src);
          av_reg[i][0] = t.x; av_reg[i][1] = t.y;
        } else {
          av_reg[i][0] = *reinterpret_cast<const uint32_t*>(src);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < C::AI_PER_T; ++i) {
      const int row = tid + i * 256;
      const int gr = R0 + row;
      ai_reg[i][0] = 0u; ai_reg[i][1] = 0u;
      if (row < BR && gr < R) {
        const uint32_t* irow = idx + int64_t(gr) * idx_row_words;
        const int ibits = vvalid * PT::B;  // valid index bits this step
        const int64_t bit0 = int64_t(s) * PT::IBS;
        const int64_t w0 = bit0 >> 5;
        const int sh = int(bit0 & 31);
        if constexpr (P == 0) {
          ai_reg[i][0] = irow[w0];
          if (ibits > 32) ai_reg[i][1] = irow[w0 + 1];
        } else if constexpr (P == 1) {
          ai_reg[i][0] = irow[w0];
        } else {
          uint64_t both = irow[w0];
          if (sh + ibits > 32) both |= uint64_t(irow[w0 + 1]) << 32;
          ai_reg[i][0] = uint32_t(both >> sh) & ((ibits >= 32) ? 0xFFFFFFFFu : ((1u << ibits) - 1u));
        }
      }
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
      const int ch = tid + i * 256;
      const int row = ch >> 3, c = ch & 7;
      const int t = T0 + row;
      const int kk = k0 + c * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ch < C::B_CHUNKS && t < T && kk < K) {
        const uint16_t* arow = act + int64_t(t) * ldx;
        if constexpr (PERM) {
          // entries outside [0, K) (a broken precondition) are clamped into
          // the row: a wrong value, never a wrong address
          const uint32_t kmax = uint32_t(K - 1);
          const int4 p0 = *reinterpret_cast<const int4*>(perm + kk);
          const int4 p1 = *reinterpret_cast<const int4*>(perm + kk + 4);
          const uint32_t q[8] = {umin(uint32_t(p0.x), kmax), umin(uint32_t(p0.y), kmax),
                                 umin(uint32_t(p0.z), kmax), umin(uint32_t(p0.w), kmax),
                                 umin(uint32_t(p1.x), kmax), umin(uint32_t(p1.y), kmax),
                                 umin(uint32_t(p1.z), kmax), umin(uint32_t(p1.w), kmax)};
          v[0] = uint32_t(arow[q[0]]) | (uint32_t(arow[q[1]]) << 16);
          v[1] = uint32_t(arow[q[2]]) | (uint32_t(arow[q[3]]) << 16);
          v[2] = uint32_t(arow[q[4]]) | (uint32_t(arow[q[5]]) << 16);
          v[3] = uint32_t(arow[q[6]]) | (uint32_t(arow[q[7]]) << 16);
        } else {
          const uint4 t4 = *reinterpret_cast<const uint4*>(arow + kk);
          v[0] = t4.x; v[1] = t4.y; v[2] = t4.z; v[3] = t4.w;
        }
      }
      b_reg[i] = v;
    }
  };

  auto store_step = [&](int buf) {
    unsigned char* base = smem + buf * C::BUF_BYTES;
#pragma unroll
    for (int i = 0; i < C::AV_PER_T; ++i) {
      const int ch = tid + i * 256;
      if (ch < C::AV_CHUNKS) {
        const int row = ch / (PT::VPS / PT::VEC), c = ch % (PT::VPS / PT::VEC);
        unsigned char* d = base + row * C::AV_STRIDE + c * PT::VEC * 2;
        if constexpr (PT::VEC == 8) {
          *reinterpret_cast<uint4*>(d) = make_uint4(av_reg[i][0], av_reg[i][1], av_reg[i][2], av_reg[i][3]);
        } else if constexpr (PT::VEC == 4) {
          *reinterpret_cast<uint2*>(d) = make_uint2(av_reg[i][0], av_reg[i][1]);
        } else {
          *reinterpret_cast<uint32_t*>(d) = av_reg[i][0];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < C::AI_PER_T; ++i) {
      const int row = tid + i * 256;
      if (row < BR)
        *reinterpret_cast<uint2*>(base + C::AV_BYTES + row * C::AI_STRIDE) =
            make_uint2(ai_reg[i][0], ai_reg[i][1]);
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
      const int ch = tid + i * 256;
      if (ch < C::B_CHUNKS) {
        const int row = ch >> 3, c = ch & 7;
        *reinterpret_cast<u32x4*>(base + C::AV_BYTES + C::AI_BYTES + row * C::B_STRIDE + c * 16) = b_reg[i];
      }
    }
  };

  f32x4 acc[C::FR][C::FT];
#pragma unroll
  for (int i = 0; i < C::FR; ++i)
#pragma unroll
    for (int j = 0; j < C::FT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_step(0);
  store_step(0);
  __syncthreads();

  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) load_step(s + 1);
    const unsigned char* base = smem + buf * C::BUF_BYTES;
    // B fragments for this wave
    u32x8 bf[C::FT];
#pragma unroll
    for (int j = 0; j < C::FT; ++j) {
      const unsigned char* p = base + C::AV_BYTES + C::AI_BYTES +
                               (wt * (BT / WT) + j * 16 + li) * C::B_STRIDE + lq * 16;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(p + 64);
      bf[j] = u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int i = 0; i < C::FR; ++i) {
      const int row = wr * (BR / WR) + i * 16 + li;
      const unsigned char* pa = base + row * C::AV_STRIDE + lq * (PT::VEC * 2);
      uint32_t raw[4] = {0u, 0u, 0u, 0u};
      if constexpr (PT::VEC == 8) {
        const u32x4 t = *reinterpret_cast<const u32x4*>(pa);
        raw[0] = t[0]; raw[1] = t[1]; raw[2] = t[2]; raw[3] = t[3];
      } else if constexpr (PT::VEC == 4) {
        const uint2 t = *reinterpret_cast<const uint2*>(pa);
        raw[0] = t.x; raw[1] = t.y;
      } else {
        raw[0] = *reinterpret_cast<const uint32_t*>(pa);
      }
      const uint64_t ibrow = *reinterpret_cast<const uint64_t*>(base + C::AV_BYTES + row * C::AI_STRIDE);
      const uint32_t ib = uint32_t(ibrow >> (lq * (PT::IBS / 4)));
      u32x4 a;
      uint32_t idx16;
      widen<P>(raw, ib, a, idx16);
#pragma unroll
      for (int j = 0; j < C::FT; ++j) acc[i][j] = smfmac<DT>(a, bf[j], acc[i][j], idx16);
    }
    if (s + 1 < nsteps) store_step(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds Y^T[t][r .. r+3] for each fragment
  const bool vec_ok = (ldy & 3) == 0;  // 4-element row pieces stay aligned
#pragma unroll
  for (int i = 0; i < C::FR; ++i) {
    const int r = R0 + wr * (BR / WR) + i * 16 + lq * 4;
#pragma unroll
    for (int j = 0; j < C::FT; ++j) {
      const int t = T0 + wt * (BT / WT) + j * 16 + li;
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

template <int P, int DT, int OUT, bool PERM, int BR, int BT, int WR, int WT>
hipError_t launch_cfg(const SpmmArgs& a, hipStream_t s) {
  using C = Cfg<P, DT, OUT, PERM, BR, BT, WR, WT>;
  const int tilesR = int((a.R + BR - 1) / BR);
  const int tilesT = int((a.T + BT - 1) / BT);
  const int64_t ntiles = int64_t(tilesR) * tilesT;
  if (ntiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int group_r = tilesR < 4 ? tilesR : 4;
  const size_t lds = 2 * C::BUF_BYTES;
  auto kern = spmm_kernel<P, DT, OUT, PERM, BR, BT, WR, WT>;
  if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), int(lds)); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(unsigned(ntiles)), dim3(256), lds, s, a.values, a.idx, int(a.R),
                     int(a.K), a.idx_row_words, a.act, int(a.T), a.ldx, a.perm, a.Y, a.ldy, tilesR,
                     tilesT, group_r);
  return hipGetLastError();
}

template <int P, int DT, int OUT, bool PERM>
hipError_t pick_tile(const SpmmArgs& a, hipStream_t s) {
  if (a.T >= 128 && a.R >= 256) return launch_cfg<P, DT, OUT, PERM, 256, 128, 2, 2>(a, s);
  if (a.T >= 64) return launch_cfg<P, DT, OUT, PERM, 128, 64, 2, 2>(a, s);
  return launch_cfg<P, DT, OUT, PERM, 64, 16, 4, 1>(a, s);
}

template <int P, int DT>
hipError_t pick_out(const SpmmArgs& a, hipStream_t s) {
  const bool perm = a.perm != nullptr;
  if (a.out_dtype == NM_F32) {
    return perm ? pick_tile<P, DT, NM_F32, true>(a, s) : pick_tile<P, DT, NM_F32, false>(a, s);
  }
  return perm ? pick_tile<P, DT, DT, true>(a, s) : pick_tile<P, DT, DT, false>(a, s);
}

template <int P>
hipError_t pick_dtype(const SpmmArgs& a, hipStream_t s) {
  return a.dtype == NM_F16 ? pick_out<P, NM_F16>(a, s) : pick_out<P, NM_BF16>(a, s);
}

}  // namespace

hipError_t launch_generic(const SpmmArgs& a, hipStream_t s) {
  if (a.n == 2 && a.m == 4) return pick_dtype<0>(a, s);
  if (a.n == 1 && a.m == 4) return pick_dtype<1>(a, s);
  if (a.n == 1 && a.m == 8) return pick_dtype<2>(a, s);
  return hipErrorInvalidValue;
}

// Kernel choice.  variant 0 picks by shape; 1..6 force one kernel family when
// the shape allows it (ablations, tests), else fall back to the choice by
// shape.  The permuted product with a large enough workspace gathers
// X' = act[:, perm] into it once and multiplies X'; without one, the map is
// applied while the kernel reads its input: in the few-token kernel
// (T <= 16), the resident-tile kernel (2:4, K % 256 == 0, K <= 4096) or the
// generic one.
hipError_t launch_spmm(const SpmmArgs& a, hipStream_t s) {
  if (a.dtype == NM_I8 || a.dtype == NM_FP8) return launch_spmm_i8(a, s);  // 8-bit weights
  if (a.perm != nullptr && a.workspace != nullptr) {
    const size_t need = spmm_perm_gather_bytes(a.T, a.K, a.dtype);
    if (need > 0 && a.workspace_bytes >= need) return launch_spmm_perm_gather(a, a.workspace, s);
  }
  switch (a.variant) {
    case NM_VARIANT_GENERIC: return launch_generic(a, s);
    case NM_VARIANT_PIPE:
      if (spmm_pipe_applies(a)) return launch_spmm_pipe(a, s);
      break;
    case NM_VARIANT_LDS:
      if (spmm_lds_applies(a)) return launch_spmm_lds(a, s);
      break;
    case NM_VARIANT_DECODE:
      if (spmm_decode_applies(a)) return launch_spmm_decode(a, s);
      break;
    case NM_VARIANT_RESIDENT:
      if (spmm_resident_applies(a)) return launch_spmm_resident(a, s);
      break;
    case NM_VARIANT_LDS_NM:
      if (spmm_lds_nm_applies(a)) return launch_spmm_lds_nm(a, s);
      break;
    default: break;
  }
  if (spmm_decode_applies(a)) return launch_spmm_decode(a, s);
  if (a.perm != nullptr) {
    if (spmm_resident_applies(a)) return launch_spmm_resident(a, s);
    return launch_generic(a, s);
  }
  if (spmm_lds_applies(a)) return launch_spmm_lds(a, s);
  if (spmm_lds_nm_applies(a)) return launch_spmm_lds_nm(a, s);
  if (spmm_pipe_applies(a)) return launch_spmm_pipe(a, s);
  return launch_generic(a, s);
}

}  // namespace nm
