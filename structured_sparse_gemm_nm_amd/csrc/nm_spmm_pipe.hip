// Pipelined sparse GEMM for large tiles (prefill shapes) on gfx950.
//
// Same product as nm_spmm.hip (Y^T[t, r] = sum_k W_nm[r, k] act[t, k], on
// v_smfmac_f32_16x16x64), organised to keep several K steps of loads in flight:
//
//   * a workgroup (4 waves) owns a 256 x BT tile of Y^T; wave w owns rows
//     [64w, 64w + 64) and all BT tokens, so its packed-A fragments are private
//     and go straight from global memory into registers in the operand layout
//     the instruction wants (16 bytes of values + 16 index bits per lane for
//     2:4), NS - 1 steps ahead of use;
//   * the activation tile (BT tokens x 64 K per step) is shared by the four
//     waves through an NS-stage LDS ring filled with direct global->LDS loads;
//     slot (token, 16-byte chunk c) sits at token*8 + (c ^ (token & 7)) so the
//     fragment reads of 8 consecutive tokens hit distinct banks;
//   * one barrier per step: it both publishes stage s and retires stage s - 1,
//     whose slot the step's new loads then reuse.
// The permuted product is not handled here (it gathers X through the index
// map); shapes with K % 64 != 0 fall back as well.
#include "nm_device.h"
#include "nm_internal.h"

namespace nm {
namespace {

constexpr int pat_n(int P) { return P == 0 ? 2 : 1; }
constexpr int pat_m(int P) { return P == 2 ? 8 : 4; }

// One lane's share of one 16-row A fragment for one K step.
struct AFrag {
  uint32_t v[4];  // packed values (pattern-dependent count used)
  uint32_t ib;    // index bits of this lane's slice
};

// Issue the loads of lane (row, lq) for step s.  Every lane issues them (rows
// past R reread row R - 1 and their outputs are dropped), so each wave issues
// exactly ALOADS_PER_FRAG loads per fragment: the counted waits rely on it.
template <int P>
__device__ inline void load_afrag(AFrag& f, const uint16_t* __restrict__ values,
                                  const uint32_t* __restrict__ idx, int64_t S, int64_t words, int row,
                                  int R, int s, int lq) {
  row = min(row, R - 1);
  const uint16_t* vrow = values + int64_t(row) * S;
  const unsigned char* irow = reinterpret_cast<const unsigned char*>(idx + int64_t(row) * words);
  if constexpr (P == 0) {  // 2:4: 8 values (16 B), 16 index bits
    const uint4 t = *reinterpret_cast<const uint4*>(vrow + s * 32 + lq * 8);
    f.v[0] = t.x; f.v[1] = t.y; f.v[2] = t.z; f.v[3] = t.w;
    f.ib = *reinterpret_cast<const uint16_t*>(irow + s * 8 + lq * 2);
  } else if constexpr (P == 1) {  // 1:4: 4 values (8 B), 8 index bits
    const uint2 t = *reinterpret_cast<const uint2*>(vrow + s * 16 + lq * 4);
    f.v[0] = t.x; f.v[1] = t.y; f.v[2] = 0u; f.v[3] = 0u;
    f.ib = irow[s * 4 + lq];
  } else {  // 1:8: 2 values (4 B), 6 index bits at bit 24 s + 6 lq of the row
    f.v[0] = *reinterpret_cast<const uint32_t*>(vrow + s * 8 + lq * 2);
    f.v[3] = 0u;
    // the aligned word holding the first bit and the next one (clamped to the
    // row's last word, whose bits then suffice): two loads from every lane,
    // kept as loaded (widen extracts the bits, so nothing here waits for them)
    const uint32_t* wrow = idx + int64_t(row) * words;
    const int bit = 24 * s + 6 * lq;
    const int w0 = bit >> 5;
    const int w1 = min(w0 + 1, int(words) - 1);
    f.v[1] = wrow[w0];
    f.v[2] = wrow[w1];
    f.ib = uint32_t(bit & 31);
  }
}

// Loads each wave issues per A fragment per step (see load_afrag).
constexpr int aloads_per_frag(int P) { return P == 2 ? 3 : 2; }

// Widen to the 2:4 smfmac operand (see nm_spmm.hip for the 1:4 / 1:8 rules).
template <int P>
__device__ inline void widen(const AFrag& f, u32x4& a, uint32_t& idx16) {
  if constexpr (P == 0) {
    a[0] = f.v[0]; a[1] = f.v[1]; a[2] = f.v[2]; a[3] = f.v[3];
    idx16 = f.ib;
  } else if constexpr (P == 1) {
    a[0] = f.v[0] & 0xFFFFu; a[1] = f.v[0] >> 16; a[2] = f.v[1] & 0xFFFFu; a[3] = f.v[1] >> 16;
    const uint32_t ib = f.ib;
    const uint32_t t = (ib & 0x3u) | ((ib & 0xCu) << 2) | ((ib & 0x30u) << 4) | ((ib & 0xC0u) << 6);
    idx16 = t | (t << 2);
  } else {
    const uint32_t v0 = f.v[0] & 0xFFFFu, v1 = f.v[0] >> 16;
    const uint32_t ib = uint32_t((uint64_t(f.v[1]) | (uint64_t(f.v[2]) << 32)) >> f.ib);
    const uint32_t p0 = ib & 7u, p1 = (ib >> 3) & 7u;
    const bool h0 = p0 >= 4, h1 = p1 >= 4;
    a[0] = h0 ? 0u : v0; a[1] = h0 ? v0 : 0u;
    a[2] = h1 ? 0u : v1; a[3] = h1 ? v1 : 0u;
    const uint32_t f0 = (p0 & 3u) * 5u, f1 = (p1 & 3u) * 5u;
    idx16 = (h0 ? (f0 << 4) : f0) | (h1 ? (f1 << 12) : (f1 << 8));
  }
}

template <int P, int DT, int OUT, int BR, int BT, int NS>
__global__ __launch_bounds__(256) void spmm_pipe_kernel(
    const uint16_t* __restrict__ values, const uint32_t* __restrict__ idx, int R, int K,
    int64_t words, const uint16_t* __restrict__ act, int T, int64_t ldx, void* __restrict__ Y,
    int64_t ldy, int tilesR, int tilesT, int group_r) {
  constexpr int WROWS = BR / 4;         // rows per wave
  constexpr int FR = WROWS / 16;        // 16-row fragments per wave
  constexpr int FT = BT / 16;           // 16-token fragments
  constexpr int STAGE = BT * 128;       // bytes of one activation stage (BT x 64 halves)
  constexpr int BLOADS = BT / 32;       // 16-byte direct loads per thread per stage
  constexpr int ALOADS = FR * aloads_per_frag(P);  // A loads per wave per step
  constexpr int PER_STEP = BLOADS + ALOADS;
  static_assert(NS >= 2, "at least double buffering");
  static_assert((NS - 2) * (BT / 32 + (BR / 64) * aloads_per_frag(P)) < 64, "vmcnt range");
  __shared__ __align__(16) unsigned char smem[NS * STAGE];

  // ---- tile: XCD-aware remap, then groups of group_r row tiles
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
  const int li = lane & 15, lq = lane >> 4;
  const int64_t S = int64_t(K) / pat_m(P) * pat_n(P);
  const int nsteps = K >> 6;

  // activation slots this thread fills each stage: instruction j covers slots
  // [(wave*BLOADS + j)*64, +64), lane l takes slot base + l
  const uint16_t* bsrc[BLOADS];
#pragma unroll
  for (int j = 0; j < BLOADS; ++j) {
    const int slot = (wave * BLOADS + j) * 64 + lane;
    const int tok = slot >> 3;
    const int chunk = (slot & 7) ^ (tok & 7);
    const int t = min(T0 + tok, T - 1);  // rows past T read a valid row; their outputs are dropped
    bsrc[j] = act + int64_t(t) * ldx + chunk * 8;
  }

  auto issue_b = [&](int s, int stage) {
#pragma unroll
    for (int j = 0; j < BLOADS; ++j) {
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(bsrc[j] + s * 64),
          (lds_byte*)(smem + stage * STAGE + (wave * BLOADS + j) * 1024), 16, 0, 0);
    }
  };

  AFrag ar[NS][FR];
  const int row0 = R0 + wave * WROWS + li;
  auto issue_a = [&](int s, AFrag* dst) {
#pragma unroll
    for (int i = 0; i < FR; ++i) load_afrag<P>(dst[i], values, idx, S, words, row0 + i * 16, R, s, lq);
  };

  f32x4 acc[FR][FT];
#pragma unroll
  for (int i = 0; i < FR; ++i)
#pragma unroll
    for (int j = 0; j < FT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- prologue: steps 0 .. NS-2 in flight
#pragma unroll
  for (int p = 0; p < NS - 1; ++p) {
    if (p < nsteps) {
      issue_b(p, p);
      issue_a(p, ar[p]);
    }
  }

  for (int s0 = 0; s0 < nsteps; s0 += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int s = s0 + u;
      if (s < nsteps) {
        // step s's loads are done once at most the later steps' loads remain
        if (s + NS - 2 < nsteps) wait_vmcnt<(NS - 2) * PER_STEP>();
        else wait_vmcnt<0>();
        barrier_no_fence();
        if (s + NS - 1 < nsteps) {
          issue_b(s + NS - 1, (u + NS - 1) % NS);
          issue_a(s + NS - 1, ar[(u + NS - 1) % NS]);
        }
        const unsigned char* st = smem + u * STAGE;
        u32x4 a[FR];
        uint32_t ix[FR];
#pragma unroll
        for (int i = 0; i < FR; ++i) widen<P>(ar[u][i], a[i], ix[i]);
        u32x8 bf[FT];
#pragma unroll
        for (int j = 0; j < FT; ++j) {
          const int tok = j * 16 + li;
          const int sw = tok & 7;
          const u32x4 lo = *reinterpret_cast<const u32x4*>(st + (tok * 8 + (lq ^ sw)) * 16);
          const u32x4 hi = *reinterpret_cast<const u32x4*>(st + (tok * 8 + ((lq + 4) ^ sw)) * 16);
          bf[j] = u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int j = 0; j < FT; ++j)
#pragma unroll
          for (int i = 0; i < FR; ++i) acc[i][j] = smfmac<DT>(a[i], bf[j], acc[i][j], ix[i]);
        // Schedule: the first half of the step's LDS fragment reads, the
        // prefetch loads, two MFMAs, the second half of the reads (hidden
        // behind the first half's MFMAs), then the remaining MFMAs.  Halves
        // keep the outstanding LDS count within the 4-bit counter, so each
        // MFMA waits only for its own fragment.
        __builtin_amdgcn_sched_group_barrier(0x100, FT, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, PER_STEP, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, FT, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, FR * FT - 2, 0);
      }
    }
  }

  // ---- epilogue
  const bool vec_ok = (ldy & 3) == 0;
#pragma unroll
  for (int i = 0; i < FR; ++i) {
    const int r = R0 + wave * WROWS + i * 16 + lq * 4;
#pragma unroll
    for (int j = 0; j < FT; ++j) {
      const int t = T0 + j * 16 + li;
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

template <int P, int DT, int OUT, int BR, int BT, int NS>
hipError_t launch_pipe(const SpmmArgs& a, hipStream_t s) {
  const int tilesR = int((a.R + BR - 1) / BR);
  const int tilesT = int((a.T + BT - 1) / BT);
  const int64_t ntiles = int64_t(tilesR) * tilesT;
  if (ntiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int group_r = tilesR < 4 ? tilesR : 4;
  hipLaunchKernelGGL((spmm_pipe_kernel<P, DT, OUT, BR, BT, NS>), dim3(unsigned(ntiles)), dim3(256), 0, s,
                     a.values, a.idx, int(a.R), int(a.K), a.idx_row_words, a.act, int(a.T), a.ldx,
                     a.Y, a.ldy, tilesR, tilesT, group_r);
  return hipGetLastError();
}

template <int P, int DT, int OUT>
hipError_t pipe_tile(const SpmmArgs& a, hipStream_t s) {
  // 256 x 128 tiles when they cover the chip's 256 CUs, else 128 x 64
  const int64_t big = ((a.R + 255) / 256) * ((a.T + 127) / 128);
  if (big >= 256) return launch_pipe<P, DT, OUT, 256, 128, 4>(a, s);
  // small tiles do little MFMA work per step: keep 7 steps of loads in flight
  return launch_pipe<P, DT, OUT, 128, 64, 8>(a, s);
}

template <int P, int DT>
hipError_t pipe_out(const SpmmArgs& a, hipStream_t s) {
  return a.out_dtype == NM_F32 ? pipe_tile<P, DT, NM_F32>(a, s) : pipe_tile<P, DT, DT>(a, s);
}

template <int P>
hipError_t pipe_dtype(const SpmmArgs& a, hipStream_t s) {
  return a.dtype == NM_F16 ? pipe_out<P, NM_F16>(a, s) : pipe_out<P, NM_BF16>(a, s);
}

}  // namespace

bool spmm_pipe_applies(const SpmmArgs& a) {
  return a.perm == nullptr && (a.K % 64) == 0 && a.T >= 64 && a.R >= 128;
}

hipError_t launch_spmm_pipe(const SpmmArgs& a, hipStream_t s) {
  if (a.n == 2 && a.m == 4) return pipe_dtype<0>(a, s);
  if (a.n == 1 && a.m == 4) return pipe_dtype<1>(a, s);
  if (a.n == 1 && a.m == 8) return pipe_dtype<2>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace nm
