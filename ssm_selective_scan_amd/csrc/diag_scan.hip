// diag_scan.hip — diagonal recurrence h_t = a_t h_{t-1} + b_t (one launch).
//
// ("mlx-recurrence" post, rglru_scan with state [B, D]; IBM Research blog
// "K-Search for MLX", section "A 20x faster prefill: the Mamba SSM kernel":
// recurrence, associative combine and the O(log N)-depth parallel scan.)
//
// One workgroup owns 16 channel groups of one batch row (a group is CPL = 1,
// 2 or 4 adjacent channels, read and written as one vector) and walks the
// sequence in tiles of 512 steps.  Inside a tile the 1024 threads split time:
// lane = 16 * (segment within wave) + group, so each of the 64 time segments
// of 8 steps is scanned sequentially in registers (a 16-lane row reads 64,
// 128 or 256 contiguous bytes of a token).  The 64 segment aggregates of each
// channel are then combined by one wave with a DPP (a, b)-pair scan, the
// carry entering the tile is folded in, and every lane finishes its segment.
// The carry between tiles lives in LDS, so any L runs in the same launch.
// CPL = 1 keeps more workgroups for small problems; wider groups are used
// once they still fill the chip.
#include "common.hpp"
#include "launch.hpp"

namespace lr {

constexpr int kDiagCT = 16;          // channels per workgroup
constexpr int kDiagSeg = 8;          // steps per lane segment
constexpr int kDiagThreads = 1024;   // 16 waves, 4 segments per wave
constexpr int kDiagSegs = kDiagThreads / kDiagCT;  // 64 segments per tile
constexpr int kDiagTile = kDiagSegs * kDiagSeg;    // 512 steps per tile
// narrow tiles (few chains): channels and threads per workgroup
constexpr int kDiagNarrowCT = 8, kDiagNarrowNT = 512;

// CPL consecutive channels per lane, read and written as one CPL-wide vector
// access (a 16-lane row of a wave then covers 16 * CPL channels of a token).
template <typename T, int CPL>
__device__ __forceinline__ void vstore(T* p, const float (&v)[CPL]) {
  if constexpr (CPL == 1) {
    Io<T>::store(p, v[0]);
  } else if constexpr (sizeof(T) == 4) {
    if constexpr (CPL == 2) *reinterpret_cast<float2*>(p) = float2{v[0], v[1]};
    else *reinterpret_cast<float4*>(p) = float4{v[0], v[1], v[2], v[3]};
  } else {
    if constexpr (CPL == 2) {
      *reinterpret_cast<uint32_t*>(p) = f2bf(v[0]) | (static_cast<uint32_t>(f2bf(v[1])) << 16);
    } else {
      *reinterpret_cast<uint2*>(p) =
          uint2{f2bf(v[0]) | (static_cast<uint32_t>(f2bf(v[1])) << 16),
                f2bf(v[2]) | (static_cast<uint32_t>(f2bf(v[3])) << 16)};
    }
  }
}

// CPL = 1: 16 channels per workgroup (small problems: more workgroups);
// CPL = 2, 4: 32 or 64 channels per workgroup with 8- or 16-byte accesses
// (large problems, where the 64-byte row pieces of CPL = 1 cost bandwidth).
// Vector widths need D % CPL == 0.
template <typename T, int CPL>
__global__ __launch_bounds__(kDiagThreads) void diag_scan_kernel(
    const T* __restrict__ a, const T* __restrict__ b, const float* __restrict__ h0,
    T* __restrict__ h, float* __restrict__ h_last, int64_t L, int64_t D) {
  constexpr int CT = kDiagCT * CPL;   // channels per workgroup
  __shared__ float aggA[kDiagSegs][CT];
  __shared__ float aggB[kDiagSegs][CT];
  __shared__ float carry_in[kDiagSegs][CT];
  __shared__ float tile_carry[CT];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int ch = (lane & (kDiagCT - 1)) * CPL;   // first of this lane's CPL channels
  const int seg = wave * 4 + (lane >> 4);
  const int64_t ntile = (D + CT - 1) / CT;
  const int64_t bi = blockIdx.x / ntile;
  const int64_t d0 = (blockIdx.x % ntile) * CT;
  const int64_t d = d0 + ch;
  const bool dok = d < D;   // D % CPL == 0: all CPL channels exist

  for (int c = tid; c < CT; c += kDiagThreads) {
    const int64_t dd = d0 + c;
    tile_carry[c] = (h0 != nullptr && dd < D) ? h0[bi * D + dd] : 0.f;
  }
  __syncthreads();

  const int64_t row = bi * L;  // token offset of this batch row
  for (int64_t t0 = 0; t0 < L; t0 += kDiagTile) {
    const int64_t ts = t0 + static_cast<int64_t>(seg) * kDiagSeg;
    const int nok = dok ? static_cast<int>(L - ts < kDiagSeg ? (L - ts > 0 ? L - ts : 0) : kDiagSeg) : 0;
    float av[kDiagSeg][CPL], bv[kDiagSeg][CPL];
    {
      const int64_t off0 = (row + ts) * D + d;
      const T* pa = a + off0;
      const T* pb = b + off0;
      if constexpr (sizeof(T) == 2) {
        // bf16: every load of the segment issued raw before any is converted
        VRaw<T, CPL> ar[kDiagSeg], br[kDiagSeg];
#pragma unroll
        for (int i = 0; i < kDiagSeg; ++i) {
          ar[i] = i < nok ? vload_raw<T, CPL>(pa) : vfill_raw<T, CPL>(1.f);
          br[i] = i < nok ? vload_raw<T, CPL>(pb) : vfill_raw<T, CPL>(0.f);
          pa += D;
          pb += D;
        }
#pragma unroll
        for (int i = 0; i < kDiagSeg; ++i) {
          vcvt<T, CPL>(ar[i], av[i]);
          vcvt<T, CPL>(br[i], bv[i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < kDiagSeg; ++i) {
          if (i < nok) {
            vcvt<T, CPL>(vload_raw<T, CPL>(pa), av[i]);
            vcvt<T, CPL>(vload_raw<T, CPL>(pb), bv[i]);
          } else {
#pragma unroll
            for (int k = 0; k < CPL; ++k) { av[i][k] = 1.f; bv[i][k] = 0.f; }
          }
          pa += D;
          pb += D;
        }
      }
    }
    // sequential scan of the segment from a zero state
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      float P = 1.f, Hs = 0.f;
#pragma unroll
      for (int i = 0; i < kDiagSeg; ++i) {
        Hs = fmaf(av[i][k], Hs, bv[i][k]);
        P *= av[i][k];
        av[i][k] = P;   // running product  a_i ... a_first
        bv[i][k] = Hs;  // running state from zero
      }
      aggA[seg][ch + k] = P;
      aggB[seg][ch + k] = Hs;
    }
    __syncthreads();

    // one wave per channel (CPL channels per wave): lane = segment index
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const int c = wave + kDiagCT * k;
      float pa = aggA[lane][c], pb = aggB[lane][c];
      const float tc = tile_carry[c];
      wave_incl_pair_scan(pa, pb);
      // exclusive prefix: the pair of the previous lane (identity at lane 0)
      const float ea = wave_shr1(pa, 1.f), eb = wave_shr1(pb, 0.f);
      carry_in[lane][c] = fmaf(ea, tc, eb);
      if (lane == 63) tile_carry[c] = fmaf(pa, tc, pb);
    }
    __syncthreads();

    float cin[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) cin[k] = carry_in[seg][ch + k];
    {
      // offset formed after the barrier (see the backward kernel)
      int64_t offs = (row + ts) * D + d;
      asm volatile("" : "+v"(offs));
      T* ph = h + offs;
#pragma unroll
      for (int i = 0; i < kDiagSeg; ++i) {
        if (i < nok) {
          float o[CPL];
#pragma unroll
          for (int k = 0; k < CPL; ++k) o[k] = fmaf(av[i][k], cin[k], bv[i][k]);
          vstore<T, CPL>(ph, o);
        }
        ph += D;
      }
    }
  }
  __syncthreads();
  if (h_last != nullptr) {
    for (int c = tid; c < CT; c += kDiagThreads) {
      const int64_t dd = d0 + c;
      if (dd < D) h_last[bi * D + dd] = tile_carry[c];
    }
  }
}

// ---------------------------------------------------------------------------
// Narrow tiles for problems with few chains (B * D small): CT = 2, 4 or 8
// channels per workgroup instead of 16, so the grid has 2-8x more
// workgroups, and 1024-step tiles (NT threads: NSEG = NT / CT lane segments
// of SEG = 1024 / NSEG steps), so a sequence of up to 1024 tokens is one
// pass of one load, two barriers and one store.  Lane = CT * segment + channel: the CT
// channels of a token are adjacent lanes.  The segments of channel c are
// joined by wave c: lane l folds its NSEG / 64 consecutive segments, then the
// 64 lane totals go through the DPP (a, b)-pair scan.
// ---------------------------------------------------------------------------
template <typename T, int CT, int NT>
__global__ __launch_bounds__(NT) void diag_scan_narrow_kernel(
    const T* __restrict__ a, const T* __restrict__ b, const float* __restrict__ h0,
    T* __restrict__ h, float* __restrict__ h_last, int64_t L, int64_t D) {
  constexpr int NSEG = NT / CT;             // lane segments per tile
  constexpr int SEG = 1024 / NSEG;          // steps per lane segment
  constexpr int TL = NSEG * SEG;            // 1024 steps per tile
  constexpr int SPL = NSEG / 64;            // segments per lane in the join
  static_assert(CT >= 2 && CT <= 8 && TL == 1024 && SPL >= 1 && CT <= NT / 64, "narrow tile shape");
  __shared__ float aggA[NSEG][CT];
  __shared__ float aggB[NSEG][CT];
  __shared__ float carry_in[NSEG][CT];
  __shared__ float tile_carry[CT];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int ch = tid % CT;
  const int seg = tid / CT;
  const int64_t ntile = (D + CT - 1) / CT;
  // consecutive tiles (channels sharing cache lines) on one XCD
  const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t bi = wid / ntile;
  const int64_t d0 = (wid % ntile) * CT;
  const int64_t d = d0 + ch;
  const bool dok = d < D;

  if (tid < CT) tile_carry[tid] = (h0 != nullptr && d0 + tid < D) ? h0[bi * D + d0 + tid] : 0.f;
  __syncthreads();

  const int64_t row = bi * L;
  for (int64_t t0 = 0; t0 < L; t0 += TL) {
    const int64_t ts = t0 + static_cast<int64_t>(seg) * SEG;
    const int nok = dok ? static_cast<int>(L - ts < SEG ? (L - ts > 0 ? L - ts : 0) : SEG) : 0;
    float av[SEG], bv[SEG];
    {
      const int64_t off0 = (row + ts) * D + d;
#pragma unroll
      for (int i = 0; i < SEG; ++i) {
        av[i] = i < nok ? Io<T>::load(a + off0 + i * D) : 1.f;
        bv[i] = i < nok ? Io<T>::load(b + off0 + i * D) : 0.f;
      }
    }
    float P = 1.f, Hs = 0.f;
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
      Hs = fmaf(av[i], Hs, bv[i]);
      P *= av[i];
      av[i] = P;    // product of the segment's decays up to step i
      bv[i] = Hs;   // state at step i from a zero start
    }
    aggA[seg][ch] = P;
    aggB[seg][ch] = Hs;
    __syncthreads();

    if (wave < CT) {
      const int c = wave;
      float pa[SPL], pb[SPL];
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        pa[j] = aggA[SPL * lane + j][c];
        pb[j] = aggB[SPL * lane + j][c];
      }
      // the lane's segments folded in order, then the scan across lanes
      float ta = pa[0], tb = pb[0];
#pragma unroll
      for (int j = 1; j < SPL; ++j) {
        tb = fmaf(pa[j], tb, pb[j]);
        ta *= pa[j];
      }
      float ia = ta, ib = tb;
      wave_incl_pair_scan(ia, ib);
      const float tc = tile_carry[c];
      // state entering the lane's first segment, then each following one
      float cin = fmaf(wave_shr1(ia, 1.f), tc, wave_shr1(ib, 0.f));
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        carry_in[SPL * lane + j][c] = cin;
        cin = fmaf(pa[j], cin, pb[j]);
      }
      if (lane == 63) tile_carry[c] = fmaf(ia, tc, ib);
    }
    __syncthreads();

    const float cin = carry_in[seg][ch];
    int64_t offs = (row + ts) * D + d;
    asm volatile("" : "+v"(offs));
#pragma unroll
    for (int i = 0; i < SEG; ++i)
      if (i < nok) Io<T>::store(h + offs + i * D, fmaf(av[i], cin, bv[i]));
  }
  __syncthreads();
  if (h_last != nullptr && tid < CT && d0 + tid < D) h_last[bi * D + d0 + tid] = tile_carry[tid];
}

// ---------------------------------------------------------------------------
// Backward.  For the loss sum_t <dh_t, h_t> + <dh_last, h_{L-1}> the adjoint
// g_t = dl/dh_t obeys the same recurrence run backwards in time,
//     g_{L-1} = dh_{L-1} + dh_last,   g_t = a_{t+1} g_{t+1} + dh_t,
// so with u = L-1-t it is a forward diagonal scan G_u = al_u G_{u-1} + dh_t
// with al_0 = 1, al_u = a_{t+1} and initial state dh_last.  The gradients
// follow per step: db_t = g_t, da_t = g_t h_{t-1} (h_{-1} = h0), and
// dh0 = a_0 g_0.  Same work split as the forward kernel, with u in place of t.
template <typename T, int CPL>
__global__ __launch_bounds__(kDiagThreads) void diag_scan_bwd_kernel(
    const T* __restrict__ a, const T* __restrict__ h, const float* __restrict__ h0,
    const T* __restrict__ dh, const float* __restrict__ dh_last, T* __restrict__ da,
    T* __restrict__ db, float* __restrict__ dh0, int64_t L, int64_t D) {
  constexpr int CT = kDiagCT * CPL;   // channels per workgroup
  __shared__ float aggA[kDiagSegs][CT];
  __shared__ float aggB[kDiagSegs][CT];
  __shared__ float carry_in[kDiagSegs][CT];
  __shared__ float tile_carry[CT];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int ch = (lane & (kDiagCT - 1)) * CPL;
  const int seg = wave * 4 + (lane >> 4);
  const int64_t ntile = (D + CT - 1) / CT;
  const int64_t bi = blockIdx.x / ntile;
  const int64_t d0 = (blockIdx.x % ntile) * CT;
  const int64_t d = d0 + ch;
  const bool dok = d < D;

  for (int c = tid; c < CT; c += kDiagThreads) {
    const int64_t dd = d0 + c;
    tile_carry[c] = (dh_last != nullptr && dd < D) ? dh_last[bi * D + dd] : 0.f;
  }
  __syncthreads();

  const int64_t row = bi * L;  // token offset of this batch row
  for (int64_t u0 = 0; u0 < L; u0 += kDiagTile) {
    const int64_t us = u0 + static_cast<int64_t>(seg) * kDiagSeg;
    // steps u = us + i, i.e. tokens t = L - 1 - us - i (descending)
    const int nok = dok ? static_cast<int>(L - us < kDiagSeg ? (L - us > 0 ? L - us : 0) : kDiagSeg) : 0;
    const int64_t t_first = L - 1 - us;
    // at CPL = 2 (and fp32 CPL = 1) all loads of the segment, and after the
    // barriers all of the states, are issued raw before any is converted,
    // which measured faster there; at CPL = 4 the registers for that are not
    // there (it spills), and each step converts its own
    constexpr bool kPre = CPL == 2 || (CPL == 1 && sizeof(T) == 4);
    float av[kDiagSeg][CPL], bv[kDiagSeg][CPL];
    if constexpr (kPre) {
      VRaw<T, CPL> ar[kDiagSeg], br[kDiagSeg];
#pragma unroll
      for (int i = 0; i < kDiagSeg; ++i) {
        const int64_t t = t_first - i;
        const bool ok = i < nok;
        ar[i] = (ok && t + 1 < L) ? vload_raw<T, CPL>(a + (row + t + 1) * D + d)
                                  : vfill_raw<T, CPL>(1.f);
        br[i] = ok ? vload_raw<T, CPL>(dh + (row + t) * D + d) : vfill_raw<T, CPL>(0.f);
      }
#pragma unroll
      for (int i = 0; i < kDiagSeg; ++i) {
        vcvt<T, CPL>(ar[i], av[i]);
        vcvt<T, CPL>(br[i], bv[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kDiagSeg; ++i) {
        const int64_t t = t_first - i;
        const bool ok = i < nok;
        if (ok && t + 1 < L) {
          vcvt<T, CPL>(vload_raw<T, CPL>(a + (row + t + 1) * D + d), av[i]);
        } else {
#pragma unroll
          for (int k = 0; k < CPL; ++k) av[i][k] = 1.f;
        }
        if (ok) {
          vcvt<T, CPL>(vload_raw<T, CPL>(dh + (row + t) * D + d), bv[i]);
        } else {
#pragma unroll
          for (int k = 0; k < CPL; ++k) bv[i][k] = 0.f;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      float P = 1.f, Gs = 0.f;
#pragma unroll
      for (int i = 0; i < kDiagSeg; ++i) {
        Gs = fmaf(av[i][k], Gs, bv[i][k]);
        P *= av[i][k];
        av[i][k] = P;
        bv[i][k] = Gs;
      }
      aggA[seg][ch + k] = P;
      aggB[seg][ch + k] = Gs;
    }
    __syncthreads();

#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const int c = wave + kDiagCT * k;
      float pa = aggA[lane][c], pb = aggB[lane][c];
      const float tc = tile_carry[c];
      wave_incl_pair_scan(pa, pb);
      const float ea = wave_shr1(pa, 1.f), eb = wave_shr1(pb, 0.f);
      carry_in[lane][c] = fmaf(ea, tc, eb);
      if (lane == 63) tile_carry[c] = fmaf(pa, tc, pb);
    }
    __syncthreads();

    float cin[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) cin[k] = carry_in[seg][ch + k];
    // element offset of token t_first, passed through an empty asm so that the
    // per-step addresses are formed here rather than kept live from the loads
    // before the barriers (which spilled them at CPL = 4)
    int64_t offt = (row + t_first) * D + d;
    asm volatile("" : "+v"(offt));
    // h_{t-1} of every step (the step at t = 0 takes h0 instead)
    VRaw<T, CPL> hr[kDiagSeg];
    if constexpr (kPre) {
#pragma unroll
      for (int i = 0; i < kDiagSeg; ++i)
        hr[i] = (i < nok && t_first - i > 0) ? vload_raw<T, CPL>(h + offt - (i + 1) * D)
                                             : vfill_raw<T, CPL>(0.f);
    }
#pragma unroll
    for (int i = 0; i < kDiagSeg; ++i) {
      if (i < nok) {
        const int64_t t = t_first - i;
        const int64_t off = offt - i * D;
        float gt[CPL], hp[CPL], dv[CPL];
#pragma unroll
        for (int k = 0; k < CPL; ++k) gt[k] = fmaf(av[i][k], cin[k], bv[i][k]);
        if constexpr (kPre) {
          vcvt<T, CPL>(hr[i], hp);
          if (t == 0 && h0 != nullptr) {
#pragma unroll
            for (int k = 0; k < CPL; ++k) hp[k] = h0[bi * D + d + k];
          }
        } else if (t > 0) {
          vcvt<T, CPL>(vload_raw<T, CPL>(h + off - D), hp);
        } else {
#pragma unroll
          for (int k = 0; k < CPL; ++k) hp[k] = h0 != nullptr ? h0[bi * D + d + k] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < CPL; ++k) dv[k] = gt[k] * hp[k];
        vstore<T, CPL>(db + off, gt);
        vstore<T, CPL>(da + off, dv);
      }
    }
  }
  __syncthreads();
  if (dh0 != nullptr) {
    for (int c = tid; c < CT; c += kDiagThreads) {
      const int64_t dd = d0 + c;
      if (dd < D) dh0[bi * D + dd] = L > 0 ? Io<T>::load(a + row * D + dd) * tile_carry[c] : tile_carry[c];
    }
  }
}

// Backward with narrow tiles (see diag_scan_narrow_kernel): step u = L-1-t
// of the reversed-time scan, 1024 steps per tile.
template <typename T, int CT, int NT>
__global__ __launch_bounds__(NT) void diag_scan_bwd_narrow_kernel(
    const T* __restrict__ a, const T* __restrict__ h, const float* __restrict__ h0,
    const T* __restrict__ dh, const float* __restrict__ dh_last, T* __restrict__ da,
    T* __restrict__ db, float* __restrict__ dh0, int64_t L, int64_t D) {
  constexpr int NSEG = NT / CT;
  constexpr int SEG = 1024 / NSEG;
  constexpr int TL = NSEG * SEG;
  constexpr int SPL = NSEG / 64;
  static_assert(CT >= 2 && CT <= 8 && TL == 1024 && SPL >= 1 && CT <= NT / 64, "narrow tile shape");
  __shared__ float aggA[NSEG][CT];
  __shared__ float aggB[NSEG][CT];
  __shared__ float carry_in[NSEG][CT];
  __shared__ float tile_carry[CT];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int ch = tid % CT;
  const int seg = tid / CT;
  const int64_t ntile = (D + CT - 1) / CT;
  // consecutive tiles (channels sharing cache lines) on one XCD
  const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t bi = wid / ntile;
  const int64_t d0 = (wid % ntile) * CT;
  const int64_t d = d0 + ch;
  const bool dok = d < D;

  if (tid < CT) tile_carry[tid] = (dh_last != nullptr && d0 + tid < D) ? dh_last[bi * D + d0 + tid] : 0.f;
  __syncthreads();

  const int64_t row = bi * L;
  for (int64_t u0 = 0; u0 < L; u0 += TL) {
    const int64_t us = u0 + static_cast<int64_t>(seg) * SEG;
    const int nok = dok ? static_cast<int>(L - us < SEG ? (L - us > 0 ? L - us : 0) : SEG) : 0;
    const int64_t t_first = L - 1 - us;   // step i is token t_first - i
    float av[SEG], bv[SEG];
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
      const int64_t t = t_first - i;
      av[i] = (i < nok && t + 1 < L) ? Io<T>::load(a + (row + t + 1) * D + d) : 1.f;
      bv[i] = i < nok ? Io<T>::load(dh + (row + t) * D + d) : 0.f;
    }
    float P = 1.f, Gs = 0.f;
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
      Gs = fmaf(av[i], Gs, bv[i]);
      P *= av[i];
      av[i] = P;
      bv[i] = Gs;
    }
    aggA[seg][ch] = P;
    aggB[seg][ch] = Gs;
    __syncthreads();

    if (wave < CT) {
      const int c = wave;
      float pa[SPL], pb[SPL];
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        pa[j] = aggA[SPL * lane + j][c];
        pb[j] = aggB[SPL * lane + j][c];
      }
      float ta = pa[0], tb = pb[0];
#pragma unroll
      for (int j = 1; j < SPL; ++j) {
        tb = fmaf(pa[j], tb, pb[j]);
        ta *= pa[j];
      }
      float ia = ta, ib = tb;
      wave_incl_pair_scan(ia, ib);
      const float tc = tile_carry[c];
      float cin = fmaf(wave_shr1(ia, 1.f), tc, wave_shr1(ib, 0.f));
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        carry_in[SPL * lane + j][c] = cin;
        cin = fmaf(pa[j], cin, pb[j]);
      }
      if (lane == 63) tile_carry[c] = fmaf(ia, tc, ib);
    }
    __syncthreads();

    const float cin = carry_in[seg][ch];
    int64_t offt = (row + t_first) * D + d;
    asm volatile("" : "+v"(offt));
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
      if (i < nok) {
        const int64_t t = t_first - i;
        const int64_t off = offt - i * D;
        const float gt = fmaf(av[i], cin, bv[i]);
        const float hp = t > 0 ? Io<T>::load(h + off - D) : (h0 != nullptr ? h0[bi * D + d] : 0.f);
        Io<T>::store(db + off, gt);
        Io<T>::store(da + off, gt * hp);
      }
    }
  }
  __syncthreads();
  if (dh0 != nullptr && tid < CT && d0 + tid < D) {
    const int64_t dd = d0 + tid;
    dh0[bi * D + dd] = L > 0 ? Io<T>::load(a + row * D + dd) * tile_carry[tid] : tile_carry[tid];
  }
}

template <typename T, int CPL>
static hipError_t launch_diag_bwd_cpl(const void* a, const void* h, const float* h0,
                                      const void* dh, const float* dh_last, void* da, void* db,
                                      float* dh0, int64_t B, int64_t L, int64_t D,
                                      hipStream_t stream) {
  const int64_t ct = kDiagCT * CPL;
  dim3 grid(static_cast<unsigned>(B * ((D + ct - 1) / ct)));
  hipLaunchKernelGGL((diag_scan_bwd_kernel<T, CPL>), grid, dim3(kDiagThreads), 0, stream,
                     static_cast<const T*>(a), static_cast<const T*>(h), h0,
                     static_cast<const T*>(dh), dh_last, static_cast<T*>(da),
                     static_cast<T*>(db), dh0, L, D);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_diag_scan_bwd(const void* a, const void* h, const float* h0, const void* dh,
                                const float* dh_last, void* da, void* db, float* dh0, int64_t B,
                                int64_t L, int64_t D, hipStream_t stream) {
  if (B * ((D + kDiagCT - 1) / kDiagCT) < 64) {   // few chains: narrow tiles
    constexpr int CT = kDiagNarrowCT, NT = kDiagNarrowNT;
    dim3 grid(static_cast<unsigned>(B * ((D + CT - 1) / CT)));
    hipLaunchKernelGGL((diag_scan_bwd_narrow_kernel<T, CT, NT>), grid, dim3(NT), 0, stream,
                       static_cast<const T*>(a), static_cast<const T*>(h), h0,
                       static_cast<const T*>(dh), dh_last, static_cast<T*>(da),
                       static_cast<T*>(db), dh0, L, D);
    return hipGetLastError();
  }
  if (D % 4 == 0 && B * (D / 64) >= 512)
    return launch_diag_bwd_cpl<T, 4>(a, h, h0, dh, dh_last, da, db, dh0, B, L, D, stream);
  if (D % 2 == 0 && B * (D / 32) >= 512)
    return launch_diag_bwd_cpl<T, 2>(a, h, h0, dh, dh_last, da, db, dh0, B, L, D, stream);
  return launch_diag_bwd_cpl<T, 1>(a, h, h0, dh, dh_last, da, db, dh0, B, L, D, stream);
}

template hipError_t launch_diag_scan_bwd<float>(const void*, const void*, const float*, const void*,
                                                const float*, void*, void*, float*, int64_t,
                                                int64_t, int64_t, hipStream_t);
template hipError_t launch_diag_scan_bwd<uint16_t>(const void*, const void*, const float*,
                                                   const void*, const float*, void*, void*,
                                                   float*, int64_t, int64_t, int64_t, hipStream_t);

template <typename T, int CPL>
static hipError_t launch_diag_cpl(const void* a, const void* b, const float* h0, void* h,
                                  float* h_last, int64_t B, int64_t L, int64_t D,
                                  hipStream_t stream) {
  const int64_t ct = kDiagCT * CPL;
  dim3 grid(static_cast<unsigned>(B * ((D + ct - 1) / ct)));
  hipLaunchKernelGGL((diag_scan_kernel<T, CPL>), grid, dim3(kDiagThreads), 0, stream,
                     static_cast<const T*>(a), static_cast<const T*>(b), h0,
                     static_cast<T*>(h), h_last, L, D);
  return hipGetLastError();
}

template <typename T, int CT, int NT>
static hipError_t launch_diag_narrow(const void* a, const void* b, const float* h0, void* h,
                                     float* h_last, int64_t B, int64_t L, int64_t D,
                                     hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(B * ((D + CT - 1) / CT)));
  hipLaunchKernelGGL((diag_scan_narrow_kernel<T, CT, NT>), grid, dim3(NT), 0, stream,
                     static_cast<const T*>(a), static_cast<const T*>(b), h0,
                     static_cast<T*>(h), h_last, L, D);
  return hipGetLastError();
}

// Few chains (fewer than 64 workgroups of 16 channels): narrow tiles of
// kDiagNarrowCT channels.  Otherwise 16 channel groups per workgroup, with
// wider groups once they still give at least two workgroups per CU (512 on
// 256 CUs); the vector accesses need D to be a multiple of the width.
template <typename T>
hipError_t launch_diag_scan(const void* a, const void* b, const float* h0, void* h,
                            float* h_last, int64_t B, int64_t L, int64_t D,
                            hipStream_t stream) {
  if (B * ((D + kDiagCT - 1) / kDiagCT) < 64)
    return launch_diag_narrow<T, kDiagNarrowCT, kDiagNarrowNT>(a, b, h0, h, h_last, B, L, D,
                                                               stream);
  if (D % 4 == 0 && B * (D / 64) >= 512)
    return launch_diag_cpl<T, 4>(a, b, h0, h, h_last, B, L, D, stream);
  if (D % 2 == 0 && B * (D / 32) >= 512)
    return launch_diag_cpl<T, 2>(a, b, h0, h, h_last, B, L, D, stream);
  return launch_diag_cpl<T, 1>(a, b, h0, h, h_last, B, L, D, stream);
}

template hipError_t launch_diag_scan<float>(const void*, const void*, const float*, void*, float*,
                                            int64_t, int64_t, int64_t, hipStream_t);
template hipError_t launch_diag_scan<uint16_t>(const void*, const void*, const float*, void*,
                                               float*, int64_t, int64_t, int64_t, hipStream_t);

}  // namespace lr
