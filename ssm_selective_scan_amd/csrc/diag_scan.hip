// diag_scan.hip — diagonal recurrence h_t = a_t h_{t-1} + b_t (one launch).
//
// ("mlx-recurrence" post, rglru_scan with state [B, D]; IBM Research blog
// "K-Search for MLX", section "A 20x faster prefill: the Mamba SSM kernel":
// recurrence, associative combine and the O(log N)-depth parallel scan.)
//
// One workgroup owns CT = 16 channels of one batch row and walks the sequence
// in tiles of 512 steps.  Inside a tile the 1024 threads split time:
// lane = 16 * (segment within wave) + channel, so each of the 64 time
// segments of 8 steps is scanned sequentially in registers (loads of 16
// consecutive channels are 64-byte coalesced).  The 64 segment aggregates of
// each channel are then combined by one wave with a DPP (a, b)-pair scan, the
// carry entering the tile is folded in, and every lane finishes its segment.
// The carry between tiles lives in LDS, so any L runs in the same launch.
#include "common.hpp"

namespace lr {

constexpr int kDiagCT = 16;          // channels per workgroup
constexpr int kDiagSeg = 8;          // steps per lane segment
constexpr int kDiagThreads = 1024;   // 16 waves, 4 segments per wave
constexpr int kDiagSegs = kDiagThreads / kDiagCT;  // 64 segments per tile
constexpr int kDiagTile = kDiagSegs * kDiagSeg;    // 512 steps per tile

template <typename T>
__global__ __launch_bounds__(kDiagThreads) void diag_scan_kernel(
    const T* __restrict__ a, const T* __restrict__ b, const float* __restrict__ h0,
    T* __restrict__ h, float* __restrict__ h_last, int64_t L, int64_t D) {
  __shared__ float aggA[kDiagSegs][kDiagCT];
  __shared__ float aggB[kDiagSegs][kDiagCT];
  __shared__ float carry_in[kDiagSegs][kDiagCT];
  __shared__ float tile_carry[kDiagCT];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int ch = lane & (kDiagCT - 1);
  const int seg = wave * 4 + (lane >> 4);
  const int64_t ntile = (D + kDiagCT - 1) / kDiagCT;
  const int64_t bi = blockIdx.x / ntile;
  const int64_t d0 = (blockIdx.x % ntile) * kDiagCT;
  const int64_t d = d0 + ch;
  const bool dok = d < D;

  if (tid < kDiagCT) {
    const int64_t dd = d0 + tid;
    tile_carry[tid] = (h0 != nullptr && dd < D) ? h0[bi * D + dd] : 0.f;
  }
  __syncthreads();

  const int64_t row = bi * L;  // token offset of this batch row
  for (int64_t t0 = 0; t0 < L; t0 += kDiagTile) {
    const int64_t ts = t0 + static_cast<int64_t>(seg) * kDiagSeg;
    float av[kDiagSeg], bv[kDiagSeg];
    {
      const int64_t off0 = (row + ts) * D + d;
      const T* pa = a + off0;
      const T* pb = b + off0;
      const int nok = dok ? static_cast<int>(L - ts < kDiagSeg ? (L - ts > 0 ? L - ts : 0) : kDiagSeg) : 0;
#pragma unroll
      for (int i = 0; i < kDiagSeg; ++i) {
        const bool ok = i < nok;
        av[i] = ok ? Io<T>::load(pa) : 1.f;
        bv[i] = ok ? Io<T>::load(pb) : 0.f;
        pa += D;
        pb += D;
      }
    }
    // sequential scan of the segment from a zero state
    float P = 1.f, Hs = 0.f;
#pragma unroll
    for (int i = 0; i < kDiagSeg; ++i) {
      Hs = fmaf(av[i], Hs, bv[i]);
      P *= av[i];
      av[i] = P;   // running product  a_i ... a_first
      bv[i] = Hs;  // running state from zero
    }
    aggA[seg][ch] = P;
    aggB[seg][ch] = Hs;
    __syncthreads();

    if (wave < kDiagCT) {
      // one wave per channel: lane = segment index
      const int c = wave;
      float pa = aggA[lane][c], pb = aggB[lane][c];
      const float tc = tile_carry[c];
      wave_incl_pair_scan(pa, pb);
      // exclusive prefix: the pair of the previous lane (identity at lane 0)
      const float ea = wave_shr1(pa, 1.f), eb = wave_shr1(pb, 0.f);
      carry_in[lane][c] = fmaf(ea, tc, eb);
      if (lane == 63) tile_carry[c] = fmaf(pa, tc, pb);
    }
    __syncthreads();

    const float cin = carry_in[seg][ch];
    {
      T* ph = h + (row + ts) * D + d;
      const int nok = dok ? static_cast<int>(L - ts < kDiagSeg ? (L - ts > 0 ? L - ts : 0) : kDiagSeg) : 0;
#pragma unroll
      for (int i = 0; i < kDiagSeg; ++i) {
        if (i < nok) Io<T>::store(ph, fmaf(av[i], cin, bv[i]));
        ph += D;
      }
    }
  }
  __syncthreads();
  if (h_last != nullptr && tid < kDiagCT) {
    const int64_t dd = d0 + tid;
    if (dd < D) h_last[bi * D + dd] = tile_carry[tid];
  }
}

// ---------------------------------------------------------------------------
// Backward.  For the loss sum_t <dh_t, h_t> + <dh_last, h_{L-1}> the adjoint
// g_t = dl/dh_t obeys the same recurrence run backwards in time,
//     g_{L-1} = dh_{L-1} + dh_last,   g_t = a_{t+1} g_{t+1} + dh_t,
// so with u = L-1-t it is a forward diagonal scan G_u = al_u G_{u-1} + dh_t
// with al_0 = 1, al_u = a_{t+1} and initial state dh_last.  The gradients
// follow per step: db_t = g_t, da_t = g_t h_{t-1} (h_{-1} = h0), and
// dh0 = a_0 g_0.  Same work split as the forward kernel, with u in place of t.
template <typename T>
__global__ __launch_bounds__(kDiagThreads) void diag_scan_bwd_kernel(
    const T* __restrict__ a, const T* __restrict__ h, const float* __restrict__ h0,
    const T* __restrict__ dh, const float* __restrict__ dh_last, T* __restrict__ da,
    T* __restrict__ db, float* __restrict__ dh0, int64_t L, int64_t D) {
  __shared__ float aggA[kDiagSegs][kDiagCT];
  __shared__ float aggB[kDiagSegs][kDiagCT];
  __shared__ float carry_in[kDiagSegs][kDiagCT];
  __shared__ float tile_carry[kDiagCT];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int ch = lane & (kDiagCT - 1);
  const int seg = wave * 4 + (lane >> 4);
  const int64_t ntile = (D + kDiagCT - 1) / kDiagCT;
  const int64_t bi = blockIdx.x / ntile;
  const int64_t d0 = (blockIdx.x % ntile) * kDiagCT;
  const int64_t d = d0 + ch;
  const bool dok = d < D;

  if (tid < kDiagCT) {
    const int64_t dd = d0 + tid;
    tile_carry[tid] = (dh_last != nullptr && dd < D) ? dh_last[bi * D + dd] : 0.f;
  }
  __syncthreads();

  const int64_t row = bi * L;  // token offset of this batch row
  for (int64_t u0 = 0; u0 < L; u0 += kDiagTile) {
    const int64_t us = u0 + static_cast<int64_t>(seg) * kDiagSeg;
    // steps u = us + i, i.e. tokens t = L - 1 - us - i (descending)
    const int nok = dok ? static_cast<int>(L - us < kDiagSeg ? (L - us > 0 ? L - us : 0) : kDiagSeg) : 0;
    float av[kDiagSeg], bv[kDiagSeg];
    {
      const int64_t t_first = L - 1 - us;
#pragma unroll
      for (int i = 0; i < kDiagSeg; ++i) {
        const int64_t t = t_first - i;
        const bool ok = i < nok;
        av[i] = (ok && t + 1 < L) ? Io<T>::load(a + (row + t + 1) * D + d) : 1.f;
        bv[i] = ok ? Io<T>::load(dh + (row + t) * D + d) : 0.f;
      }
    }
    float P = 1.f, Gs = 0.f;
#pragma unroll
    for (int i = 0; i < kDiagSeg; ++i) {
      Gs = fmaf(av[i], Gs, bv[i]);
      P *= av[i];
      av[i] = P;
      bv[i] = Gs;
    }
    aggA[seg][ch] = P;
    aggB[seg][ch] = Gs;
    __syncthreads();

    if (wave < kDiagCT) {
      const int c = wave;
      float pa = aggA[lane][c], pb = aggB[lane][c];
      const float tc = tile_carry[c];
      wave_incl_pair_scan(pa, pb);
      const float ea = wave_shr1(pa, 1.f), eb = wave_shr1(pb, 0.f);
      carry_in[lane][c] = fmaf(ea, tc, eb);
      if (lane == 63) tile_carry[c] = fmaf(pa, tc, pb);
    }
    __syncthreads();

    const float cin = carry_in[seg][ch];
    {
      const int64_t t_first = L - 1 - us;
#pragma unroll
      for (int i = 0; i < kDiagSeg; ++i) {
        if (i < nok) {
          const int64_t t = t_first - i;
          const float gt = fmaf(av[i], cin, bv[i]);
          const float hp = t > 0 ? Io<T>::load(h + (row + t - 1) * D + d)
                                 : (h0 != nullptr ? h0[bi * D + d] : 0.f);
          Io<T>::store(db + (row + t) * D + d, gt);
          Io<T>::store(da + (row + t) * D + d, gt * hp);
        }
      }
    }
  }
  __syncthreads();
  if (dh0 != nullptr && tid < kDiagCT) {
    const int64_t dd = d0 + tid;
    if (dd < D) dh0[bi * D + dd] = L > 0 ? Io<T>::load(a + row * D + dd) * tile_carry[tid] : tile_carry[tid];
  }
}

template <typename T>
hipError_t launch_diag_scan_bwd(const void* a, const void* h, const float* h0, const void* dh,
                                const float* dh_last, void* da, void* db, float* dh0, int64_t B,
                                int64_t L, int64_t D, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(B * ((D + kDiagCT - 1) / kDiagCT)));
  hipLaunchKernelGGL(diag_scan_bwd_kernel<T>, grid, dim3(kDiagThreads), 0, stream,
                     static_cast<const T*>(a), static_cast<const T*>(h), h0,
                     static_cast<const T*>(dh), dh_last, static_cast<T*>(da),
                     static_cast<T*>(db), dh0, L, D);
  return hipGetLastError();
}

template hipError_t launch_diag_scan_bwd<float>(const void*, const void*, const float*, const void*,
                                                const float*, void*, void*, float*, int64_t,
                                                int64_t, int64_t, hipStream_t);
template hipError_t launch_diag_scan_bwd<uint16_t>(const void*, const void*, const float*,
                                                   const void*, const float*, void*, void*,
                                                   float*, int64_t, int64_t, int64_t, hipStream_t);

template <typename T>
hipError_t launch_diag_scan(const void* a, const void* b, const float* h0, void* h,
                            float* h_last, int64_t B, int64_t L, int64_t D,
                            hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(B * ((D + kDiagCT - 1) / kDiagCT)));
  hipLaunchKernelGGL(diag_scan_kernel<T>, grid, dim3(kDiagThreads), 0, stream,
                     static_cast<const T*>(a), static_cast<const T*>(b), h0,
                     static_cast<T*>(h), h_last, L, D);
  return hipGetLastError();
}

template hipError_t launch_diag_scan<float>(const void*, const void*, const float*, void*, float*,
                                            int64_t, int64_t, int64_t, hipStream_t);
template hipError_t launch_diag_scan<uint16_t>(const void*, const void*, const float*, void*,
                                               float*, int64_t, int64_t, int64_t, hipStream_t);

}  // namespace lr
