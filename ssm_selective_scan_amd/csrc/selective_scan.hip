// selective_scan.hip — Mamba-1 selective scan with ZOH/Euler discretisation
// and the readout y = C.h + D.x fused into the scan (one launch).
//
// ("lrnnx: A library for Linear RNNs", Key Contributions 2-3: time-varying
// selective scan, ZOH discretisation, fused scan + output projection; IBM
// Research blog "K-Search for MLX", section "Translating CUDA expertise to
// MLX": evaluate exp as exp2 with log2(e) folded into the argument.)
//
// Work split: a workgroup owns one batch row and 64 consecutive channels d
// (lane = d, so every per-token load and store is a coalesced row segment).
// Its waves split the state index n: wave w owns n in [4w, 4w+4), so the
// (d, n) chains it carries stay in registers for the whole sequence and the
// hidden state never touches memory.  Tokens are staged through LDS in tiles
// of TT steps; each wave writes its partial readout sum_n C h to LDS and the
// workgroup adds the partials, D.x, and stores y.
//
// Per (t, d, n) the ZOH update costs one v_exp_f32 and six VALU operations:
//   e = 2^(dt A log2e);  v = (B x)/A;  h = e (h + v) - v;  y += C h
// which equals h = e h + expm1(dt A)/A B x.  Its absolute rounding error is
// about ulp(h) per step when |A| is not small.  A workgroup that sees any
// |A| < 0.5 (including A = 0) switches, uniformly, to the precise form
// phi = dt (1 + l/2 + l^2/6 + l^3/24) for |l| = |dt A| < 0.1, else
// (e - 1)/A, which keeps phi accurate to fp32 rounding at every A.
#include "common.hpp"

namespace lr {

constexpr int kSelNPW = 4;     // state indices per wave
constexpr int kSelCT = 64;     // channels per workgroup (one per lane)

enum { kDiscZoh = 0, kDiscEuler = 1 };

template <typename T, int DISC, bool PRECISE, int TT>
__device__ __forceinline__ void selective_body(
    const T* __restrict__ x, const T* __restrict__ dt, const T* __restrict__ Bm,
    const T* __restrict__ Cm, const float* __restrict__ Dskip, T* __restrict__ y,
    float* __restrict__ smem, float (&h)[kSelNPW], const float (&A2)[kSelNPW],
    const float (&iA)[kSelNPW], const float (&An)[kSelNPW], int64_t bi, int64_t d0, int64_t L,
    int64_t D, int N) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int w = tid >> 6, lane = tid & 63;
  const int nw = nthr >> 6;
  const int n0 = w * kSelNPW;
  float* xs = smem;               // [TT][64]
  float* dts = xs + TT * 64;      // [TT][64]
  float* Bs = dts + TT * 64;      // [TT][64]  (n < N used)
  float* Cs = Bs + TT * 64;       // [TT][64]
  float* Dk = Cs + TT * 64;       // [64]
  float* yp = Dk + 64;            // [nw][TT][64]

  for (int64_t t0 = 0; t0 < L; t0 += TT) {
    // ---- stage a tile of TT tokens
    for (int idx = tid; idx < TT * 64; idx += nthr) {
      const int tt = idx >> 6, dd = idx & 63;
      const int64_t t = t0 + tt;
      const bool ok = t < L && d0 + dd < D;
      const int64_t off = (bi * L + t) * D + d0 + dd;
      xs[idx] = ok ? Io<T>::load(x + off) : 0.f;
      dts[idx] = ok ? Io<T>::load(dt + off) : 0.f;
    }
    for (int idx = tid; idx < TT * N; idx += nthr) {
      const int tt = idx / N, n = idx - tt * N;
      const int64_t t = t0 + tt;
      const bool ok = t < L;
      const int64_t off = (bi * L + t) * N + n;
      Bs[tt * 64 + n] = ok ? Io<T>::load(Bm + off) : 0.f;
      Cs[tt * 64 + n] = ok ? Io<T>::load(Cm + off) : 0.f;
    }
    __syncthreads();

    // ---- the recurrence for this wave's (d, n) chains
    const int tend = static_cast<int>((L - t0) < TT ? (L - t0) : TT);
    for (int tt = 0; tt < tend; ++tt) {
      const float xv = xs[tt * 64 + lane];
      const float dv = dts[tt * 64 + lane];
      const float4 b4 = *reinterpret_cast<const float4*>(Bs + tt * 64 + n0);
      const float4 c4 = *reinterpret_cast<const float4*>(Cs + tt * 64 + n0);
      const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
      const float cc[4] = {c4.x, c4.y, c4.z, c4.w};
      const float ux = (DISC == kDiscEuler) ? dv * xv : 0.f;
      float yacc = 0.f;
#pragma unroll
      for (int j = 0; j < kSelNPW; ++j) {
        if (n0 + j < N) {  // uniform across the wave
          const float e = fast_exp2(dv * A2[j]);
          if (DISC == kDiscEuler) {
            h[j] = fmaf(e, h[j], bb[j] * ux);
          } else if (!PRECISE) {
            const float v = (bb[j] * xv) * iA[j];
            h[j] = fmaf(e, h[j] + v, -v);
          } else {
            const float l = dv * An[j];
            const float ser = dv * fmaf(l, fmaf(l, fmaf(l, 1.f / 24.f, 1.f / 6.f), 0.5f), 1.f);
            const float phi = fabsf(l) < 0.1f ? ser : (e - 1.f) * iA[j];
            h[j] = fmaf(e, h[j], phi * (bb[j] * xv));
          }
          yacc = fmaf(cc[j], h[j], yacc);
        }
      }
      yp[(w * TT + tt) * 64 + lane] = yacc;
    }
    __syncthreads();

    // ---- sum the per-wave partial readouts, add D x, store y
    for (int idx = tid; idx < TT * 64; idx += nthr) {
      const int tt = idx >> 6, dd = idx & 63;
      const int64_t t = t0 + tt;
      if (t < L && d0 + dd < D) {
        float s = Dk[dd] * xs[idx];
        for (int ww = 0; ww < nw; ++ww) s += yp[(ww * TT + tt) * 64 + dd];
        Io<T>::store(y + (bi * L + t) * D + d0 + dd, s);
      }
    }
    __syncthreads();
  }
}

template <typename T, int DISC, int TT>
__global__ __launch_bounds__(1024) void selective_scan_kernel(
    const T* __restrict__ x, const T* __restrict__ dt, const float* __restrict__ A,
    const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ Dskip,
    const float* __restrict__ h0, T* __restrict__ y, float* __restrict__ h_last, int64_t L,
    int64_t D, int N) {
  extern __shared__ float smem[];
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int64_t ndt = (D + kSelCT - 1) / kSelCT;
  const int64_t bi = blockIdx.x / ndt;
  const int64_t d0 = (blockIdx.x % ndt) * kSelCT;
  const int64_t d = d0 + lane;
  const bool dok = d < D;
  const int n0 = w * kSelNPW;

  float A2[kSelNPW], iA[kSelNPW], An[kSelNPW], h[kSelNPW];
  bool small = false;
#pragma unroll
  for (int j = 0; j < kSelNPW; ++j) {
    const int n = n0 + j;
    const bool ok = dok && n < N;
    const float a = ok ? A[d * N + n] : -1.f;
    An[j] = a;
    A2[j] = a * kLog2e;
    iA[j] = 1.f / a;
    small |= ok && fabsf(a) < 0.5f;
    h[j] = (ok && h0 != nullptr) ? h0[(bi * D + d) * N + n] : 0.f;
  }
  {
    float* Dk = smem + 4 * TT * 64;
    if (tid < 64) Dk[tid] = (Dskip != nullptr && d0 + tid < D) ? Dskip[d0 + tid] : 0.f;
  }
  const bool precise = __syncthreads_or(small ? 1 : 0) != 0;

  if (DISC == kDiscEuler) {
    selective_body<T, DISC, false, TT>(x, dt, Bm, Cm, Dskip, y, smem, h, A2, iA, An, bi, d0, L, D, N);
  } else if (precise) {
    selective_body<T, DISC, true, TT>(x, dt, Bm, Cm, Dskip, y, smem, h, A2, iA, An, bi, d0, L, D, N);
  } else {
    selective_body<T, DISC, false, TT>(x, dt, Bm, Cm, Dskip, y, smem, h, A2, iA, An, bi, d0, L, D, N);
  }

  if (h_last != nullptr && dok) {
#pragma unroll
    for (int j = 0; j < kSelNPW; ++j)
      if (n0 + j < N) h_last[(bi * D + d) * N + n0 + j] = h[j];
  }
}

template <typename T, int DISC, int TT>
static hipError_t launch_sel(const void* x, const void* dt, const float* A, const void* Bm,
                             const void* Cm, const float* Dskip, const float* h0, void* y,
                             float* h_last, int64_t B, int64_t L, int64_t D, int N,
                             hipStream_t stream) {
  const int nw = (N + kSelNPW - 1) / kSelNPW;
  const size_t lds = (4 * TT * 64 + 64 + static_cast<size_t>(nw) * TT * 64) * sizeof(float);
  dim3 grid(static_cast<unsigned>(B * ((D + kSelCT - 1) / kSelCT)));
  hipLaunchKernelGGL((selective_scan_kernel<T, DISC, TT>), grid, dim3(64 * nw), lds, stream,
                     static_cast<const T*>(x), static_cast<const T*>(dt), A,
                     static_cast<const T*>(Bm), static_cast<const T*>(Cm), Dskip, h0,
                     static_cast<T*>(y), h_last, L, D, N);
  return hipGetLastError();
}

// TT = 32 tokens per LDS tile while the per-wave partial buffers fit
// (N <= 32); larger N uses TT = 16.
template <typename T>
hipError_t launch_selective_scan(int disc, const void* x, const void* dt, const float* A,
                                 const void* Bm, const void* Cm, const float* Dskip,
                                 const float* h0, void* y, float* h_last, int64_t B, int64_t L,
                                 int64_t D, int N, hipStream_t stream) {
  if (N <= 32) {
    return disc == kDiscEuler
               ? launch_sel<T, kDiscEuler, 32>(x, dt, A, Bm, Cm, Dskip, h0, y, h_last, B, L, D, N, stream)
               : launch_sel<T, kDiscZoh, 32>(x, dt, A, Bm, Cm, Dskip, h0, y, h_last, B, L, D, N, stream);
  }
  return disc == kDiscEuler
             ? launch_sel<T, kDiscEuler, 16>(x, dt, A, Bm, Cm, Dskip, h0, y, h_last, B, L, D, N, stream)
             : launch_sel<T, kDiscZoh, 16>(x, dt, A, Bm, Cm, Dskip, h0, y, h_last, B, L, D, N, stream);
}

template hipError_t launch_selective_scan<float>(int, const void*, const void*, const float*,
                                                 const void*, const void*, const float*,
                                                 const float*, void*, float*, int64_t, int64_t,
                                                 int64_t, int, hipStream_t);
template hipError_t launch_selective_scan<uint16_t>(int, const void*, const void*, const float*,
                                                    const void*, const void*, const float*,
                                                    const float*, void*, float*, int64_t,
                                                    int64_t, int64_t, int, hipStream_t);

}  // namespace lr
