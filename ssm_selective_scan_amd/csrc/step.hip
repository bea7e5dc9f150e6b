// step.hip — single-token (decode) steps of the four recurrences.
//
// ("lrnnx: A library for Linear RNNs", Key Contributions 1 and the Benchmarks
// paragraphs: every layer has a step method for autoregressive generation,
// checked against the parallel and recurrent modes, and the decode loop runs
// under graph capture to avoid a host round trip per step.)
//
// Each call advances a caller-owned fp32 state by one token in place and
// writes that token's output.  A step reads and writes the whole state once,
// so these kernels are bound by HBM bandwidth on the state; they use 16-byte
// accesses along the state's contiguous dimension, and none of them
// allocates, synchronises or issues memset, so a loop of steps can be
// captured into a HIP graph and replayed.
#include "common.hpp"
#include "launch.hpp"

namespace lr {

enum { kStepZoh = 0, kStepEuler = 1, kStepBilinear = 2, kStepDirac = 3 };

template <int DISC>
__device__ __forceinline__ void step_disc(float dtv, float Av, float& e, float& phi) {
  const float lam = dtv * Av;
  if (DISC == kStepBilinear) {
    const float r = __builtin_amdgcn_rcpf(1.f - 0.5f * lam);
    e = (1.f + 0.5f * lam) * r;
    phi = dtv * r;
    return;
  }
  e = fast_exp2(lam * kLog2e);
  if (DISC == kStepEuler) {
    phi = dtv;
  } else if (DISC == kStepDirac) {
    phi = 1.f;
  } else {
    const float ser =
        dtv * fmaf(lam, fmaf(lam, fmaf(lam, fmaf(lam, 1.f / 120.f, 1.f / 24.f), 1.f / 6.f), 0.5f), 1.f);
    phi = fabsf(lam) < 0.1f ? ser : (e - 1.f) / Av;
  }
}

// ---------------------------------------------------------------------------
// diagonal: h = a h + b, out = h
template <typename T>
__global__ __launch_bounds__(256) void diag_step_kernel(const T* __restrict__ a, const T* __restrict__ b,
                                                        float* __restrict__ h, T* __restrict__ out,
                                                        int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const float v = fmaf(Io<T>::load(a + i), h[i], Io<T>::load(b + i));
  h[i] = v;
  if (out != nullptr) Io<T>::store(out + i, v);
}

// ---------------------------------------------------------------------------
// selective: per (b, d) a group of NP lanes (NP = N rounded up to a power of
// two) holds one state index each; y = sum_n C h + D x by a shuffle reduction
template <typename T, int DISC>
__global__ __launch_bounds__(256) void selective_step_kernel(
    const T* __restrict__ x, const T* __restrict__ dt, const float* __restrict__ A,
    const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ Dskip,
    float* __restrict__ h, T* __restrict__ y, int64_t B, int64_t D, int N, int lgNP) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int NP = 1 << lgNP;
  const int n = static_cast<int>(gid & (NP - 1));
  const int64_t bd = gid >> lgNP;
  const bool ok = bd < B * D && n < N;
  float contrib = 0.f;
  float xv = 0.f;
  if (bd < B * D) {
    const int64_t b = bd / D, d = bd % D;
    xv = Io<T>::load(x + bd);
    if (ok) {
      float e, phi;
      step_disc<DISC>(Io<T>::load(dt + bd), A[d * N + n], e, phi);
      const int64_t hi = bd * N + n;
      const float hv = fmaf(e, h[hi], phi * Io<T>::load(Bm + b * N + n) * xv);
      h[hi] = hv;
      contrib = Io<T>::load(Cm + b * N + n) * hv;
    }
  }
  for (int off = NP >> 1; off > 0; off >>= 1) contrib += __shfl_xor(contrib, off);
  if (bd < B * D && n == 0) {
    const float dk = Dskip != nullptr ? Dskip[bd % D] : 0.f;
    Io<T>::store(y + bd, fmaf(dk, xv, contrib));
  }
}

// ---------------------------------------------------------------------------
// SSD: state rows h[b, h, p, 0:N) (n contiguous).  Four lanes per row, each
// with N/4 consecutive n as float4; y[p] = sum_n C h by a 4-lane reduction.
template <int DISC, int NS>
__global__ __launch_bounds__(256) void ssd_step_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ dt, const float* __restrict__ A,
    const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ Cm,
    const float* __restrict__ Dskip, float* __restrict__ hs, uint16_t* __restrict__ y, int64_t B,
    int64_t H, int64_t P, int64_t G) {
  constexpr int kPer = NS / 4;          // n per lane
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int q = static_cast<int>(gid & 3);
  const int64_t row = gid >> 2;         // (b H + h) P + p
  const bool ok = row < B * H * P;
  float acc = 0.f, xv = 0.f;
  if (ok) {
    const int64_t bh = row / P;
    const int64_t b = bh / H, hh = bh % H;
    const int64_t g = hh / (H / G);
    xv = bf2f(x[row]);
    float e, phi;
    step_disc<DISC>(bf2f(dt[bh]), A[hh], e, phi);
    const float u = phi * xv;
    const uint16_t* Bp = Bm + (b * G + g) * NS + kPer * q;
    const uint16_t* Cp = Cm + (b * G + g) * NS + kPer * q;
    float* hp = hs + row * NS + kPer * q;
#pragma unroll
    for (int c = 0; c < kPer; c += 4) {
      f32x4 hv = *reinterpret_cast<const f32x4*>(hp + c);
      const u16x4 bv = *reinterpret_cast<const u16x4*>(Bp + c);
      const u16x4 cv = *reinterpret_cast<const u16x4*>(Cp + c);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        hv[r] = fmaf(e, hv[r], u * bf2f(bv[r]));
        acc = fmaf(bf2f(cv[r]), hv[r], acc);
      }
      *reinterpret_cast<f32x4*>(hp + c) = hv;
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  if (ok && q == 0) {
    const float dk = Dskip != nullptr ? Dskip[(row / P) % H] : 0.f;
    y[row] = f2bf(fmaf(dk, xv, acc));
  }
}

// ---------------------------------------------------------------------------
// GLA: state S[b, h, k, v] (v contiguous).  A workgroup owns one (b, h) and
// 64 columns v; wave w updates rows k = w, w + 8, ... of those columns (one
// column per lane) and the 8 per-wave partial outputs are summed in LDS.
__global__ __launch_bounds__(512) void gla_step_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ g, float* __restrict__ S, uint16_t* __restrict__ o, int64_t B,
    int64_t H, int64_t K, int64_t V) {
  __shared__ float part[8][64];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int64_t nvs = V / 64;
  const int64_t vs = blockIdx.x % nvs, bh = blockIdx.x / nvs;
  const int64_t col = 64 * vs + lane;
  const float gv = bf2f(g[bh]);
  const float vv = bf2f(v[bh * V + col]);
  float* Sp = S + bh * K * V + col;
  float acc = 0.f;
  for (int64_t kk = w; kk < K; kk += 8) {
    const float sv = fmaf(gv, Sp[kk * V], bf2f(k[bh * K + kk]) * vv);
    Sp[kk * V] = sv;
    acc = fmaf(bf2f(q[bh * K + kk]), sv, acc);
  }
  part[w][lane] = acc;
  __syncthreads();
  if (w == 0) {
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < 8; ++ww) s += part[ww][lane];
    o[bh * V + col] = f2bf(s);
  }
}

// ---------------------------------------------------------------------------
template <typename T>
hipError_t launch_diag_step(const void* a, const void* b, float* h, void* out, int64_t n,
                            hipStream_t s) {
  hipLaunchKernelGGL(diag_step_kernel<T>, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                     s, static_cast<const T*>(a), static_cast<const T*>(b), h, static_cast<T*>(out),
                     n);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_selective_step(int disc, const void* x, const void* dt, const float* A,
                                 const void* Bm, const void* Cm, const float* Dskip, float* h,
                                 void* y, int64_t B, int64_t D, int N, hipStream_t s) {
  int lg = 0;
  while ((1 << lg) < N) ++lg;
  const int64_t threads = (B * D) << lg;
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, static_cast<const T*>(x),
                       static_cast<const T*>(dt), A, static_cast<const T*>(Bm),
                       static_cast<const T*>(Cm), Dskip, h, static_cast<T*>(y), B, D, N, lg);
  };
  switch (disc) {
    case kStepEuler: go(selective_step_kernel<T, kStepEuler>); break;
    case kStepBilinear: go(selective_step_kernel<T, kStepBilinear>); break;
    case kStepDirac: go(selective_step_kernel<T, kStepDirac>); break;
    default: go(selective_step_kernel<T, kStepZoh>);
  }
  return hipGetLastError();
}

hipError_t launch_ssd_step(int disc, const void* x, const void* dt, const float* A, const void* Bm,
                           const void* Cm, const float* Dskip, float* h, void* y, int64_t B,
                           int64_t H, int64_t P, int64_t G, int64_t N, hipStream_t s) {
  const int64_t threads = B * H * P * 4;
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, static_cast<const uint16_t*>(x),
                       static_cast<const uint16_t*>(dt), A, static_cast<const uint16_t*>(Bm),
                       static_cast<const uint16_t*>(Cm), Dskip, h, static_cast<uint16_t*>(y), B, H,
                       P, G);
  };
  if (N == 128) {
    switch (disc) {
      case kStepEuler: go(ssd_step_kernel<kStepEuler, 128>); break;
      case kStepBilinear: go(ssd_step_kernel<kStepBilinear, 128>); break;
      case kStepDirac: go(ssd_step_kernel<kStepDirac, 128>); break;
      default: go(ssd_step_kernel<kStepZoh, 128>);
    }
  } else {
    switch (disc) {
      case kStepEuler: go(ssd_step_kernel<kStepEuler, 64>); break;
      case kStepBilinear: go(ssd_step_kernel<kStepBilinear, 64>); break;
      case kStepDirac: go(ssd_step_kernel<kStepDirac, 64>); break;
      default: go(ssd_step_kernel<kStepZoh, 64>);
    }
  }
  return hipGetLastError();
}

hipError_t launch_gla_step(const void* q, const void* k, const void* v, const void* g, float* S,
                           void* o, int64_t B, int64_t H, int64_t K, int64_t V, hipStream_t s) {
  hipLaunchKernelGGL(gla_step_kernel, dim3(static_cast<unsigned>(B * H * (V / 64))), dim3(512), 0, s,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(g), S,
                     static_cast<uint16_t*>(o), B, H, K, V);
  return hipGetLastError();
}

template hipError_t launch_diag_step<float>(const void*, const void*, float*, void*, int64_t,
                                            hipStream_t);
template hipError_t launch_diag_step<uint16_t>(const void*, const void*, float*, void*, int64_t,
                                               hipStream_t);
template hipError_t launch_selective_step<float>(int, const void*, const void*, const float*,
                                                 const void*, const void*, const float*, float*,
                                                 void*, int64_t, int64_t, int, hipStream_t);
template hipError_t launch_selective_step<uint16_t>(int, const void*, const void*, const float*,
                                                    const void*, const void*, const float*, float*,
                                                    void*, int64_t, int64_t, int, hipStream_t);

}  // namespace lr
