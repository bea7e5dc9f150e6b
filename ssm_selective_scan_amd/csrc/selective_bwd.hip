// selective_bwd.hip — backward of the Mamba-1 selective scan with segment
// checkpoints and recompute.
//
// ("lrnnx: A library for Linear RNNs", Key Contributions 2-3: the
// time-varying selective scan with ZOH discretisation and fused readout;
// "mlx-recurrence" post, Apple Developer Forums thread 840535: the training
// path keeps the state at segment boundaries in the forward and recomputes
// inside each segment in the backward.)
//
// Loss l = sum(dy * y) + <dh_last, h_last>.  Per chain (b, d, n), with
// G_t = dl/dh_t:
//   G_t = e_{t+1} G_{t+1} + dy_t C_t[n],          dh0 = e_0 G_0
//   dx_t[d] = sum_n G phi B_t[n] + D[d] dy_t[d]
//   dB_t[n] = sum_d G phi x_t[d],   dC_t[n] = sum_d h_t dy_t[d]
//   de = G h_{t-1},  dphi = G B_t[n] x_t[d]  -> ddt (sum over n), dA (sum over b, t)
//
// Work split: one workgroup per (batch row, 64 channels), 8 waves, wave w
// owning state indices n = 2w, 2w + 1 of every channel (lane = channel), as
// in the forward.  The workgroup walks the segments last to first carrying
// G in registers.  Per segment it first runs the forward from the segment's
// checkpoint, keeping the state entering every 32-token chunk in a
// workspace slice of its own (cache resident), then walks the chunks last to
// first: recompute the chunk's 32 states into LDS, then the reverse steps.
// Sums over n (dx, ddt) go through LDS across the waves (written over the
// chunk's states once a step has read them); sums over the 64 channels of a
// wave (dB, dC) pair lanes with the gfx950 lane-swap instructions and finish
// with DPP row shifts; sums over channel tiles (dB, dC) and batch rows (dA,
// dD) are fixed-order partial sums reduced by a second launch, so results
// are deterministic.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace lr {

constexpr int kSbNW = 8;      // waves
constexpr int kSbCT = 64;     // channels per workgroup

// NPW state indices per lane, so a workgroup covers NN = 8 NPW of them;
// chunks of TC tokens, SUB chunks per segment (seg <= 256).  N <= 16 runs
// with 2 x 32, N <= 32 with 4 x 16, N <= 64 with 8 x 8 (the chunk's states
// fill the same LDS).
template <int NPW>
struct SbCfg {
  static constexpr int TC = NPW == 2 ? 32 : (NPW == 4 ? 16 : 8);
  static constexpr int SUB = 256 / TC;
  static constexpr int NN = NPW * kSbNW;
};

enum { kSbZoh = 0, kSbEuler = 1, kSbBilinear = 2, kSbDirac = 3 };

struct SelBwdArgs {
  const void* x; const void* dt; const float* A; const void* Bm; const void* Cm;
  const float* Dskip; const float* ckpt; const void* dy; const float* dh_last;
  void* dx; void* ddt; float* dh0;
  float* dBpart; float* dCpart;   // [ntile][B][L][N]
  float* dApart;                  // [B][D][N]
  float* dDpart;                  // [B][D]
  float* subck;                   // [B * ntile][SUB][kSbNW][NPW][64]: state entering each chunk
  void* dBm; void* dCm; float* dA; float* dD;
  int64_t B, L, D, N, seg, nseg, ntile;
};

// e, phi and their derivatives for one (dt, A).  ZOH: phi = expm1(dt A) / A
// through a series near dt A = 0 (A = 0 included); dphi/dA = (dt e - phi)/A,
// also through its series there.  Bilinear: e = (1 + l/2) r, phi = dt r with
// r = 1 / (1 - l/2).  Dirac: phi = 1.
// iA = 1/A (any value where A == 0: the series branch is taken there).
template <int DISC>
__device__ __forceinline__ void sb_disc(float dtv, float Av, float iA, float& e, float& phi) {
  const float lam = dtv * Av;
  if (DISC == kSbBilinear) {
    const float r = __builtin_amdgcn_rcpf(1.f - 0.5f * lam);
    e = (1.f + 0.5f * lam) * r;
    phi = dtv * r;
    return;
  }
  e = fast_exp2(lam * kLog2e);
  if (DISC == kSbEuler) {
    phi = dtv;
  } else if (DISC == kSbDirac) {
    phi = 1.f;
  } else {
    const float ser =
        dtv * fmaf(lam, fmaf(lam, fmaf(lam, fmaf(lam, 1.f / 120.f, 1.f / 24.f), 1.f / 6.f), 0.5f), 1.f);
    phi = fabsf(lam) < 0.1f ? ser : (e - 1.f) * iA;
  }
}

// (de/ddt, de/dA, dphi/ddt, dphi/dA) at (dt, A) with e, phi from sb_disc.
template <int DISC>
__device__ __forceinline__ void sb_grads(float dtv, float Av, float iA, float e, float phi,
                                         float& dedt, float& dedA, float& dpdt, float& dpdA) {
  if (DISC == kSbBilinear) {
    const float r = __builtin_amdgcn_rcpf(1.f - 0.5f * dtv * Av);
    const float r2 = r * r;
    dedt = Av * r2;
    dedA = dtv * r2;
    dpdt = r2;
    dpdA = 0.5f * dtv * dtv * r2;
    return;
  }
  dedt = Av * e;
  dedA = dtv * e;
  if (DISC == kSbEuler) {
    dpdt = 1.f;
    dpdA = 0.f;
  } else if (DISC == kSbDirac) {
    dpdt = 0.f;
    dpdA = 0.f;
  } else {
    const float lam = dtv * Av;
    const float ser = dtv * dtv *
                      fmaf(lam, fmaf(lam, fmaf(lam, fmaf(lam, 1.f / 144.f, 1.f / 30.f), 1.f / 8.f), 1.f / 3.f), 0.5f);
    dpdt = e;
    dpdA = fabsf(lam) < 0.1f ? ser : (dtv * e - phi) * iA;
  }
}

template <int NPW>
struct SbLds {
  static constexpr int TC = SbCfg<NPW>::TC, NN = SbCfg<NPW>::NN;
  float xs[TC][kSbCT], dts[TC][kSbCT], dys[TC][kSbCT];
  float Bs[TC][NN], Cs[TC][NN];                       // n >= N stay zero
  // each wave's states of the chunk; the reverse step of token i overwrites
  // its slot with the wave's partial sums of dx ([0]) and ddt ([1])
  float hsl[kSbNW][TC][NPW][kSbCT];
  float rbc[TC][2][NN];                               // dB, dC of the chunk
};   // 160 KB (NPW = 2), 148 KB (NPW = 4), 142 KB (NPW = 8)

// Sum over the 64 lanes of v[0..3]; on return lane 15 of row q (lanes
// 16 q .. 16 q + 15) holds the total of v[q].  Halves and rows are paired
// with the gfx950 lane-swap instructions (permlane32_swap exchanges the
// upper 32 lanes of its first operand with the lower 32 of its second,
// permlane16_swap the odd rows of the first with the even rows of the
// second), then each row is reduced with DPP row shifts.
__device__ __forceinline__ float sum4_over_lanes(const float (&v)[4]) {
  const auto p0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0]), __float_as_uint(v[2]),
                                                   false, false);
  const auto p1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[1]), __float_as_uint(v[3]),
                                                   false, false);
  // lanes < 32: sums of v[0], v[1] over lane pairs (l, l + 32); lanes >= 32: of v[2], v[3]
  const float a0 = __uint_as_float(p0[0]) + __uint_as_float(p0[1]);
  const float a1 = __uint_as_float(p1[0]) + __uint_as_float(p1[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(a0), __float_as_uint(a1), false,
                                                  false);
  float r = __uint_as_float(q[0]) + __uint_as_float(q[1]);
  r += dpp_f<0x111, 0xf>(0.f, r);   // row_shr:1
  r += dpp_f<0x112, 0xf>(0.f, r);   // row_shr:2
  r += dpp_f<0x114, 0xf>(0.f, r);   // row_shr:4
  r += dpp_f<0x118, 0xf>(0.f, r);   // row_shr:8
  return r;
}

// FAST: ZOH with bf16 I/O and every |A| of the workgroup >= 0.5, where
// phi = (e - 1)/A and v = B x / A need no series (their relative error,
// about 6e-8 / |dt A|, stays below bf16 rounding).  Then, with h_t the
// state after step t,
//   dh_t/ddt = A h_t + B x                  (the continuous-time derivative)
//   dh_t/dA  = dt h_t + (dt - phi) B x / A
// which use h_t only (no h_{t-1}).  Other cases use sb_disc/sb_grads.
template <typename T, int DISC, bool FAST, int NPW>
__device__ __forceinline__ void selective_bwd_body(const SelBwdArgs& a, SbLds<NPW>& sm, int64_t b,
                                                   int64_t tile, const float (&Av)[NPW],
                                                   const float (&iAv)[NPW], const bool (&okj)[NPW],
                                                   float (&G)[NPW], float (&dAacc)[NPW],
                                                   float& dDacc) {
  constexpr int kSbTC = SbCfg<NPW>::TC, kSbSub = SbCfg<NPW>::SUB;
  const T* x = static_cast<const T*>(a.x);
  const T* dt = static_cast<const T*>(a.dt);
  const T* Bm = static_cast<const T*>(a.Bm);
  const T* Cm = static_cast<const T*>(a.Cm);
  const T* dy = static_cast<const T*>(a.dy);
  T* dx = static_cast<T*>(a.dx);
  T* ddt = static_cast<T*>(a.ddt);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int64_t d0 = tile * kSbCT;
  const int N = static_cast<int>(a.N);
  const int n0 = NPW * w;
  const int64_t D = a.D, L = a.L;
  float* subp = a.subck + static_cast<int64_t>(blockIdx.x) * kSbSub * kSbNW * NPW * kSbCT;
  // this lane's slot of chain j in the state entering chunk c
  auto sub_at = [&](int c, int j) -> float& { return subp[((c * kSbNW + w) * NPW + j) * kSbCT + lane]; };
  const float Dd = (a.Dskip != nullptr && d0 + lane < D) ? a.Dskip[d0 + lane] : 0.f;
  float A2[NPW];   // A log2(e)
#pragma unroll
  for (int j = 0; j < NPW; ++j) A2[j] = Av[j] * kLog2e;

  // e, phi of one step
  auto disc = [&](float dtv, int j, float& e, float& phi) {
    if constexpr (FAST) {
      e = fast_exp2(dtv * A2[j]);
      phi = (e - 1.f) * iAv[j];
    } else {
      sb_disc<DISC>(dtv, Av[j], iAv[j], e, phi);
    }
  };

  // Staging: a chunk's inputs are loaded into registers one chunk ahead
  // (fetch) and written to LDS when the chunk starts (put).  The registers
  // keep the raw elements and put() converts them, so no conversion next to
  // a load makes the wave wait for it.  Missing tokens and channels are
  // zeros: dt = 0 gives e = 1, phi = 0, so they leave the state unchanged.
  constexpr int kSt = kSbTC * kSbCT / 512;   // staged x/dt/dy elements per thread
  T rx[kSt], rdt[kSt], rdy[kSt], rb = T(0), rc = T(0);
  auto fetch = [&](int64_t t0, int nv, bool with_dy) {
#pragma unroll
    for (int k = 0; k < kSt; ++k) {
      const int i = tid + 512 * k;     // [TC][64]
      const int r = i >> 6, c = i & 63;
      const bool ok = r < nv && d0 + c < D;
      const int64_t off = (b * L + t0 + r) * D + d0 + c;
      rx[k] = ok ? x[off] : T(0);
      rdt[k] = ok ? dt[off] : T(0);
      rdy[k] = (ok && with_dy) ? dy[off] : T(0);
    }
    if (tid < kSbTC * N) {
      const int r = tid / N, n = tid % N;
      const bool ok = r < nv;
      const int64_t off = (b * L + t0 + r) * N + n;
      rb = ok ? Bm[off] : T(0);
      rc = ok ? Cm[off] : T(0);
    }
  };
  auto put = [&]() {
#pragma unroll
    for (int k = 0; k < kSt; ++k) {
      const int i = tid + 512 * k;
      const int r = i >> 6, c = i & 63;
      sm.xs[r][c] = Io<T>::cvt(rx[k]);
      sm.dts[r][c] = Io<T>::cvt(rdt[k]);
      sm.dys[r][c] = Io<T>::cvt(rdy[k]);
    }
    if (tid < kSbTC * N) {
      const int r = tid / N, n = tid % N;
      sm.Bs[r][n] = Io<T>::cvt(rb);
      sm.Cs[r][n] = Io<T>::cvt(rc);
    }
  };
  auto chunk_len = [&](int64_t t0, int64_t tse) {
    return static_cast<int>((tse - t0) < kSbTC ? (tse - t0) : kSbTC);
  };
  if (a.nseg > 0) {
    const int64_t ts0 = (a.nseg - 1) * a.seg;
    fetch(ts0, chunk_len(ts0, (ts0 + a.seg < L) ? ts0 + a.seg : L), true);
  }

  for (int64_t s = a.nseg - 1; s >= 0; --s) {
    const int64_t ts0 = s * a.seg;
    const int64_t tse = (ts0 + a.seg < L) ? ts0 + a.seg : L;
    const int nch = static_cast<int>((tse - ts0 + kSbTC - 1) / kSbTC);
    float h[NPW];
#pragma unroll
    for (int j = 0; j < NPW; ++j)
      h[j] = okj[j] ? a.ckpt[((s * a.B + b) * D + d0 + lane) * N + n0 + j] : 0.f;

    // ---- forward over the segment: the state entering every chunk (the
    // last chunk's own steps are not needed; the staged registers hold this
    // segment's first chunk with dy, which the reverse pass uses if nch == 1)
    for (int c = 0; c < nch - 1; ++c) {
      const int64_t t0 = ts0 + static_cast<int64_t>(c) * kSbTC;
#pragma unroll
      for (int j = 0; j < NPW; ++j) sub_at(c, j) = h[j];
      put();
      __syncthreads();
      {
        // next: chunk c + 1, or the segment's last chunk (with dy) for the reverse pass
        const int64_t tn = c + 2 < nch ? t0 + kSbTC : ts0 + static_cast<int64_t>(nch - 1) * kSbTC;
        fetch(tn, chunk_len(tn, tse), c + 2 >= nch);
      }
#pragma unroll
      for (int i = 0; i < kSbTC; ++i) {
        const float xv = sm.xs[i][lane], dtv = sm.dts[i][lane];
#pragma unroll
        for (int j = 0; j < NPW; ++j) {
          if constexpr (FAST) {   // h = e (h + v) - v, v = B x / A
            const float e = fast_exp2(dtv * A2[j]);
            const float v = (sm.Bs[i][n0 + j] * xv) * iAv[j];
            h[j] = fmaf(e, h[j] + v, -v);
          } else {
            float e, phi;
            disc(dtv, j, e, phi);
            h[j] = fmaf(e, h[j], phi * sm.Bs[i][n0 + j] * xv);
          }
        }
      }
      __syncthreads();
    }
    if (nch > 0) {
#pragma unroll
      for (int j = 0; j < NPW; ++j) sub_at(nch - 1, j) = h[j];
    }

    // ---- chunks last to first
    for (int c = nch - 1; c >= 0; --c) {
      const int64_t t0 = ts0 + static_cast<int64_t>(c) * kSbTC;
      const int nv = chunk_len(t0, tse);
      // the state entering the chunk (this lane wrote it in the forward
      // pass); loaded before the barrier so its latency overlaps the staging
      float hin[NPW];
#pragma unroll
      for (int j = 0; j < NPW; ++j) hin[j] = sub_at(c, j);
      put();
      __syncthreads();
      if (c > 0) {
        fetch(t0 - kSbTC, kSbTC, true);
      } else if (s > 0) {   // the previous segment's first chunk (with dy, see above)
        const int64_t tp = (s - 1) * a.seg;
        fetch(tp, chunk_len(tp, ts0), true);
      }
      // this wave's states of the chunk -> LDS (read back by the same lanes)
      {
        float hh[NPW];
#pragma unroll
        for (int j = 0; j < NPW; ++j) hh[j] = hin[j];
#pragma unroll
        for (int i = 0; i < kSbTC; ++i) {
          const float xv = sm.xs[i][lane], dtv = sm.dts[i][lane];
#pragma unroll
          for (int j = 0; j < NPW; ++j) {
            float e, phi;
            disc(dtv, j, e, phi);
            hh[j] = fmaf(e, hh[j], phi * (sm.Bs[i][n0 + j] * xv));
            sm.hsl[w][i][j][lane] = hh[j];
          }
        }
      }
      constexpr int kUnroll = NPW == 2 ? 8 : (NPW == 4 ? 4 : 2);
#pragma unroll kUnroll
      for (int i = kSbTC - 1; i >= 0; --i) {
        const float xv = sm.xs[i][lane], dtv = sm.dts[i][lane], dyv = sm.dys[i][lane];
        float hsl_i[NPW];
#pragma unroll
        for (int j = 0; j < NPW; ++j) hsl_i[j] = sm.hsl[w][i][j][lane];
        float dxp = 0.f, ddtp = 0.f, v[2 * NPW];
#pragma unroll
        for (int j = 0; j < NPW; ++j) {
          const float Bv = sm.Bs[i][n0 + j], Cv = sm.Cs[i][n0 + j];
          float e, ph;
          disc(dtv, j, e, ph);
          const float ht = hsl_i[j];
          G[j] = fmaf(dyv, Cv, G[j]);        // dl/dh_t
          const float gphi = G[j] * ph;
          dxp = fmaf(gphi, Bv, dxp);
          v[j] = gphi * xv;                  // dB partial
          v[NPW + j] = ht * dyv;             // dC partial
          const float bx = Bv * xv;
          if constexpr (FAST) {
            // ddt term G (A h + B x); the dA term G (dt h + (dt - phi) B x / A)
            // is accumulated times A, as dt G (A h + B x) - phi G B x, which
            // reuses both products (the 1/A is applied once, after the sweep)
            const float u = G[j] * fmaf(Av[j], ht, bx);
            ddtp += u;
            dAacc[j] = fmaf(dtv, u, fmaf(-gphi, bx, dAacc[j]));
          } else {
            const float hp = i > 0 ? sm.hsl[w][i > 0 ? i - 1 : 0][j][lane] : hin[j];
            const float de = G[j] * hp;
            const float dphi = G[j] * bx;
            float dedt, dedA, dpdt, dpdA;
            sb_grads<DISC>(dtv, Av[j], iAv[j], e, ph, dedt, dedA, dpdt, dpdA);
            ddtp += fmaf(de, dedt, dphi * dpdt);
            dAacc[j] += fmaf(de, dedA, dphi * dpdA);
          }
          G[j] *= e;
        }
        // pairs of state indices: (dB, dB, dC, dC) of n0 + 2k, n0 + 2k + 1
#pragma unroll
        for (int k = 0; k < NPW / 2; ++k) {
          const float vk[4] = {v[2 * k], v[2 * k + 1], v[NPW + 2 * k], v[NPW + 2 * k + 1]};
          const float r = sum4_over_lanes(vk);
          if ((lane & 15) == 15) sm.rbc[i][lane >> 5][n0 + 2 * k + ((lane >> 4) & 1)] = r;
        }
        sm.hsl[w][i][0][lane] = dxp;   // h of token i is no longer needed
        sm.hsl[w][i][1][lane] = ddtp;
        if (w == 0) dDacc = fmaf(dyv, xv, dDacc);
      }
      __syncthreads();
      // sums over the waves -> dx, ddt; the chunk's dB, dC partials
#pragma unroll
      for (int k = 0; k < kSt; ++k) {
        const int i = tid + 512 * k;
        const int r = i >> 6, cc = i & 63;
        if (r < nv && d0 + cc < D) {
          float sx = 0.f, st = 0.f;
#pragma unroll
          for (int ww = 0; ww < kSbNW; ++ww) {
            sx += sm.hsl[ww][r][0][cc];
            st += sm.hsl[ww][r][1][cc];
          }
          const int64_t off = (b * L + t0 + r) * D + d0 + cc;
          Io<T>::store(dx + off, fmaf(Dd, sm.dys[r][cc], sx));   // cc == lane
          Io<T>::store(ddt + off, st);
        }
      }
      if (tid < kSbTC * N) {
        const int r = tid / N, n = tid % N;
        if (r < nv) {
          const int64_t off = ((tile * a.B + b) * L + t0 + r) * N + n;
          a.dBpart[off] = sm.rbc[r][0][n];
          a.dCpart[off] = sm.rbc[r][1][n];
        }
      }
      __syncthreads();
    }
  }
}

template <typename T, int DISC, int NPW>
__global__ __launch_bounds__(512) void selective_bwd_kernel(SelBwdArgs a) {
  constexpr int kSbTC = SbCfg<NPW>::TC, NN = SbCfg<NPW>::NN;
  __shared__ SbLds<NPW> sm;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int64_t tile = blockIdx.x % a.ntile;
  const int64_t b = blockIdx.x / a.ntile;
  const int64_t d = tile * kSbCT + lane;
  const bool dok = d < a.D;
  const int N = static_cast<int>(a.N);
  const int n0 = NPW * w;
  const int64_t D = a.D;

  float Av[NPW], iAv[NPW], G[NPW], dAacc[NPW];
  bool okj[NPW];
  bool small = false;
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    dAacc[j] = 0.f;
    okj[j] = dok && n0 + j < N;
    Av[j] = okj[j] ? a.A[d * N + n0 + j] : 0.f;
    iAv[j] = Av[j] != 0.f ? 1.f / Av[j] : 0.f;
    small |= okj[j] && fabsf(Av[j]) < 0.5f;
    G[j] = (okj[j] && a.dh_last != nullptr) ? a.dh_last[(b * D + d) * N + n0 + j] : 0.f;
  }
  float dDacc = 0.f;

  // B and C columns n >= N stay zero for the whole kernel
  for (int i = tid; i < kSbTC * NN; i += 512) {
    (&sm.Bs[0][0])[i] = 0.f;
    (&sm.Cs[0][0])[i] = 0.f;
  }
  // the choice is uniform over the workgroup: one flag per wave in the dB/dC
  // slots (first written after several more barriers); the barrier also
  // orders the zeros above
  float* flags = &sm.rbc[0][0][0];
  const bool wsmall = __builtin_amdgcn_ballot_w64(small) != 0;   // all lanes take part
  if (lane == 0) flags[w] = wsmall ? 1.f : 0.f;
  __syncthreads();
  bool precise = false;
#pragma unroll
  for (int ww = 0; ww < kSbNW; ++ww) precise |= flags[ww] != 0.f;
  // the closed-form gradients lose digits in (dt - phi)/A at small |dt A|
  // (as the forward's fast form does): fp32 I/O always takes the series
  if (DISC == kSbZoh && !precise && sizeof(T) == 2) {
    selective_bwd_body<T, DISC, true, NPW>(a, sm, b, tile, Av, iAv, okj, G, dAacc, dDacc);
#pragma unroll
    for (int j = 0; j < NPW; ++j) dAacc[j] *= iAv[j];   // accumulated times A (see the body)
  } else
    selective_bwd_body<T, DISC, false, NPW>(a, sm, b, tile, Av, iAv, okj, G, dAacc, dDacc);

#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    if (okj[j]) {
      const int64_t o = (b * D + d) * N + n0 + j;
      if (a.dh0 != nullptr) a.dh0[o] = G[j];
      a.dApart[o] = dAacc[j];
    }
  }
  if (w == 0 && dok) a.dDpart[b * D + d] = dDacc;
}

// Fixed-order sums: dB, dC over channel tiles; dA, dD over batch rows.
template <typename T>
__global__ __launch_bounds__(256) void selective_bwd_reduce_kernel(SelBwdArgs a) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t nbc = a.B * a.L * a.N;
  if (idx < nbc) {
    float sb = 0.f, sc = 0.f;
    for (int64_t t = 0; t < a.ntile; ++t) {
      sb += a.dBpart[t * nbc + idx];
      sc += a.dCpart[t * nbc + idx];
    }
    Io<T>::store(static_cast<T*>(a.dBm) + idx, sb);
    Io<T>::store(static_cast<T*>(a.dCm) + idx, sc);
    return;
  }
  const int64_t i2 = idx - nbc;
  const int64_t DN = a.D * a.N;
  if (i2 < DN) {
    float s = 0.f;
    for (int64_t bb = 0; bb < a.B; ++bb) s += a.dApart[bb * DN + i2];
    a.dA[i2] = s;
    return;
  }
  const int64_t i3 = i2 - DN;
  if (i3 < a.D && a.dD != nullptr) {
    float s = 0.f;
    for (int64_t bb = 0; bb < a.B; ++bb) s += a.dDpart[bb * a.D + i3];
    a.dD[i3] = s;
  }
}

// Empty sequence (B * L == 0): dA = dD = 0, dh0 = dh_last (or 0).
__global__ __launch_bounds__(256) void selective_bwd_empty_kernel(float* dA, float* dD, float* dh0,
                                                                  const float* dh_last, int64_t DN,
                                                                  int64_t D, int64_t nstate) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < DN) dA[i] = 0.f;
  if (dD != nullptr && i < D) dD[i] = 0.f;
  if (dh0 != nullptr && i < nstate) dh0[i] = dh_last != nullptr ? dh_last[i] : 0.f;
}

static inline int64_t sb_align(int64_t v) { return (v + 255) & ~int64_t(255); }

struct SbLayout { int64_t dB, dC, dA, dD, sub, total; };

static SbLayout sb_layout(int64_t B, int64_t L, int64_t D, int64_t N) {
  const int64_t nt = (D + kSbCT - 1) / kSbCT;
  SbLayout w;
  int64_t o = 0;
  w.dB = o; o = sb_align(o + nt * B * L * N * 4);
  w.dC = o; o = sb_align(o + nt * B * L * N * 4);
  w.dA = o; o = sb_align(o + B * D * N * 4);
  w.dD = o; o = sb_align(o + B * D * 4);
  const int64_t sub = N <= 2 * kSbNW ? SbCfg<2>::SUB * 2
                      : (N <= 4 * kSbNW ? SbCfg<4>::SUB * 4 : SbCfg<8>::SUB * 8);   // SUB x NPW
  w.sub = o; o = sb_align(o + B * nt * sub * kSbNW * kSbCT * 4);
  w.total = o;
  return w;
}

bool selective_bwd_supported(int64_t N, int64_t seg) {
  return N >= 1 && N <= 8 * kSbNW && seg >= 32 && seg <= 256 && seg % 32 == 0;
}

size_t selective_bwd_workspace(int64_t B, int64_t L, int64_t D, int64_t N) {
  if (B * L == 0) return 0;
  return static_cast<size_t>(sb_layout(B, L, D, N).total);
}

template <typename T>
hipError_t launch_selective_bwd(int disc, const void* x, const void* dt, const float* A,
                                const void* Bm, const void* Cm, const float* Dskip,
                                const float* ckpt, const void* dy, const float* dh_last, void* dx,
                                void* ddt, float* dA, void* dBm, void* dCm, float* dD, float* dh0,
                                void* ws, int64_t B, int64_t L, int64_t D, int64_t N, int64_t seg,
                                hipStream_t stream) {
  if (B * L == 0) {
    const int64_t n = (B * D * N > D * N) ? B * D * N : D * N;
    hipLaunchKernelGGL(selective_bwd_empty_kernel, dim3((n + 255) / 256 > 0 ? (n + 255) / 256 : 1),
                       dim3(256), 0, stream, dA, dD, dh0, dh_last, D * N, D, B * D * N);
    return hipGetLastError();
  }
  const SbLayout lay = sb_layout(B, L, D, N);
  char* base = static_cast<char*>(ws);
  SelBwdArgs a;
  a.x = x; a.dt = dt; a.A = A; a.Bm = Bm; a.Cm = Cm; a.Dskip = Dskip; a.ckpt = ckpt; a.dy = dy;
  a.dh_last = dh_last; a.dx = dx; a.ddt = ddt; a.dh0 = dh0;
  a.dBpart = reinterpret_cast<float*>(base + lay.dB);
  a.dCpart = reinterpret_cast<float*>(base + lay.dC);
  a.dApart = reinterpret_cast<float*>(base + lay.dA);
  a.dDpart = reinterpret_cast<float*>(base + lay.dD);
  a.subck = reinterpret_cast<float*>(base + lay.sub);
  a.dBm = dBm; a.dCm = dCm; a.dA = dA; a.dD = dD;
  a.B = B; a.L = L; a.D = D; a.N = N; a.seg = seg; a.nseg = (L + seg - 1) / seg;
  a.ntile = (D + kSbCT - 1) / kSbCT;
  const dim3 grid(static_cast<unsigned>(B * a.ntile));
  auto go = [&](auto npw) {
    constexpr int NPW = decltype(npw)::value;
    switch (disc) {
      case kSbEuler:
        hipLaunchKernelGGL((selective_bwd_kernel<T, kSbEuler, NPW>), grid, dim3(512), 0, stream, a);
        break;
      case kSbBilinear:
        hipLaunchKernelGGL((selective_bwd_kernel<T, kSbBilinear, NPW>), grid, dim3(512), 0, stream, a);
        break;
      case kSbDirac:
        hipLaunchKernelGGL((selective_bwd_kernel<T, kSbDirac, NPW>), grid, dim3(512), 0, stream, a);
        break;
      default:
        hipLaunchKernelGGL((selective_bwd_kernel<T, kSbZoh, NPW>), grid, dim3(512), 0, stream, a);
    }
  };
  if (N <= 2 * kSbNW) go(std::integral_constant<int, 2>{});
  else if (N <= 4 * kSbNW) go(std::integral_constant<int, 4>{});
  else go(std::integral_constant<int, 8>{});
  const int64_t nred = B * L * N + D * N + D;
  hipLaunchKernelGGL(selective_bwd_reduce_kernel<T>, dim3((nred + 255) / 256), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template hipError_t launch_selective_bwd<float>(int, const void*, const void*, const float*,
                                                const void*, const void*, const float*,
                                                const float*, const void*, const float*, void*,
                                                void*, float*, void*, void*, float*, float*, void*,
                                                int64_t, int64_t, int64_t, int64_t, int64_t,
                                                hipStream_t);
template hipError_t launch_selective_bwd<uint16_t>(int, const void*, const void*, const float*,
                                                   const void*, const void*, const float*,
                                                   const float*, const void*, const float*, void*,
                                                   void*, float*, void*, void*, float*, float*,
                                                   void*, int64_t, int64_t, int64_t, int64_t,
                                                   int64_t, hipStream_t);

}  // namespace lr
