// rotlru.hip — rotational LRU: a complex-diagonal recurrence over channel
// pairs with a magnitude gate and a per-step rotation (one launch).
//
// ("mlx-recurrence" post, Apple Developer Forums thread 840535, rotlru_scan:
// state [B, D] as interleaved channel pairs.)  Pair i of the state is the
// complex number z = h[2i] + i h[2i+1] and
//     z_t = a_t z_{t-1} + w_t,   a_t = r_t (cos theta_t + i sin theta_t),
//     w_t = u_t[2i] + i u_t[2i+1]
// which is the recurrence of the diagonal scan with complex (a, b) and the
// same associative combine (a2, b2) o (a1, b1) = (a2 a1, a2 b1 + b2)
// (IBM Research blog "K-Search for MLX", section "A 20x faster prefill: the
// Mamba SSM kernel", combine equation), here with complex products.
//
// Work split as the diagonal scan: one workgroup owns 16 pairs of one batch
// row and walks the sequence in tiles of 512 steps; 1024 threads split a
// tile into 64 segments of 8 steps scanned sequentially per lane, one wave
// per pair combines the 64 segment aggregates with a DPP complex pair scan,
// and the carry between tiles stays in LDS.
#include "common.hpp"
#include "launch.hpp"

namespace lr {

constexpr int kRotCP = 16;          // pairs per workgroup
constexpr int kRotSeg = 8;          // steps per lane segment
constexpr int kRotThreads = 1024;
constexpr int kRotSegs = kRotThreads / kRotCP;   // 64
constexpr int kRotTile = kRotSegs * kRotSeg;     // 512 steps
// narrow tiles (few chains): pairs and threads per workgroup
constexpr int kRotNarrowCP = 4, kRotNarrowNT = 512;

struct cplx {
  float re, im;
};
__device__ __forceinline__ cplx cmul(cplx a, cplx b) {
  return {fmaf(a.re, b.re, -a.im * b.im), fmaf(a.re, b.im, a.im * b.re)};
}
__device__ __forceinline__ cplx cfma(cplx a, cplx b, cplx c) {   // a b + c
  return {fmaf(a.re, b.re, fmaf(-a.im, b.im, c.re)), fmaf(a.re, b.im, fmaf(a.im, b.re, c.im))};
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void cpair_step(cplx& a, cplx& b) {
  const cplx pa = {dpp_f<CTRL, ROW_MASK>(1.f, a.re), dpp_f<CTRL, ROW_MASK>(0.f, a.im)};
  const cplx pb = {dpp_f<CTRL, ROW_MASK>(0.f, b.re), dpp_f<CTRL, ROW_MASK>(0.f, b.im)};
  b = cfma(a, pb, b);
  a = cmul(a, pa);
}

// inclusive scan of complex (a, b) pairs over the 64 lanes (lane 0 earliest)
__device__ __forceinline__ void cwave_incl_pair_scan(cplx& a, cplx& b) {
  cpair_step<0x111, 0xf>(a, b);
  cpair_step<0x112, 0xf>(a, b);
  cpair_step<0x114, 0xf>(a, b);
  cpair_step<0x118, 0xf>(a, b);
  cpair_step<0x142, 0xa>(a, b);
  cpair_step<0x143, 0xc>(a, b);
}

template <typename T>
__global__ __launch_bounds__(kRotThreads) void rotlru_scan_kernel(
    const T* __restrict__ r, const T* __restrict__ theta, const T* __restrict__ u,
    const float* __restrict__ h0, T* __restrict__ h, float* __restrict__ h_last, int64_t L,
    int64_t Dp) {
  __shared__ cplx aggA[kRotSegs][kRotCP];
  __shared__ cplx aggB[kRotSegs][kRotCP];
  __shared__ cplx carry_in[kRotSegs][kRotCP];
  __shared__ cplx tile_carry[kRotCP];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int pr = lane & (kRotCP - 1);
  const int seg = wave * 4 + (lane >> 4);
  const int64_t ntile = (Dp + kRotCP - 1) / kRotCP;
  const int64_t bi = blockIdx.x / ntile;
  const int64_t p0 = (blockIdx.x % ntile) * kRotCP;
  const int64_t p = p0 + pr;
  const bool pok = p < Dp;
  const int64_t D = 2 * Dp;

  if (tid < kRotCP) {
    const int64_t pp = p0 + tid;
    tile_carry[tid] = (h0 != nullptr && pp < Dp) ? cplx{h0[bi * D + 2 * pp], h0[bi * D + 2 * pp + 1]}
                                                 : cplx{0.f, 0.f};
  }
  __syncthreads();

  for (int64_t t0 = 0; t0 < L; t0 += kRotTile) {
    const int64_t ts = t0 + static_cast<int64_t>(seg) * kRotSeg;
    const int nok = pok ? static_cast<int>(L - ts < kRotSeg ? (L - ts > 0 ? L - ts : 0) : kRotSeg) : 0;
    cplx Pv[kRotSeg], Hv[kRotSeg];
    {
      cplx P = {1.f, 0.f}, Hs = {0.f, 0.f};
#pragma unroll
      for (int i = 0; i < kRotSeg; ++i) {
        cplx a = {1.f, 0.f}, w = {0.f, 0.f};
        if (i < nok) {
          const int64_t rowp = (bi * L + ts + i) * Dp + p;
          const int64_t rowu = (bi * L + ts + i) * D + 2 * p;
          const float rv = Io<T>::load(r + rowp);
          float sn, cs;
          sincosf(Io<T>::load(theta + rowp), &sn, &cs);
          a = {rv * cs, rv * sn};
          w = {Io<T>::load(u + rowu), Io<T>::load(u + rowu + 1)};
        }
        Hs = cfma(a, Hs, w);
        P = cmul(a, P);
        Pv[i] = P;
        Hv[i] = Hs;
      }
      aggA[seg][pr] = P;
      aggB[seg][pr] = Hs;
    }
    __syncthreads();

    if (wave < kRotCP) {
      const int c = wave;
      cplx pa = aggA[lane][c], pb = aggB[lane][c];
      const cplx tc = tile_carry[c];
      cwave_incl_pair_scan(pa, pb);
      // exclusive prefix: the previous lane's pair (identity at lane 0)
      const cplx ea = {wave_shr1(pa.re, 1.f), wave_shr1(pa.im, 0.f)};
      const cplx eb = {wave_shr1(pb.re, 0.f), wave_shr1(pb.im, 0.f)};
      carry_in[lane][c] = cfma(ea, tc, eb);
      if (lane == 63) tile_carry[c] = cfma(pa, tc, pb);
    }
    __syncthreads();

    const cplx cin = carry_in[seg][pr];
#pragma unroll
    for (int i = 0; i < kRotSeg; ++i) {
      if (i < nok) {
        const cplx z = cfma(Pv[i], cin, Hv[i]);
        const int64_t rowu = (bi * L + ts + i) * D + 2 * p;
        Io<T>::store(h + rowu, z.re);
        Io<T>::store(h + rowu + 1, z.im);
      }
    }
  }
  __syncthreads();
  if (h_last != nullptr && tid < kRotCP) {
    const int64_t pp = p0 + tid;
    if (pp < Dp) {
      h_last[bi * D + 2 * pp] = tile_carry[tid].re;
      h_last[bi * D + 2 * pp + 1] = tile_carry[tid].im;
    }
  }
}

// ---------------------------------------------------------------------------
// Narrow tiles for problems with few chains (B * Dp small), as the diagonal
// scan's narrow kernel: CT pairs per workgroup instead of 16 and 1024-step
// tiles (NT threads: NSEG = NT / CT lane segments of SEG = 1024 / NSEG
// steps), so a sequence of up to 1024 tokens is one pass of one load, two
// barriers and one store.  Lane = CT * segment + pair: the CT pairs of a
// token are adjacent lanes.  Wave c joins the segments of pair c: lane l
// folds its NSEG / 64 consecutive segments, then the 64 lane totals go
// through the complex DPP pair scan.  A segment's inputs are all loaded
// (raw) before any is converted, so the loads are in flight together.
// ---------------------------------------------------------------------------
template <typename T, int CT, int NT>
__global__ __launch_bounds__(NT) void rotlru_scan_narrow_kernel(
    const T* __restrict__ r, const T* __restrict__ theta, const T* __restrict__ u,
    const float* __restrict__ h0, T* __restrict__ h, float* __restrict__ h_last, int64_t L,
    int64_t Dp) {
  constexpr int NSEG = NT / CT;          // lane segments per tile
  constexpr int SEG = 1024 / NSEG;       // steps per lane segment
  constexpr int TL = NSEG * SEG;         // 1024 steps per tile
  constexpr int SPL = NSEG / 64;         // segments per lane in the join
  static_assert(CT >= 2 && CT <= 8 && TL == 1024 && SPL >= 1 && CT <= NT / 64, "narrow tile shape");
  __shared__ cplx aggA[NSEG][CT];
  __shared__ cplx aggB[NSEG][CT];
  __shared__ cplx carry_in[NSEG][CT];
  __shared__ cplx tile_carry[CT];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int pc = tid % CT;
  const int seg = tid / CT;
  const int64_t ntile = (Dp + CT - 1) / CT;
  // consecutive tiles (channels sharing cache lines) on one XCD
  const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t bi = wid / ntile;
  const int64_t p0 = (wid % ntile) * CT;
  const int64_t p = p0 + pc;
  const bool pok = p < Dp;
  const int64_t D = 2 * Dp;

  if (tid < CT) {
    const int64_t pp = p0 + tid;
    tile_carry[tid] = (h0 != nullptr && pp < Dp) ? cplx{h0[bi * D + 2 * pp], h0[bi * D + 2 * pp + 1]}
                                                 : cplx{0.f, 0.f};
  }
  __syncthreads();

  for (int64_t t0 = 0; t0 < L; t0 += TL) {
    const int64_t ts = t0 + static_cast<int64_t>(seg) * SEG;
    const int nok = pok ? static_cast<int>(L - ts < SEG ? (L - ts > 0 ? L - ts : 0) : SEG) : 0;
    T rr[SEG], tr[SEG], ur[SEG], vr[SEG];
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
      const bool ok = i < nok;
      const int64_t rowp = (bi * L + ts + i) * Dp + p;
      const int64_t rowu = (bi * L + ts + i) * D + 2 * p;
      rr[i] = ok ? r[rowp] : T(0);
      tr[i] = ok ? theta[rowp] : T(0);
      ur[i] = ok ? u[rowu] : T(0);
      vr[i] = ok ? u[rowu + 1] : T(0);
    }
    // the segment from a zero state; steps past L are the identity (a = 1, w = 0)
    cplx Pv[SEG], Hv[SEG];
    {
      cplx P = {1.f, 0.f}, Hs = {0.f, 0.f};
#pragma unroll
      for (int i = 0; i < SEG; ++i) {
        float sn, cs;
        sincosf(Io<T>::cvt(tr[i]), &sn, &cs);
        const float rv = Io<T>::cvt(rr[i]);
        const bool ok = i < nok;
        const cplx a = {ok ? rv * cs : 1.f, ok ? rv * sn : 0.f};
        const cplx w = {Io<T>::cvt(ur[i]), Io<T>::cvt(vr[i])};
        Hs = cfma(a, Hs, w);
        P = cmul(a, P);
        Pv[i] = P;
        Hv[i] = Hs;
      }
      aggA[seg][pc] = P;
      aggB[seg][pc] = Hs;
    }
    __syncthreads();

    if (wave < CT) {
      const int c = wave;
      cplx pa[SPL], pb[SPL];
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        pa[j] = aggA[SPL * lane + j][c];
        pb[j] = aggB[SPL * lane + j][c];
      }
      // the lane's segments folded in order, then the scan across lanes
      cplx ta = pa[0], tb = pb[0];
#pragma unroll
      for (int j = 1; j < SPL; ++j) {
        tb = cfma(pa[j], tb, pb[j]);
        ta = cmul(pa[j], ta);
      }
      cplx ia = ta, ib = tb;
      cwave_incl_pair_scan(ia, ib);
      const cplx tc = tile_carry[c];
      // state entering the lane's first segment, then each following one
      const cplx ea = {wave_shr1(ia.re, 1.f), wave_shr1(ia.im, 0.f)};
      const cplx eb = {wave_shr1(ib.re, 0.f), wave_shr1(ib.im, 0.f)};
      cplx cin = cfma(ea, tc, eb);
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        carry_in[SPL * lane + j][c] = cin;
        cin = cfma(pa[j], cin, pb[j]);
      }
      if (lane == 63) tile_carry[c] = cfma(ia, tc, ib);
    }
    __syncthreads();

    const cplx cin = carry_in[seg][pc];
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
      if (i < nok) {
        const cplx z = cfma(Pv[i], cin, Hv[i]);
        const int64_t rowu = (bi * L + ts + i) * D + 2 * p;
        Io<T>::store(h + rowu, z.re);
        Io<T>::store(h + rowu + 1, z.im);
      }
    }
  }
  __syncthreads();
  if (h_last != nullptr && tid < CT) {
    const int64_t pp = p0 + tid;
    if (pp < Dp) {
      h_last[bi * D + 2 * pp] = tile_carry[tid].re;
      h_last[bi * D + 2 * pp + 1] = tile_carry[tid].im;
    }
  }
}

// Wide variant for problems that still fill the chip with 32 pairs per
// workgroup: PPL = 2 adjacent pairs per lane, so the u and h accesses are 16
// bytes (8 for bf16) and r, theta 8 bytes.  Segments hold 4 steps (tiles of
// 256), so a lane keeps as many running products and states as the narrow
// kernel above (which stays faster for small, latency-bound problems).
template <typename T, int N>
__device__ __forceinline__ void rvload(const T* p, float (&v)[N]) {
  if constexpr (N == 1) {
    v[0] = Io<T>::load(p);
  } else if constexpr (sizeof(T) == 4) {
    if constexpr (N == 2) {
      const float2 x = *reinterpret_cast<const float2*>(p);
      v[0] = x.x; v[1] = x.y;
    } else {
      const float4 x = *reinterpret_cast<const float4*>(p);
      v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    }
  } else {
    if constexpr (N == 2) {
      const uint32_t x = *reinterpret_cast<const uint32_t*>(p);
      v[0] = bf2f(static_cast<uint16_t>(x)); v[1] = bf2f(static_cast<uint16_t>(x >> 16));
    } else {
      const uint2 x = *reinterpret_cast<const uint2*>(p);
      v[0] = bf2f(static_cast<uint16_t>(x.x)); v[1] = bf2f(static_cast<uint16_t>(x.x >> 16));
      v[2] = bf2f(static_cast<uint16_t>(x.y)); v[3] = bf2f(static_cast<uint16_t>(x.y >> 16));
    }
  }
}
template <typename T, int N>
__device__ __forceinline__ void rvstore(T* p, const float (&v)[N]) {
  if constexpr (sizeof(T) == 4) {
    if constexpr (N == 2) *reinterpret_cast<float2*>(p) = float2{v[0], v[1]};
    else *reinterpret_cast<float4*>(p) = float4{v[0], v[1], v[2], v[3]};
  } else {
    if constexpr (N == 2) {
      *reinterpret_cast<uint32_t*>(p) = f2bf(v[0]) | (static_cast<uint32_t>(f2bf(v[1])) << 16);
    } else {
      *reinterpret_cast<uint2*>(p) =
          uint2{f2bf(v[0]) | (static_cast<uint32_t>(f2bf(v[1])) << 16),
                f2bf(v[2]) | (static_cast<uint32_t>(f2bf(v[3])) << 16)};
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kRotThreads) void rotlru_scan_wide_kernel(
    const T* __restrict__ r, const T* __restrict__ theta, const T* __restrict__ u,
    const float* __restrict__ h0, T* __restrict__ h, float* __restrict__ h_last, int64_t L,
    int64_t Dp) {
  constexpr int PPL = 2;             // pairs per lane
  constexpr int CP = kRotCP * PPL;   // pairs per workgroup
  constexpr int SEG = kRotSeg / PPL;  // steps per lane segment (same registers)
  constexpr int TILE = kRotSegs * SEG;
  __shared__ cplx aggA[kRotSegs][CP];
  __shared__ cplx aggB[kRotSegs][CP];
  __shared__ cplx carry_in[kRotSegs][CP];
  __shared__ cplx tile_carry[CP];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int pr = (lane & (kRotCP - 1)) * PPL;   // first of this lane's pairs
  const int seg = wave * 4 + (lane >> 4);
  const int64_t ntile = (Dp + CP - 1) / CP;
  const int64_t bi = blockIdx.x / ntile;
  const int64_t p0 = (blockIdx.x % ntile) * CP;
  const int64_t p = p0 + pr;
  const bool pok = p < Dp;   // Dp % PPL == 0: all PPL pairs exist
  const int64_t D = 2 * Dp;

  for (int c = tid; c < CP; c += kRotThreads) {
    const int64_t pp = p0 + c;
    tile_carry[c] = (h0 != nullptr && pp < Dp) ? cplx{h0[bi * D + 2 * pp], h0[bi * D + 2 * pp + 1]}
                                               : cplx{0.f, 0.f};
  }
  __syncthreads();

  for (int64_t t0 = 0; t0 < L; t0 += TILE) {
    const int64_t ts = t0 + static_cast<int64_t>(seg) * SEG;
    const int nok = pok ? static_cast<int>(L - ts < SEG ? (L - ts > 0 ? L - ts : 0) : SEG) : 0;
    cplx Pv[SEG][PPL], Hv[SEG][PPL];
    {
      cplx P[PPL], Hs[PPL];
#pragma unroll
      for (int k = 0; k < PPL; ++k) { P[k] = {1.f, 0.f}; Hs[k] = {0.f, 0.f}; }
      // loads are unconditional, from a clamped token and pair (always in
      // bounds, L > 0 here), and steps past the end take the identity: no
      // branch around a load, so all of a segment's loads are in flight at once
      const int64_t pc = pok ? p : Dp - PPL;
      // bf16: every load of the segment issued raw, converted afterwards
      // (fp32 measured faster with each step's loads next to its use)
      constexpr bool kPre = sizeof(T) == 2;
      VRaw<T, PPL> rr[SEG], tr[SEG];
      VRaw<T, 2 * PPL> ur[SEG];
      if constexpr (kPre) {
#pragma unroll
        for (int i = 0; i < SEG; ++i) {
          const int64_t tc = ts + i < L ? ts + i : L - 1;
          const int64_t rowp = (bi * L + tc) * Dp + pc;
          rr[i] = vload_raw<T, PPL>(r + rowp);
          tr[i] = vload_raw<T, PPL>(theta + rowp);
          ur[i] = vload_raw<T, 2 * PPL>(u + 2 * rowp);
        }
      }
#pragma unroll
      for (int i = 0; i < SEG; ++i) {
        float rv[PPL], tv[PPL], uv[2 * PPL];
        if constexpr (kPre) {
          vcvt<T, PPL>(rr[i], rv);
          vcvt<T, PPL>(tr[i], tv);
          vcvt<T, 2 * PPL>(ur[i], uv);
        } else {
          const int64_t tc = ts + i < L ? ts + i : L - 1;
          const int64_t rowp = (bi * L + tc) * Dp + pc;
          rvload<T, PPL>(r + rowp, rv);
          rvload<T, PPL>(theta + rowp, tv);
          rvload<T, 2 * PPL>(u + 2 * rowp, uv);
        }
        const bool ok = i < nok;
#pragma unroll
        for (int k = 0; k < PPL; ++k) {
          float sn, cs;
          sincosf(tv[k], &sn, &cs);
          const cplx a = ok ? cplx{rv[k] * cs, rv[k] * sn} : cplx{1.f, 0.f};
          const cplx w = ok ? cplx{uv[2 * k], uv[2 * k + 1]} : cplx{0.f, 0.f};
          Hs[k] = cfma(a, Hs[k], w);
          P[k] = cmul(a, P[k]);
          Pv[i][k] = P[k];
          Hv[i][k] = Hs[k];
        }
      }
#pragma unroll
      for (int k = 0; k < PPL; ++k) {
        aggA[seg][pr + k] = P[k];
        aggB[seg][pr + k] = Hs[k];
      }
    }
    __syncthreads();

    // one wave per pair (PPL pairs per wave): lane = segment index
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
      const int c = wave + kRotCP * k;
      cplx pa = aggA[lane][c], pb = aggB[lane][c];
      const cplx tc = tile_carry[c];
      cwave_incl_pair_scan(pa, pb);
      // exclusive prefix: the previous lane's pair (identity at lane 0)
      const cplx ea = {wave_shr1(pa.re, 1.f), wave_shr1(pa.im, 0.f)};
      const cplx eb = {wave_shr1(pb.re, 0.f), wave_shr1(pb.im, 0.f)};
      carry_in[lane][c] = cfma(ea, tc, eb);
      if (lane == 63) tile_carry[c] = cfma(pa, tc, pb);
    }
    __syncthreads();

    cplx cin[PPL];
#pragma unroll
    for (int k = 0; k < PPL; ++k) cin[k] = carry_in[seg][pr + k];
    // element offset of this lane's first output, formed after the barrier
    // so that per-step addresses are not kept live across it
    int64_t offu = (bi * L + ts) * D + 2 * p;
    asm volatile("" : "+v"(offu));
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
      if (i < nok) {
        float o[2 * PPL];
#pragma unroll
        for (int k = 0; k < PPL; ++k) {
          const cplx z = cfma(Pv[i][k], cin[k], Hv[i][k]);
          o[2 * k] = z.re;
          o[2 * k + 1] = z.im;
        }
        rvstore<T, 2 * PPL>(h + offu + i * D, o);
      }
    }
  }
  __syncthreads();
  if (h_last != nullptr) {
    for (int c = tid; c < CP; c += kRotThreads) {
      const int64_t pp = p0 + c;
      if (pp < Dp) {
        h_last[bi * D + 2 * pp] = tile_carry[c].re;
        h_last[bi * D + 2 * pp + 1] = tile_carry[c].im;
      }
    }
  }
}

// Backward of the rotational LRU for the loss sum_t <dh_t, h_t> + <dh_last, h_last>
// (real inner products over the interleaved pairs).  In complex form, with
// G_t the gradient of the loss with respect to z_t (real part + i imaginary
// part), the adjoint runs the same recurrence backwards in time with the
// conjugate coefficient:
//     G_{L-1} = dh_{L-1} + dh_last,   G_t = conj(a_{t+1}) G_{t+1} + dh_t,
// so it is scanned with the same combine over reversed steps.  Each step then
// gives du_t = G_t and, with q = G_t conj(e^{i theta_t} z_{t-1}) (z_{-1} = h0),
// dr_t = Re q and dtheta_t = r_t Im q; dh0 = conj(a_0) G_0.  The forward
// already wrote every state, so nothing is recomputed.  Work split as the
// forward: 16 pairs per workgroup, 64 segments of 8 reversed steps per tile.
template <typename T>
__global__ __launch_bounds__(kRotThreads) void rotlru_scan_bwd_kernel(
    const T* __restrict__ r, const T* __restrict__ theta, const T* __restrict__ h,
    const float* __restrict__ h0, const T* __restrict__ dh, const float* __restrict__ dh_last,
    T* __restrict__ dr, T* __restrict__ dtheta, T* __restrict__ du, float* __restrict__ dh0,
    int64_t L, int64_t Dp) {
  __shared__ cplx aggA[kRotSegs][kRotCP];
  __shared__ cplx aggB[kRotSegs][kRotCP];
  __shared__ cplx carry_in[kRotSegs][kRotCP];
  __shared__ cplx tile_carry[kRotCP];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int pr = lane & (kRotCP - 1);
  const int seg = wave * 4 + (lane >> 4);
  const int64_t ntile = (Dp + kRotCP - 1) / kRotCP;
  const int64_t bi = blockIdx.x / ntile;
  const int64_t p0 = (blockIdx.x % ntile) * kRotCP;
  const int64_t p = p0 + pr;
  const bool pok = p < Dp;
  const int64_t D = 2 * Dp;

  if (tid < kRotCP) {
    const int64_t pp = p0 + tid;
    tile_carry[tid] = (dh_last != nullptr && pp < Dp)
                          ? cplx{dh_last[bi * D + 2 * pp], dh_last[bi * D + 2 * pp + 1]}
                          : cplx{0.f, 0.f};
  }
  __syncthreads();

  const int64_t row = bi * L;  // token offset of this batch row
  for (int64_t u0 = 0; u0 < L; u0 += kRotTile) {
    const int64_t us = u0 + static_cast<int64_t>(seg) * kRotSeg;
    // reversed steps u = us + i are tokens t = t_first - i (descending)
    const int64_t t_first = L - 1 - us;
    const int nok = pok ? static_cast<int>(L - us < kRotSeg ? (L - us > 0 ? L - us : 0) : kRotSeg) : 0;
    // gate and unit rotation of tokens t_first + 1 - j, j = 0..kRotSeg: entry j
    // is the coefficient of reversed step j (conjugated) and, for j >= 1, the
    // rotation of the output of step j - 1 (whose gate is reloaded there, an
    // L2 hit, to keep the register count down); identity where there is no token
    cplx ev[kRotSeg + 1];
    float rv[kRotSeg + 1];
#pragma unroll
    for (int j = 0; j <= kRotSeg; ++j) {
      const int64_t tj = t_first + 1 - j;
      const bool ok = j == 0 ? (nok > 0 && tj < L) : (j - 1 < nok);
      ev[j] = {1.f, 0.f};
      rv[j] = 1.f;
      if (ok) {
        const int64_t rowp = (row + tj) * Dp + p;
        rv[j] = Io<T>::load(r + rowp);
        float sn, cs;
        sincosf(Io<T>::load(theta + rowp), &sn, &cs);
        ev[j] = {cs, sn};
      }
    }
    cplx Pv[kRotSeg], Hv[kRotSeg];
    {
      cplx P = {1.f, 0.f}, Gs = {0.f, 0.f};
#pragma unroll
      for (int i = 0; i < kRotSeg; ++i) {
        cplx a = {1.f, 0.f}, w = {0.f, 0.f};
        if (i < nok) {
          a = {rv[i] * ev[i].re, -rv[i] * ev[i].im};
          const int64_t rowu = (row + t_first - i) * D + 2 * p;
          w = {Io<T>::load(dh + rowu), Io<T>::load(dh + rowu + 1)};
        }
        Gs = cfma(a, Gs, w);
        P = cmul(a, P);
        Pv[i] = P;
        Hv[i] = Gs;
      }
      aggA[seg][pr] = P;
      aggB[seg][pr] = Gs;
    }
    __syncthreads();

    if (wave < kRotCP) {
      const int c = wave;
      cplx pa = aggA[lane][c], pb = aggB[lane][c];
      const cplx tc = tile_carry[c];
      cwave_incl_pair_scan(pa, pb);
      const cplx ea = {wave_shr1(pa.re, 1.f), wave_shr1(pa.im, 0.f)};
      const cplx eb = {wave_shr1(pb.re, 0.f), wave_shr1(pb.im, 0.f)};
      carry_in[lane][c] = cfma(ea, tc, eb);
      if (lane == 63) tile_carry[c] = cfma(pa, tc, pb);
    }
    __syncthreads();

    const cplx cin = carry_in[seg][pr];
    // element offsets of token t_first, passed through an empty asm so that the
    // per-step addresses are formed here rather than kept live from the loads
    // before the barrier (which spilled them)
    int64_t offu = (row + t_first) * D + 2 * p, offp = (row + t_first) * Dp + p;
    asm volatile("" : "+v"(offu), "+v"(offp));
#pragma unroll
    for (int i = 0; i < kRotSeg; ++i) {
      if (i < nok) {
        const int64_t t = t_first - i;
        const cplx g = cfma(Pv[i], cin, Hv[i]);
        cplx zp;
        const int64_t rowu = offu - i * D;
        const int64_t rowp = offp - i * Dp;
        if (t > 0) {
          const int64_t rowq = rowu - D;
          zp = {Io<T>::load(h + rowq), Io<T>::load(h + rowq + 1)};
        } else {
          zp = h0 != nullptr ? cplx{h0[bi * D + 2 * p], h0[bi * D + 2 * p + 1]} : cplx{0.f, 0.f};
        }
        // q = g conj(e z_prev) with e = ev[i + 1] the rotation of token t
        const cplx ez = cmul(ev[i + 1], zp);
        const float qre = fmaf(g.re, ez.re, g.im * ez.im);
        const float qim = fmaf(g.im, ez.re, -g.re * ez.im);
        Io<T>::store(dr + rowp, qre);
        Io<T>::store(dtheta + rowp, Io<T>::load(r + rowp) * qim);
        Io<T>::store(du + rowu, g.re);
        Io<T>::store(du + rowu + 1, g.im);
      }
    }
  }
  __syncthreads();
  if (dh0 != nullptr && tid < kRotCP) {
    const int64_t pp = p0 + tid;
    if (pp < Dp) {
      cplx g = tile_carry[tid];
      if (L > 0) {
        const float r0 = Io<T>::load(r + row * Dp + pp);
        float sn, cs;
        sincosf(Io<T>::load(theta + row * Dp + pp), &sn, &cs);
        g = cmul({r0 * cs, -r0 * sn}, g);
      }
      dh0[bi * D + 2 * pp] = g.re;
      dh0[bi * D + 2 * pp + 1] = g.im;
    }
  }
}

// Narrow tiles for the backward of problems with few chains, as
// rotlru_scan_narrow_kernel: CT pairs per workgroup, 1024-step tiles of NSEG
// lane segments of SEG reversed steps, joined per pair by one wave.
template <typename T, int CT, int NT>
__global__ __launch_bounds__(NT) void rotlru_scan_bwd_narrow_kernel(
    const T* __restrict__ r, const T* __restrict__ theta, const T* __restrict__ h,
    const float* __restrict__ h0, const T* __restrict__ dh, const float* __restrict__ dh_last,
    T* __restrict__ dr, T* __restrict__ dtheta, T* __restrict__ du, float* __restrict__ dh0,
    int64_t L, int64_t Dp) {
  constexpr int NSEG = NT / CT;          // lane segments per tile
  constexpr int SEG = 1024 / NSEG;       // reversed steps per lane segment
  constexpr int TL = NSEG * SEG;         // 1024 steps per tile
  constexpr int SPL = NSEG / 64;         // segments per lane in the join
  static_assert(CT >= 2 && CT <= 8 && TL == 1024 && SPL >= 1 && CT <= NT / 64, "narrow tile shape");
  __shared__ cplx aggA[NSEG][CT];
  __shared__ cplx aggB[NSEG][CT];
  __shared__ cplx carry_in[NSEG][CT];
  __shared__ cplx tile_carry[CT];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int pr = tid % CT;
  const int seg = tid / CT;
  const int64_t ntile = (Dp + CT - 1) / CT;
  // consecutive tiles (channels sharing cache lines) on one XCD
  const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t bi = wid / ntile;
  const int64_t p0 = (wid % ntile) * CT;
  const int64_t p = p0 + pr;
  const bool pok = p < Dp;
  const int64_t D = 2 * Dp;

  if (tid < CT) {
    const int64_t pp = p0 + tid;
    tile_carry[tid] = (dh_last != nullptr && pp < Dp)
                          ? cplx{dh_last[bi * D + 2 * pp], dh_last[bi * D + 2 * pp + 1]}
                          : cplx{0.f, 0.f};
  }
  __syncthreads();

  const int64_t row = bi * L;  // token offset of this batch row
  for (int64_t u0 = 0; u0 < L; u0 += TL) {
    const int64_t us = u0 + static_cast<int64_t>(seg) * SEG;
    // reversed steps u = us + i are tokens t = t_first - i (descending)
    const int64_t t_first = L - 1 - us;
    const int nok = pok ? static_cast<int>(L - us < SEG ? (L - us > 0 ? L - us : 0) : SEG) : 0;
    // gate and unit rotation of tokens t_first + 1 - j, j = 0..SEG: entry j
    // is the coefficient of reversed step j (conjugated) and, for j >= 1, the
    // gate and rotation of the output of step j - 1; identity where there is
    // no token.  All loads of the segment are issued raw before any is converted.
    T rr[SEG + 1], tr[SEG + 1], gr[SEG], gi[SEG];
    bool okj[SEG + 1];
#pragma unroll
    for (int j = 0; j <= SEG; ++j) {
      const int64_t tj = t_first + 1 - j;
      okj[j] = j == 0 ? (nok > 0 && tj < L) : (j - 1 < nok);
      const int64_t rowp = (row + tj) * Dp + p;
      rr[j] = okj[j] ? r[rowp] : T(0);
      tr[j] = okj[j] ? theta[rowp] : T(0);
      if (j < SEG) {
        const int64_t rowu = (row + t_first - j) * D + 2 * p;
        gr[j] = j < nok ? dh[rowu] : T(0);
        gi[j] = j < nok ? dh[rowu + 1] : T(0);
      }
    }
    cplx ev[SEG + 1];
    float rv[SEG + 1];
#pragma unroll
    for (int j = 0; j <= SEG; ++j) {
      float sn, cs;
      sincosf(Io<T>::cvt(tr[j]), &sn, &cs);
      ev[j] = {okj[j] ? cs : 1.f, okj[j] ? sn : 0.f};
      rv[j] = okj[j] ? Io<T>::cvt(rr[j]) : 1.f;
    }
    cplx Pv[SEG], Hv[SEG];
    {
      cplx P = {1.f, 0.f}, Gs = {0.f, 0.f};
#pragma unroll
      for (int i = 0; i < SEG; ++i) {
        const bool ok = i < nok;
        const cplx a = {ok ? rv[i] * ev[i].re : 1.f, ok ? -rv[i] * ev[i].im : 0.f};
        const cplx w = {Io<T>::cvt(gr[i]), Io<T>::cvt(gi[i])};
        Gs = cfma(a, Gs, w);
        P = cmul(a, P);
        Pv[i] = P;
        Hv[i] = Gs;
      }
      aggA[seg][pr] = P;
      aggB[seg][pr] = Gs;
    }
    __syncthreads();

    if (wave < CT) {
      const int c = wave;
      cplx pa[SPL], pb[SPL];
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        pa[j] = aggA[SPL * lane + j][c];
        pb[j] = aggB[SPL * lane + j][c];
      }
      cplx ta = pa[0], tb = pb[0];
#pragma unroll
      for (int j = 1; j < SPL; ++j) {
        tb = cfma(pa[j], tb, pb[j]);
        ta = cmul(pa[j], ta);
      }
      cplx ia = ta, ib = tb;
      cwave_incl_pair_scan(ia, ib);
      const cplx tc = tile_carry[c];
      const cplx ea = {wave_shr1(ia.re, 1.f), wave_shr1(ia.im, 0.f)};
      const cplx eb = {wave_shr1(ib.re, 0.f), wave_shr1(ib.im, 0.f)};
      cplx cin = cfma(ea, tc, eb);
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        carry_in[SPL * lane + j][c] = cin;
        cin = cfma(pa[j], cin, pb[j]);
      }
      if (lane == 63) tile_carry[c] = cfma(ia, tc, ib);
    }
    __syncthreads();

    const cplx cin = carry_in[seg][pr];
    // element offsets of token t_first, passed through an empty asm so that the
    // per-step addresses are formed here rather than kept live from the loads
    // before the barrier (which spilled them)
    int64_t offu = (row + t_first) * D + 2 * p, offp = (row + t_first) * Dp + p;
    asm volatile("" : "+v"(offu), "+v"(offp));
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
      if (i < nok) {
        const int64_t t = t_first - i;
        const cplx g = cfma(Pv[i], cin, Hv[i]);
        cplx zp;
        const int64_t rowu = offu - i * D;
        const int64_t rowp = offp - i * Dp;
        if (t > 0) {
          const int64_t rowq = rowu - D;
          zp = {Io<T>::load(h + rowq), Io<T>::load(h + rowq + 1)};
        } else {
          zp = h0 != nullptr ? cplx{h0[bi * D + 2 * p], h0[bi * D + 2 * p + 1]} : cplx{0.f, 0.f};
        }
        // q = g conj(e z_prev) with e = ev[i + 1] the rotation of token t
        const cplx ez = cmul(ev[i + 1], zp);
        const float qre = fmaf(g.re, ez.re, g.im * ez.im);
        const float qim = fmaf(g.im, ez.re, -g.re * ez.im);
        Io<T>::store(dr + rowp, qre);
        Io<T>::store(dtheta + rowp, rv[i + 1] * qim);
        Io<T>::store(du + rowu, g.re);
        Io<T>::store(du + rowu + 1, g.im);
      }
    }
  }
  __syncthreads();
  if (dh0 != nullptr && tid < CT) {
    const int64_t pp = p0 + tid;
    if (pp < Dp) {
      cplx g = tile_carry[tid];
      if (L > 0) {
        const float r0 = Io<T>::load(r + row * Dp + pp);
        float sn, cs;
        sincosf(Io<T>::load(theta + row * Dp + pp), &sn, &cs);
        g = cmul({r0 * cs, -r0 * sn}, g);
      }
      dh0[bi * D + 2 * pp] = g.re;
      dh0[bi * D + 2 * pp + 1] = g.im;
    }
  }
}

// Wide backward for the problems the wide forward serves: 2 adjacent pairs
// per lane (vector accesses), 4 reversed steps per segment.
template <typename T>
__global__ __launch_bounds__(kRotThreads) void rotlru_scan_bwd_wide_kernel(
    const T* __restrict__ r, const T* __restrict__ theta, const T* __restrict__ h,
    const float* __restrict__ h0, const T* __restrict__ dh, const float* __restrict__ dh_last,
    T* __restrict__ dr, T* __restrict__ dtheta, T* __restrict__ du, float* __restrict__ dh0,
    int64_t L, int64_t Dp) {
  constexpr int PPL = 2;
  constexpr int CP = kRotCP * PPL;
  constexpr int SEG = kRotSeg / PPL;
  constexpr int TILE = kRotSegs * SEG;
  __shared__ cplx aggA[kRotSegs][CP];
  __shared__ cplx aggB[kRotSegs][CP];
  __shared__ cplx carry_in[kRotSegs][CP];
  __shared__ cplx tile_carry[CP];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int pr = (lane & (kRotCP - 1)) * PPL;
  const int seg = wave * 4 + (lane >> 4);
  const int64_t ntile = (Dp + CP - 1) / CP;
  const int64_t bi = blockIdx.x / ntile;
  const int64_t p0 = (blockIdx.x % ntile) * CP;
  const int64_t p = p0 + pr;
  const bool pok = p < Dp;   // Dp % 2 == 0: both pairs exist
  const int64_t D = 2 * Dp;

  for (int c = tid; c < CP; c += kRotThreads) {
    const int64_t pp = p0 + c;
    tile_carry[c] = (dh_last != nullptr && pp < Dp)
                        ? cplx{dh_last[bi * D + 2 * pp], dh_last[bi * D + 2 * pp + 1]}
                        : cplx{0.f, 0.f};
  }
  __syncthreads();

  const int64_t row = bi * L;
  for (int64_t u0 = 0; u0 < L; u0 += TILE) {
    const int64_t us = u0 + static_cast<int64_t>(seg) * SEG;
    const int64_t t_first = L - 1 - us;
    const int nok = pok ? static_cast<int>(L - us < SEG ? (L - us > 0 ? L - us : 0) : SEG) : 0;
    // as the narrow kernel: entry j is token t_first + 1 - j
    cplx ev[SEG + 1][PPL];
    float rv[SEG + 1][PPL];
#pragma unroll
    for (int j = 0; j <= SEG; ++j) {
      const int64_t tj = t_first + 1 - j;
      const bool ok = j == 0 ? (nok > 0 && tj < L) : (j - 1 < nok);
#pragma unroll
      for (int k = 0; k < PPL; ++k) { ev[j][k] = {1.f, 0.f}; rv[j][k] = 1.f; }
      if (ok) {
        const int64_t rowp = (row + tj) * Dp + p;
        float tv[PPL];
        rvload<T, PPL>(r + rowp, rv[j]);
        rvload<T, PPL>(theta + rowp, tv);
#pragma unroll
        for (int k = 0; k < PPL; ++k) {
          float sn, cs;
          sincosf(tv[k], &sn, &cs);
          ev[j][k] = {cs, sn};
        }
      }
    }
    cplx Pv[SEG][PPL], Hv[SEG][PPL];
    {
      cplx P[PPL], Gs[PPL];
#pragma unroll
      for (int k = 0; k < PPL; ++k) { P[k] = {1.f, 0.f}; Gs[k] = {0.f, 0.f}; }
#pragma unroll
      for (int i = 0; i < SEG; ++i) {
        float wv[2 * PPL];
        if (i < nok) {
          rvload<T, 2 * PPL>(dh + (row + t_first - i) * D + 2 * p, wv);
        }
#pragma unroll
        for (int k = 0; k < PPL; ++k) {
          cplx a = {1.f, 0.f}, w = {0.f, 0.f};
          if (i < nok) {
            a = {rv[i][k] * ev[i][k].re, -rv[i][k] * ev[i][k].im};
            w = {wv[2 * k], wv[2 * k + 1]};
          }
          Gs[k] = cfma(a, Gs[k], w);
          P[k] = cmul(a, P[k]);
          Pv[i][k] = P[k];
          Hv[i][k] = Gs[k];
        }
      }
#pragma unroll
      for (int k = 0; k < PPL; ++k) {
        aggA[seg][pr + k] = P[k];
        aggB[seg][pr + k] = Gs[k];
      }
    }
    __syncthreads();

#pragma unroll
    for (int k = 0; k < PPL; ++k) {
      const int c = wave + kRotCP * k;
      cplx pa = aggA[lane][c], pb = aggB[lane][c];
      const cplx tc = tile_carry[c];
      cwave_incl_pair_scan(pa, pb);
      const cplx ea = {wave_shr1(pa.re, 1.f), wave_shr1(pa.im, 0.f)};
      const cplx eb = {wave_shr1(pb.re, 0.f), wave_shr1(pb.im, 0.f)};
      carry_in[lane][c] = cfma(ea, tc, eb);
      if (lane == 63) tile_carry[c] = cfma(pa, tc, pb);
    }
    __syncthreads();

    cplx cin[PPL];
#pragma unroll
    for (int k = 0; k < PPL; ++k) cin[k] = carry_in[seg][pr + k];
    int64_t offu = (row + t_first) * D + 2 * p, offp = (row + t_first) * Dp + p;
    asm volatile("" : "+v"(offu), "+v"(offp));
#pragma unroll
    for (int i = 0; i < SEG; ++i) {
      if (i < nok) {
        const int64_t t = t_first - i;
        const int64_t rowu = offu - i * D;
        const int64_t rowp = offp - i * Dp;
        float zv[2 * PPL];
        if (t > 0) {
          rvload<T, 2 * PPL>(h + rowu - D, zv);
        } else {
#pragma unroll
          for (int k = 0; k < 2 * PPL; ++k) zv[k] = h0 != nullptr ? h0[bi * D + 2 * p + k] : 0.f;
        }
        float gv[2 * PPL], qr[PPL], qi[PPL];
#pragma unroll
        for (int k = 0; k < PPL; ++k) {
          const cplx g = cfma(Pv[i][k], cin[k], Hv[i][k]);
          const cplx ez = cmul(ev[i + 1][k], cplx{zv[2 * k], zv[2 * k + 1]});
          qr[k] = fmaf(g.re, ez.re, g.im * ez.im);
          qi[k] = fmaf(g.im, ez.re, -g.re * ez.im) * rv[i + 1][k];
          gv[2 * k] = g.re;
          gv[2 * k + 1] = g.im;
        }
        rvstore<T, PPL>(dr + rowp, qr);
        rvstore<T, PPL>(dtheta + rowp, qi);
        rvstore<T, 2 * PPL>(du + rowu, gv);
      }
    }
  }
  __syncthreads();
  if (dh0 != nullptr) {
    for (int c = tid; c < CP; c += kRotThreads) {
      const int64_t pp = p0 + c;
      if (pp < Dp) {
        cplx g = tile_carry[c];
        if (L > 0) {
          const float r0 = Io<T>::load(r + row * Dp + pp);
          float sn, cs;
          sincosf(Io<T>::load(theta + row * Dp + pp), &sn, &cs);
          g = cmul({r0 * cs, -r0 * sn}, g);
        }
        dh0[bi * D + 2 * pp] = g.re;
        dh0[bi * D + 2 * pp + 1] = g.im;
      }
    }
  }
}

template <typename T>
hipError_t launch_rotlru_scan_bwd(const void* r, const void* theta, const void* h,
                                  const float* h0, const void* dh, const float* dh_last, void* dr,
                                  void* dtheta, void* du, float* dh0, int64_t B, int64_t L,
                                  int64_t D, hipStream_t stream) {
  const int64_t Dp = D / 2;
  if (B * ((Dp + kRotCP - 1) / kRotCP) < 64) {   // few chains: narrow tiles
    dim3 grid(static_cast<unsigned>(B * ((Dp + kRotNarrowCP - 1) / kRotNarrowCP)));
    hipLaunchKernelGGL((rotlru_scan_bwd_narrow_kernel<T, kRotNarrowCP, kRotNarrowNT>), grid,
                       dim3(kRotNarrowNT), 0, stream, static_cast<const T*>(r),
                       static_cast<const T*>(theta), static_cast<const T*>(h), h0,
                       static_cast<const T*>(dh), dh_last, static_cast<T*>(dr),
                       static_cast<T*>(dtheta), static_cast<T*>(du), dh0, L, Dp);
    return hipGetLastError();
  }
  if (Dp % 2 == 0 && B * (Dp / 32) >= 512) {
    dim3 grid(static_cast<unsigned>(B * ((Dp + 2 * kRotCP - 1) / (2 * kRotCP))));
    hipLaunchKernelGGL(rotlru_scan_bwd_wide_kernel<T>, grid, dim3(kRotThreads), 0, stream,
                       static_cast<const T*>(r), static_cast<const T*>(theta),
                       static_cast<const T*>(h), h0, static_cast<const T*>(dh), dh_last,
                       static_cast<T*>(dr), static_cast<T*>(dtheta), static_cast<T*>(du), dh0, L,
                       Dp);
    return hipGetLastError();
  }
  dim3 grid(static_cast<unsigned>(B * ((Dp + kRotCP - 1) / kRotCP)));
  hipLaunchKernelGGL(rotlru_scan_bwd_kernel<T>, grid, dim3(kRotThreads), 0, stream,
                     static_cast<const T*>(r), static_cast<const T*>(theta),
                     static_cast<const T*>(h), h0, static_cast<const T*>(dh), dh_last,
                     static_cast<T*>(dr), static_cast<T*>(dtheta), static_cast<T*>(du), dh0, L,
                     Dp);
  return hipGetLastError();
}

template hipError_t launch_rotlru_scan_bwd<float>(const void*, const void*, const void*,
                                                  const float*, const void*, const float*, void*,
                                                  void*, void*, float*, int64_t, int64_t, int64_t,
                                                  hipStream_t);
template hipError_t launch_rotlru_scan_bwd<uint16_t>(const void*, const void*, const void*,
                                                     const float*, const void*, const float*,
                                                     void*, void*, void*, float*, int64_t,
                                                     int64_t, int64_t, hipStream_t);

template <typename T>
hipError_t launch_rotlru_scan(const void* r, const void* theta, const void* u, const float* h0,
                              void* h, float* h_last, int64_t B, int64_t L, int64_t D,
                              hipStream_t stream) {
  const int64_t Dp = D / 2;
  if (B * ((Dp + kRotCP - 1) / kRotCP) < 64) {   // few chains: narrow tiles
    dim3 grid(static_cast<unsigned>(B * ((Dp + kRotNarrowCP - 1) / kRotNarrowCP)));
    hipLaunchKernelGGL((rotlru_scan_narrow_kernel<T, kRotNarrowCP, kRotNarrowNT>), grid,
                       dim3(kRotNarrowNT), 0, stream, static_cast<const T*>(r),
                       static_cast<const T*>(theta), static_cast<const T*>(u), h0,
                       static_cast<T*>(h), h_last, L, Dp);
  } else if (Dp % 2 == 0 && B * (Dp / 32) >= 512) {
    dim3 grid(static_cast<unsigned>(B * ((Dp + 2 * kRotCP - 1) / (2 * kRotCP))));
    hipLaunchKernelGGL(rotlru_scan_wide_kernel<T>, grid, dim3(kRotThreads), 0, stream,
                       static_cast<const T*>(r), static_cast<const T*>(theta),
                       static_cast<const T*>(u), h0, static_cast<T*>(h), h_last, L, Dp);
  } else {
    dim3 grid(static_cast<unsigned>(B * ((Dp + kRotCP - 1) / kRotCP)));
    hipLaunchKernelGGL(rotlru_scan_kernel<T>, grid, dim3(kRotThreads), 0, stream,
                       static_cast<const T*>(r), static_cast<const T*>(theta),
                       static_cast<const T*>(u), h0, static_cast<T*>(h), h_last, L, Dp);
  }
  return hipGetLastError();
}

template hipError_t launch_rotlru_scan<float>(const void*, const void*, const void*, const float*,
                                              void*, float*, int64_t, int64_t, int64_t,
                                              hipStream_t);
template hipError_t launch_rotlru_scan<uint16_t>(const void*, const void*, const void*,
                                                 const float*, void*, float*, int64_t, int64_t,
                                                 int64_t, hipStream_t);

}  // namespace lr
