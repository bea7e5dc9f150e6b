// ssd_bwd.hip — backward of the Mamba-2 SSD scan with segment checkpoints.
//
// ("mlx-recurrence" post, Apple Developer Forums thread 840535: the training
// path keeps the state only at segment boundaries in the forward and
// recomputes inside each segment in the backward.)
//
// Loss l = sum(dy * y) + <dh_last, h_last>.  Per (b, h), with G_t = dl/dh_t:
//   G_t = e_{t+1} G_{t+1} + dy_t (x) C_t,  dx_t = phi_t G_t B_t + D dy_t,
//   dB_t += phi_t G_t^T x_t,  dC_t += h_t^T dy_t,  dphi_t = x_t^T G_t B_t,
//   d(log e_t) = <G_t, h_{t-1}> e_t,  dh0 = e_0 G_0.
// Evaluated per 64-token block on MFMA.  With c the inclusive cumulative
// log-decay inside the block, E_t = e^{c_t}, sE_t = e^{c_end - c_t} and the
// decayed causal masks
//   Mp[u][t] = (C_u . B_t) e^{c_u - c_t},  W[u][t] = (dy_u . x_t) e^{c_u - c_t}
// for u >= t, and Gamma the adjoint of the block's last state from later
// tokens and h_prev the state entering the block:
//   dx_t  = phi_t (sum_u Mp[u][t] dy_u + sE_t Gamma B_t) + D dy_t
//   dB_t += phi_t (sum_u W[u][t] C_u + sE_t Gamma^T x_t)
//   dC_u += sum_t W[u][t] phi_t B_t + E_u h_prev^T dy_u
//   Gamma_prev = E_end Gamma + sum_u E_u dy_u (x) C_u
// and the log-decay gradient follows from dl/dc_j (pairs (u, t) contribute
// T[u][t] = Mp phi_t (dy_u . x_t) with + to c_u and - to c_t; the entering
// state and Gamma add boundary terms) by a reverse prefix sum over the block.
//
// Launches:
//   gloc:     per (b, h, segment): Gamma_loc = adjoint of the segment's own
//             outputs w.r.t. its entering state, and the segment decay.
//   gcombine: per state element, backwards over segments,
//             Gamma_out(s-1) = Lambda_s Gamma_out(s) + Gamma_loc(s)
//             (the (a, b) combine again, run in reverse); also gives dh0.
//   main:     per (b, h, segment): recompute the block-entry states from the
//             checkpoint (kept in registers), then the blocks in reverse.
//             Writes dx, ddt and per-head partial sums of dB, dC (rounded to
//             bf16, the precision of the final dB, dC; this halves the
//             partial traffic), dA, dD (fp32).
//   reduce:   fixed-order fp32 sums of the partials over heads (and batch
//             and segments for dA, dD), so results are deterministic.
// The launches run per slice of batch rows (bounded workspace); from the
// second slice on, gloc shares one launch with the previous slice's dB, dC
// reduction (gloc_reduce), which overlaps the bandwidth-bound sums with the
// latency-bound gloc.
#include "common.hpp"
#include "launch.hpp"

namespace lr {

constexpr int kBQ = 64;          // tokens per block
constexpr int kBP = 64;          // head dim P (one 64-wide slice)
constexpr int kBLd = kBQ + 8;    // leading dim of 64-wide LDS tiles

// Recurrence kinds: SSD with ZOH or Euler discretisation, and GLA, which is
// the same recurrence with x <-> v, B <-> k, C <-> q, phi = 1 and the decay
// given directly as the gate g (log-decay ln g).  A GLA head of V columns is
// run as V / 64 "heads" of 64 columns that form one group sharing k and q.
enum { kBwdZoh = 0, kBwdEuler = 1, kBwdGla = 2, kBwdDirac = 3, kBwdBilinear = 4 };

struct BwdArgs {
  const uint16_t* x; const uint16_t* dt; const float* A; const uint16_t* Bm; const uint16_t* Cm;
  const float* Dskip; const float* ckpt; const uint16_t* dy; const float* dh_last;
  const float* h0;                // SSD: [B][H][P][N] or null; replaces ckpt[0] when given
  uint16_t* dx; uint16_t* ddt; float* dA; uint16_t* dBm; uint16_t* dCm; float* dD; float* dh0;
  uint16_t* dBpart; uint16_t* dCpart;   // [B][L][H][N] bf16 per-head partials (heads
                                        // innermost: the heads running together write
                                        // one contiguous run per token)
  float* gseg;                    // [nseg][B][H][P][N]: Gamma_loc, then Gamma_out
  float* lam;                     // [nseg][B][H]
  float* dApart; float* dDpart;   // [B][H][nseg]
  float* dgpart;                  // GLA: [B][L][H] log-gate gradient per 64-column slice
  uint16_t* dg;                   // GLA: [B][L][G] gate gradient
  int64_t B, L, H, G, N, seg, nseg;
  int64_t ckB;                    // batch size of ckpt ([nseg][ckB][H][P][N]), the whole
                                  // batch when the launches cover a slice of it
};

// Gate (SSD dt, GLA g) of token t of head h in group grp, as its raw bf16
// bits: the prefetches keep these, so that no conversion next to the load
// makes the wave wait for it.
template <int MODE>
__device__ __forceinline__ uint16_t gate_raw(const BwdArgs& a, int64_t b, int64_t t, int64_t h,
                                             int64_t grp) {
  return MODE == kBwdGla ? a.dt[(b * a.L + t) * a.G + grp] : a.dt[(b * a.L + t) * a.H + h];
}

// Offset of state element idx = ((b H + h) P + p) N + n of the internal
// [B][H][P][N] order in the caller's dh_last / dh0 layout: the same for SSD,
// [B][G][N][V] (V = 64 H / G) for GLA.
template <int MODE>
__device__ __forceinline__ int64_t state_off(const BwdArgs& a, int64_t idx) {
  if (MODE != kBwdGla) return idx;
  const int64_t PN = static_cast<int64_t>(64) * a.N;
  const int64_t bh = idx / PN, pn = idx % PN;
  const int64_t p = pn / a.N, n = pn % a.N;
  const int64_t b = bh / a.H, hh = bh % a.H;
  const int64_t hpg = a.H / a.G, grp = hh / hpg, vs = hh % hpg;
  return ((b * a.G + grp) * a.N + n) * (64 * hpg) + 64 * vs + p;
}

// Per-token scalars of one token: log2 decay, phi, e.  Masked tokens
// (ok == false) get no decay and no input.  For SSD the gate is dt; for GLA
// it is g itself.
template <int DISC>
__device__ __forceinline__ void block_scalars(float gate, bool ok, float Ah, float& l2, float& ph,
                                              float& ek) {
  if (DISC == kBwdGla) {
    ek = ok ? gate : 1.f;
    l2 = fast_log2(ek);
    ph = ok ? 1.f : 0.f;
    return;
  }
  const float dtv = ok ? gate : 0.f;
  const float lam = dtv * Ah;
  if (DISC == kBwdBilinear) {
    // e = (1 + l/2)/(1 - l/2), negative for l < -2: its magnitude goes into
    // the log2 sums and its sign into a parity scan (sign_scan)
    const float r = __builtin_amdgcn_rcpf(1.f - 0.5f * lam);
    ek = (1.f + 0.5f * lam) * r;
    l2 = fmaxf(fast_log2(fabsf(ek)), -126.f);
    ph = dtv * r;
    return;
  }
  l2 = lam * kLog2e;
  ek = fast_exp2(l2);
  if (DISC == kBwdDirac) {
    ph = ok ? 1.f : 0.f;
  } else if (DISC == kBwdEuler) {
    ph = dtv;
  } else {
    const float ser = dtv * fmaf(lam, fmaf(lam, fmaf(lam, 1.f / 24.f, 1.f / 6.f), 0.5f), 1.f);
    ph = fabsf(lam) < 0.1f ? ser : (ek - 1.f) / Ah;
  }
}

// Bilinear only (else both signs are 1): sgc = sign of the decay product
// from the block start through token `lane` (parity of the negative decays),
// sge = the same over the whole block.
template <int DISC>
__device__ __forceinline__ void sign_scan(float ek, float& sgc, float& sge) {
  sgc = 1.f;
  sge = 1.f;
  if constexpr (DISC == kBwdBilinear) {
    const float nneg = wave_incl_sum(ek < 0.f ? 1.f : 0.f);
    sgc = (static_cast<int>(nneg) & 1) ? -1.f : 1.f;
    sge = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sgc), 63));
  }
}

// Sum over the 16 lanes of a DPP row (lanes with the same l / 16): an
// inclusive row scan, so the total lands in the row's last lane (l % 16 == 15).
__device__ __forceinline__ float row16_sum_last(float v) {
  v += dpp_f<0x111, 0xf>(0.f, v);   // row_shr:1
  v += dpp_f<0x112, 0xf>(0.f, v);   // row_shr:2
  v += dpp_f<0x114, 0xf>(0.f, v);   // row_shr:4
  v += dpp_f<0x118, 0xf>(0.f, v);   // row_shr:8
  return v;
}
// Sum over the 4 lanes l % 16 == c (the 4 rows of a wave), in all of them:
// gfx950's permlane16_swap pairs rows (0, 1) and (2, 3), permlane32_swap the
// two halves.
__device__ __forceinline__ float col4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Sum over the wave, the same in every lane.
__device__ __forceinline__ float wave_sum(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_incl_sum(v)), 63));
}

// ---------------------------------------------------------------------------
// gloc: Gamma_loc(s) = sum_u E_u dy_u (x) C_u over the segment (E from the
// segment start), accumulated block by block backwards; Lambda_s = E_end.
// ---------------------------------------------------------------------------
template <int NS>
struct GlocLds {
  uint16_t Cs[kBQ * (NS + 8)]; // C[u][n]
  uint16_t dyE[kBQ * kBLd];    // E_u dy[u][p]
};

// Per segment, last block first.  A block's C, dy and gates are loaded into
// registers one block ahead (in flight during the previous block's MFMA);
// every wave scans the block's gates itself (lane = token), so dy is scaled
// by E_u while it is written to LDS, with no extra pass or barrier.
template <int MODE, int NS>
__device__ __forceinline__ void gloc_body(const BwdArgs& a, int64_t wid) {
  constexpr int NT = NS / 16;
  constexpr int kCC = kBQ * (NS / 8) / 256;    // 16-byte C chunks per thread
  constexpr int kDC = kBQ * (kBP / 8) / 256;   // 16-byte dy chunks per thread
  __shared__ GlocLds<NS> sm;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int g4 = lane >> 4, c16 = lane & 15;
  // heads vary fastest: the workgroups that run together on an XCD are the
  // heads of one (batch row, segment), which read the same B and C rows
  // (groups shared by heads), so those come from the XCD's L2
  const int64_t h = wid % a.H;
  const int64_t sg = (wid / a.H) % a.nseg;
  const int64_t b = wid / (a.H * a.nseg);
  const int64_t grp = h / (a.H / a.G);
  const float Ah = MODE == kBwdGla ? 0.f : a.A[h];
  const int64_t ts0 = sg * a.seg;
  const int64_t tse = (ts0 + a.seg < a.L) ? ts0 + a.seg : a.L;
  const int nb = static_cast<int>((tse - ts0 + kBQ - 1) / kBQ);

  u16x8 creg[kCC], dreg[kDC];
  uint16_t gv = 0;   // gate of token `lane` of the block (raw bf16: no wait at the load)
  auto fetch = [&](int j) {
    const int64_t t0 = ts0 + static_cast<int64_t>(j) * kBQ;
    const int nv = static_cast<int>((tse - t0) < kBQ ? (tse - t0) : kBQ);
#pragma unroll
    for (int k = 0; k < kCC; ++k) {
      const int idx = tid + 256 * k, u = idx / (NS / 8), c = idx % (NS / 8);
      creg[k] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (u < nv) creg[k] = *reinterpret_cast<const u16x8*>(a.Cm + ((b * a.L + t0 + u) * a.G + grp) * NS + 8 * c);
    }
#pragma unroll
    for (int k = 0; k < kDC; ++k) {
      const int idx = tid + 256 * k, u = idx >> 3, c = idx & 7;
      dreg[k] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (u < nv) dreg[k] = *reinterpret_cast<const u16x8*>(a.dy + ((b * a.L + t0 + u) * a.H + h) * kBP + 8 * c);
    }
    gv = lane < nv ? gate_raw<MODE>(a, b, t0 + lane, h, grp) : uint16_t(0);
  };

  f32x4 gacc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) gacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;   // log2 of the segment decay's magnitude
  float ssign = 1.f;  // and its sign

  if (nb > 0) fetch(nb - 1);
  for (int j = nb - 1; j >= 0; --j) {
    const int64_t t0 = ts0 + static_cast<int64_t>(j) * kBQ;
    const int nv = static_cast<int>((tse - t0) < kBQ ? (tse - t0) : kBQ);
    float l2, ph, ek;
    block_scalars<MODE>(bf2f(gv), lane < nv, Ah, l2, ph, ek);
    float sgc, sge;
    sign_scan<MODE>(ek, sgc, sge);
    const float c = wave_incl_sum(l2);
    const float cend = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), 63));
    const float el = fast_exp2(c) * sgc;
    // token-major copies; the contraction over tokens reads them transposed
#pragma unroll
    for (int k = 0; k < kCC; ++k) {
      const int idx = tid + 256 * k, u = idx / (NS / 8), cc = idx % (NS / 8);
      *reinterpret_cast<u16x8*>(sm.Cs + u * (NS + 8) + 8 * cc) = creg[k];
    }
#pragma unroll
    for (int k = 0; k < kDC; ++k) {
      const int idx = tid + 256 * k, u = idx >> 3, cc = idx & 7;
      const float e = __shfl(el, u);
      u16x8 o;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = f2bf(bf2f(dreg[k][i]) * e);
      *reinterpret_cast<u16x8*>(sm.dyE + u * kBLd + 8 * cc) = o;
    }
    __syncthreads();
    if (j > 0) fetch(j - 1);
    const float dec = fast_exp2(cend) * sge;
    lsum += cend;
    ssign *= sge;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      gacc[nt] *= dec;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        gacc[nt] = mfma16x16x32(lds_tile_tr(sm.Cs, NS + 8, 32 * ks, 16 * nt, lane),
                                lds_tile_tr(sm.dyE, kBLd, 32 * ks, 16 * w, lane), gacc[nt]);
    }
    __syncthreads();
  }
  float* out = a.gseg + ((sg * a.B + b) * a.H + h) * kBP * NS;
  const int p = 16 * w + c16;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    *reinterpret_cast<f32x4*>(out + p * NS + 16 * nt + 4 * g4) = gacc[nt];
  if (tid == 0) a.lam[(sg * a.B + b) * a.H + h] = fast_exp2(lsum) * ssign;
}

template <int MODE, int NS>
__global__ __launch_bounds__(256) void ssd_bwd_gloc_kernel(BwdArgs a) {
  gloc_body<MODE, NS>(a, xcd_remap(blockIdx.x, gridDim.x));
}

// ---------------------------------------------------------------------------
// gcombine: one thread per state element; backwards over segments replace
// Gamma_loc(s) by Gamma_out(s) = adjoint of the state at the end of segment s.
// ---------------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(256) void ssd_bwd_gcombine_kernel(BwdArgs a, int64_t PN) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t BH = a.B * a.H;
  if (idx >= BH * PN) return;
  const int64_t bh = idx / PN;
  const int64_t so = state_off<MODE>(a, idx);
  float carry = a.dh_last != nullptr ? a.dh_last[so] : 0.f;
  for (int64_t s = a.nseg - 1; s >= 0; --s) {
    float* gp = a.gseg + s * BH * PN + idx;
    const float gl = *gp;
    *gp = carry;
    carry = fmaf(a.lam[s * BH + bh], carry, gl);
  }
  if (a.dh0 != nullptr) a.dh0[so] = carry;
}

// ---------------------------------------------------------------------------
// main
// ---------------------------------------------------------------------------
template <int NS>
struct alignas(16) MainLds {
  static constexpr int kLdN = NS + 8;
  uint16_t Cs[kBQ * kLdN];     // C[u][n]
  uint16_t Bs[kBQ * kLdN];     // B[t][n]                     (recompute: B_w[s][n])
  uint16_t xs[kBQ * kBLd];     // x[t][p]
  uint16_t dys[kBQ * kBLd];    // dy[u][p]
  uint16_t dyE[kBQ * kBLd];    // E_u dy[u][p]
  uint16_t Mt[kBQ * kBLd];     // Mp[u][t] as [t][u]
  uint16_t Wt[kBQ * kBLd];     // phi_t W[u][t] as [t][u]
  uint16_t Gs[kBP * kLdN];     // Gamma[p][n], then h_prev[p][n]
  // Operands that contract over tokens (or over p) are read from these
  // row-major tiles with the transposing LDS read (lds_tile_tr), so every
  // tile is written with 8- or 16-byte stores.
  float cum[kBQ], E[kBQ], sE[kBQ], phi[kBQ], dtv[kBQ], ek[kBQ];
  float sg[kBQ];               // sign of the decay product from the block start (bilinear)
  // T sums of the (u-tile j, t-tile i) tiles: rowT4[j][i][u % 16] over t,
  // colT4[i][j][t % 16] over u; slots of tiles never formed stay zero
  float rowT4[4][4][16], colT4[4][4][16];
  float toffp[4][kBQ], dphip[4][kBQ], up[4][kBQ];
  float uprevp[4];
  float ddp[4];                // per-wave dD sums
};

// the 12 (u-tile j, t-tile i) tiles of a block: the 10 causal ones plus (0,1)
// and (2,3), all-zero, which complete the 32-wide k steps of the consumers
__constant__ int kTileJ[12] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3, 0, 2};
__constant__ int kTileI[12] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3, 1, 3};

template <int DISC, int NS, int NBS>
__global__ __launch_bounds__(256) void ssd_bwd_main_kernel(BwdArgs a) {
  constexpr int NT = NS / 16, NK = NS / 32;
  constexpr int kLdN = MainLds<NS>::kLdN;
  __shared__ MainLds<NS> sm;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
  // heads vary fastest: the workgroups that run together on an XCD are the
  // heads of one (batch row, segment), which read the same B and C rows
  // (groups shared by heads), so those come from the XCD's L2
  const int64_t h = wid % a.H;
  const int64_t sg = (wid / a.H) % a.nseg;
  const int64_t b = wid / (a.H * a.nseg);
  const int64_t grp = h / (a.H / a.G);
  const float Ah = DISC == kBwdGla ? 0.f : a.A[h];
  const float invA = DISC == kBwdZoh ? 1.f / Ah : 0.f;   // unused (series branch) when A = 0
  const float Dh = a.Dskip != nullptr ? a.Dskip[h] : 0.f;
  const int64_t ts0 = sg * a.seg;
  const int64_t tse = (ts0 + a.seg < a.L) ? ts0 + a.seg : a.L;
  const int nb = static_cast<int>((tse - ts0 + kBQ - 1) / kBQ);
  const int64_t xrow = a.H * kBP;              // elements between tokens of x, dy, dx
  const int64_t xoff = h * kBP;
  const int64_t bcrow = a.G * NS;
  const int64_t bcoff = grp * NS;
  const int p = 16 * w + c16;                  // this lane's p column
  (&sm.rowT4[0][0][0])[tid] = 0.f;
  (&sm.colT4[0][0][0])[tid] = 0.f;

  // C, B, x, dy and the gate of one block of the backward sweep, loaded into
  // registers one block ahead.  Lane = token; wave w takes 16-byte column
  // chunks w, w + 4, ...
  constexpr int kSB = kBQ * (NS / 8) / 256, kSX = kBQ * (kBP / 8) / 256;
  u16x8 sc[kSB], sb[kSB], sx[kSX], sd[kSX];
  uint16_t sgr = 0;
  auto sfetch = [&](int j) {
    const int64_t t0 = ts0 + static_cast<int64_t>(j) * kBQ;
    const bool ok = lane < ((tse - t0) < kBQ ? (tse - t0) : kBQ);
    sgr = ok ? gate_raw<DISC>(a, b, t0 + lane, h, grp) : uint16_t(0);
    const int64_t bco = (b * a.L + t0 + lane) * bcrow + bcoff;
    const int64_t xo = (b * a.L + t0 + lane) * xrow + xoff;
#pragma unroll
    for (int k = 0; k < kSB; ++k) {
      sc[k] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      sb[k] = sc[k];
      if (ok) {
        sc[k] = *reinterpret_cast<const u16x8*>(a.Cm + bco + 8 * (w + 4 * k));
        sb[k] = *reinterpret_cast<const u16x8*>(a.Bm + bco + 8 * (w + 4 * k));
      }
    }
#pragma unroll
    for (int k = 0; k < kSX; ++k) {
      sx[k] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      sd[k] = sx[k];
      if (ok) {
        sx[k] = *reinterpret_cast<const u16x8*>(a.x + xo + 8 * (w + 4 * k));
        sd[k] = *reinterpret_cast<const u16x8*>(a.dy + xo + 8 * (w + 4 * k));
      }
    }
  };
  sfetch(nb - 1);   // in flight during the recompute

  // ---- forward recompute of the block-entry states of this segment; they
  // are kept in registers as packed bf16 MFMA operands (hsb[j][kk] holds
  // n-tiles 2kk and 2kk+1 in the operand order of pack_dd)
  bf16x8 hsb[NBS][NK];
  f32x4 hacc[NT];
  {
    const float* cp = (sg == 0 && a.h0 != nullptr)
                          ? a.h0 + (b * a.H + h) * kBP * NS
                          : a.ckpt + ((sg * a.ckB + b) * a.H + h) * kBP * NS;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) hacc[nt] = *reinterpret_cast<const f32x4*>(cp + p * NS + 16 * nt + 4 * g4);
  }
  // B, x and the gate of every recompute block, all loaded up front so that
  // their latencies overlap.  Blocks before the last are full, and as in
  // sfetch lane = token and wave w takes 16-byte column chunks w, w + 4, ...;
  // every wave scans the block's gates itself, so B is scaled to B_w while
  // it is written to LDS.
  constexpr int kRJ = NBS > 1 ? NBS - 1 : 1;
  u16x8 rb[kRJ][kSB], rx[kRJ][kSX];
  uint16_t rg[kRJ];
#pragma unroll
  for (int j = 0; j + 1 < NBS; ++j) {
    if (j + 1 < nb) {
      const int64_t t = ts0 + static_cast<int64_t>(j) * kBQ + lane, tok = b * a.L + t;
      rg[j] = gate_raw<DISC>(a, b, t, h, grp);
#pragma unroll
      for (int k = 0; k < kSB; ++k)
        rb[j][k] = *reinterpret_cast<const u16x8*>(a.Bm + tok * bcrow + bcoff + 8 * (w + 4 * k));
#pragma unroll
      for (int k = 0; k < kSX; ++k)
        rx[j][k] = *reinterpret_cast<const u16x8*>(a.x + tok * xrow + xoff + 8 * (w + 4 * k));
    }
  }
#pragma unroll
  for (int j = 0; j < NBS; ++j) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) hsb[j][kk] = pack_dd(hacc[2 * kk], hacc[2 * kk + 1]);
    if (j + 1 < nb) {
      float l2, ph, ek;
      block_scalars<DISC>(bf2f(rg[j]), true, Ah, l2, ph, ek);
      float sgc, sge;
      sign_scan<DISC>(ek, sgc, sge);
      const float c = wave_incl_sum(l2);
      const float cend = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), 63));
      const float ws = fast_exp2(cend - c) * (sge * sgc) * ph;
#pragma unroll
      for (int k = 0; k < kSB; ++k) {
        u16x8 o;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = f2bf(bf2f(rb[j][k][i]) * ws);
        *reinterpret_cast<u16x8*>(sm.Bs + lane * kLdN + 8 * (w + 4 * k)) = o;   // B_w
      }
#pragma unroll
      for (int k = 0; k < kSX; ++k)
        *reinterpret_cast<u16x8*>(sm.xs + lane * kBLd + 8 * (w + 4 * k)) = rx[j][k];
      __syncthreads();
      const float dec = fast_exp2(cend) * sge;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        hacc[nt] *= dec;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          hacc[nt] = mfma16x16x32(lds_tile_tr(sm.Bs, kLdN, 32 * ks, 16 * nt, lane),
                                  lds_tile_tr(sm.xs, kBLd, 32 * ks, 16 * w, lane), hacc[nt]);
      }
      __syncthreads();
    }
  }

  // ---- adjoint of the segment's last state from later tokens
  f32x4 gacc[NT];
  {
    const float* gp = a.gseg + ((sg * a.B + b) * a.H + h) * kBP * NS;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) gacc[nt] = *reinterpret_cast<const f32x4*>(gp + p * NS + 16 * nt + 4 * g4);
  }
  float dA_acc = 0.f, dD_acc = 0.f;


#pragma unroll 1
  for (int j = nb - 1; j >= 0; --j) {
    // the stash entry of this block (uniform switch keeps register indices static)
    bf16x8 hcur[NK];
#pragma unroll
    for (int jj = 0; jj < NBS; ++jj)
      if (jj == j) {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) hcur[kk] = hsb[jj][kk];
      }
    const int64_t t0 = ts0 + static_cast<int64_t>(j) * kBQ;
    const int nv = static_cast<int>((tse - t0) < kBQ ? (tse - t0) : kBQ);

    // ---- stage the block from the registers sfetch filled.  Every staged
    // row is token `lane` of the block, so each wave computes the per-token
    // scalars itself and scales dy (by E) as it is written; wave 0 also keeps
    // the scalars in LDS for the later phases.
    {
      const bool ok = lane < nv;
      const float dtv = bf2f(sgr);   // 0 for masked tokens
      float l2, ph, ek;
      block_scalars<DISC>(dtv, ok, Ah, l2, ph, ek);
      ph = ok ? ph : 0.f;
      float sgc, sge;
      sign_scan<DISC>(ek, sgc, sge);
      const float c = wave_incl_sum(l2);
      const float el = fast_exp2(c) * sgc;
      if (w == 0) {
        const float cend = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), 63));
        sm.cum[lane] = c;
        sm.sg[lane] = sgc;
        sm.E[lane] = el;
        sm.sE[lane] = fast_exp2(cend - c) * (sge * sgc);
        sm.phi[lane] = ph;
        sm.dtv[lane] = dtv;
        sm.ek[lane] = ek;
      }
#pragma unroll
      for (int k = 0; k < kSB; ++k) {
        const int cc = w + 4 * k;
        *reinterpret_cast<u16x8*>(sm.Cs + lane * kLdN + 8 * cc) = sc[k];
        *reinterpret_cast<u16x8*>(sm.Bs + lane * kLdN + 8 * cc) = sb[k];
      }
#pragma unroll
      for (int k = 0; k < kSX; ++k) {
        const int cc = w + 4 * k;
        *reinterpret_cast<u16x8*>(sm.xs + lane * kBLd + 8 * cc) = sx[k];
        *reinterpret_cast<u16x8*>(sm.dys + lane * kBLd + 8 * cc) = sd[k];
        u16x8 de;
#pragma unroll
        for (int i = 0; i < 8; ++i) de[i] = f2bf(bf2f(sd[k][i]) * el);
        *reinterpret_cast<u16x8*>(sm.dyE + lane * kBLd + 8 * cc) = de;
      }
    }
    // the next block's loads are in flight during this block's phases
    if (j > 0) sfetch(j - 1);
    __syncthreads();

    // ---- decayed masks and the T sums
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int tile = 3 * w + q;
      const int tj = kTileJ[tile], ti = kTileI[tile];
      const int t = 16 * ti + c16;           // this lane's column (source token)
      const int u0 = 16 * tj + 4 * g4;       // this lane's 4 rows (output tokens)
      u16x4 om = {0, 0, 0, 0}, ow = om;
      float rsum[4] = {0.f, 0.f, 0.f, 0.f}, csum = 0.f;
      if (tj >= ti) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f}, rr = s;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
          s = mfma16x16x32(lds_tile(sm.Cs, kLdN, 16 * tj, 32 * kk, lane),
                           lds_tile(sm.Bs, kLdN, 16 * ti, 32 * kk, lane), s);
#pragma unroll
        for (int kp = 0; kp < 2; ++kp)
          rr = mfma16x16x32(lds_tile(sm.dys, kBLd, 16 * tj, 32 * kp, lane),
                            lds_tile(sm.xs, kBLd, 16 * ti, 32 * kp, lane), rr);
        const float ct = sm.cum[t], pt = sm.phi[t];
        const float st = DISC == kBwdBilinear ? sm.sg[t] : 1.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int u = u0 + r;
          // loads and exponential unconditional, then a select: no per-lane
          // branches around LDS reads (inf above the diagonal is discarded)
          float m = fast_exp2(sm.cum[u] - ct);
          if (DISC == kBwdBilinear) m *= st * sm.sg[u];
          m = (u >= t) ? m : 0.f;
          const float mp = s[r] * m, wv = rr[r] * m * pt;
          const float tv = mp * pt * rr[r];
          om[r] = f2bf(mp);
          ow[r] = f2bf(wv);
          rsum[r] = tv;
          csum += tv;
        }
      }
      *reinterpret_cast<u16x4*>(sm.Mt + t * kBLd + u0) = om;
      *reinterpret_cast<u16x4*>(sm.Wt + t * kBLd + u0) = ow;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float rs = row16_sum_last(rsum[r]);
        if (c16 == 15) sm.rowT4[tj][ti][4 * g4 + r] = rs;
      }
      const float cs = col4_sum(csum);
      if (g4 == 0) sm.colT4[ti][tj][c16] = cs;
    }
    __syncthreads();

    // ---- recomputed C h_prev (for the c-gradient), dx, dphi, U, dD, U_prev.
    // The three products are formed transposed, [p][t] (lane: token
    // 16 ti + c16, p rows 16 w + 4 g4 .. + 3), so that the sums over p are
    // register adds plus one col4_sum, and x, dy and dx move 4 p at a time.
    {
      f32x4 yo[4], dxa[4], dxb[4];
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        yo[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
        dxa[ti] = yo[ti];
        dxb[ti] = yo[ti];
      }
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const bf16x8 hb = hcur[kk];
        const bf16x8 gb = pack_dd(gacc[2 * kk], gacc[2 * kk + 1]);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          yo[ti] = mfma16x16x32(hb, lds_tile_perm(sm.Cs, kLdN, 16 * ti, 32 * kk, lane), yo[ti]);
          dxb[ti] = mfma16x16x32(gb, lds_tile_perm(sm.Bs, kLdN, 16 * ti, 32 * kk, lane), dxb[ti]);
        }
      }
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if (ks == 0 && ti >= 2) continue;   // Mp[u][t] = 0 for u < t
          dxa[ti] = mfma16x16x32(lds_tile_tr(sm.dys, kBLd, 32 * ks, 16 * w, lane),
                                 lds_tile(sm.Mt, kBLd, 16 * ti, 32 * ks, lane), dxa[ti]);
        }
      }
      float ddsum = 0.f;
      const int pr = 16 * w + 4 * g4;   // this lane's 4 p rows
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        const int t = 16 * ti + c16;    // this lane's token
        const u16x4 xv4 = *reinterpret_cast<const u16x4*>(sm.xs + t * kBLd + pr);
        const u16x4 dy4 = *reinterpret_cast<const u16x4*>(sm.dys + t * kBLd + pr);
        const float se = sm.sE[t], ph = sm.phi[t];
        float toff = 0.f, dph = 0.f, uu = 0.f;
        u16x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float xv = bf2f(xv4[r]), dyv = bf2f(dy4[r]);
          const float xb = dxb[ti][r] * se;
          const float gB = dxa[ti][r] + xb;
          o[r] = f2bf(fmaf(ph, gB, Dh * dyv));
          toff = fmaf(yo[ti][r], dyv, toff);
          dph = fmaf(xv, gB, dph);
          uu = fmaf(xv, xb, uu);
          ddsum = fmaf(dyv, xv, ddsum);
        }
        if (t < nv) *reinterpret_cast<u16x4*>(a.dx + (b * a.L + t0 + t) * xrow + xoff + pr) = o;
        toff = col4_sum(toff);   // times E_t in the decay phase
        dph = col4_sum(dph);
        uu = col4_sum(uu) * ph;
        if (g4 == 0) {
          sm.toffp[w][t] = toff;
          sm.dphip[w][t] = dph;
          sm.up[w][t] = uu;
        }
      }
      dD_acc += wave_sum(ddsum);
      float up = 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const u16x8 hv = __builtin_bit_cast(u16x8, hcur[nt >> 1]);
#pragma unroll
        for (int r = 0; r < 4; ++r) up += gacc[nt][r] * bf2f(hv[4 * (nt & 1) + r]);
      }
      up = wave_sum(up);
      if (lane == 0) sm.uprevp[w] = up;
    }

    // ---- dB: Gamma to LDS, then (phi W)^T C + phi_t sE_t x Gamma
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      *reinterpret_cast<u16x4*>(sm.Gs + p * kLdN + 16 * nt + 4 * g4) =
          u16x4{f2bf(gacc[nt][0]), f2bf(gacc[nt][1]), f2bf(gacc[nt][2]), f2bf(gacc[nt][3])};
    __syncthreads();
    // per-token scales of the dB and dC epilogues, read here once: the empty
    // asm keeps the reads (and their wait) out of the ragged-tail branches
    float psE[4], eU[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      psE[q] = sm.phi[16 * q + c16] * sm.sE[16 * q + c16];
      eU[q] = sm.E[16 * q + c16];
      asm volatile("" : "+v"(psE[q]), "+v"(eU[q]));
    }
    {
      // the wave's n-tiles' operands of C and Gamma serve all four token
      // tiles, and each token tile's operands of W and x serve both n-tiles
      constexpr int NA = NT / 4;
      bf16x8 ct[NA][2], gt[NA][2];
#pragma unroll
      for (int aa = 0; aa < NA; ++aa)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          ct[aa][k2] = lds_tile_tr(sm.Cs, kLdN, 32 * k2, 16 * (NA * w + aa), lane);
          gt[aa][k2] = lds_tile_tr(sm.Gs, kLdN, 32 * k2, 16 * (NA * w + aa), lane);
        }
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        bf16x8 wt[2], xt[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          if (!(k2 == 0 && ti >= 2)) wt[k2] = lds_tile(sm.Wt, kBLd, 16 * ti, 32 * k2, lane);
          xt[k2] = lds_tile(sm.xs, kBLd, 16 * ti, 32 * k2, lane);
        }
        const int t = 16 * ti + c16;
#pragma unroll
        for (int aa = 0; aa < NA; ++aa) {
          const int nt = NA * w + aa;
          f32x4 d1 = {0.f, 0.f, 0.f, 0.f}, d2 = d1;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            if (ks == 0 && ti >= 2) continue;
            d1 = mfma16x16x32(ct[aa][ks], wt[ks], d1);
          }
#pragma unroll
          for (int kp = 0; kp < 2; ++kp) d2 = mfma16x16x32(gt[aa][kp], xt[kp], d2);
          if (t < nv) {
            f32x4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = fmaf(psE[ti], d2[r], d1[r]);
            *reinterpret_cast<u16x4*>(a.dBpart + ((b * a.L + t0 + t) * a.H + h) * NS + 16 * nt + 4 * g4) =
                u16x4{f2bf(v[0]), f2bf(v[1]), f2bf(v[2]), f2bf(v[3])};
          }
        }
      }
    }
    // ---- Gamma for the previous block: E_end Gamma + sum_u E_u dy_u (x) C_u
    {
      const float dec = fast_exp2(sm.cum[kBQ - 1]) * (DISC == kBwdBilinear ? sm.sg[kBQ - 1] : 1.f);
      const bf16x8 de0 = lds_tile_tr(sm.dyE, kBLd, 0, 16 * w, lane);
      const bf16x8 de1 = lds_tile_tr(sm.dyE, kBLd, 32, 16 * w, lane);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        gacc[nt] *= dec;
        gacc[nt] = mfma16x16x32(lds_tile_tr(sm.Cs, kLdN, 0, 16 * nt, lane), de0, gacc[nt]);
        gacc[nt] = mfma16x16x32(lds_tile_tr(sm.Cs, kLdN, 32, 16 * nt, lane), de1, gacc[nt]);
      }
    }
    __syncthreads();

    // ---- dC: h_prev to LDS, then (phi W) B + E_u dy h_prev
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const u16x8 hv = __builtin_bit_cast(u16x8, hcur[nt >> 1]);
      *reinterpret_cast<u16x4*>(sm.Gs + p * kLdN + 16 * nt + 4 * g4) =
          u16x4{hv[4 * (nt & 1)], hv[4 * (nt & 1) + 1], hv[4 * (nt & 1) + 2], hv[4 * (nt & 1) + 3]};
    }
    __syncthreads();
    {
      // as for dB: n-tile operands of B and h_prev, token-tile operands of W
      // and dy, each read once
      constexpr int NA = NT / 4;
      bf16x8 bt[NA][2], ht[NA][2];
#pragma unroll
      for (int aa = 0; aa < NA; ++aa)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          bt[aa][k2] = lds_tile_tr(sm.Bs, kLdN, 32 * k2, 16 * (NA * w + aa), lane);
          ht[aa][k2] = lds_tile_tr(sm.Gs, kLdN, 32 * k2, 16 * (NA * w + aa), lane);
        }
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) {
        bf16x8 wt[2], dt2[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          if (!(k2 == 1 && tj < 2)) wt[k2] = lds_tile_tr(sm.Wt, kBLd, 32 * k2, 16 * tj, lane);
          dt2[k2] = lds_tile(sm.dys, kBLd, 16 * tj, 32 * k2, lane);
        }
        const int u = 16 * tj + c16;
#pragma unroll
        for (int aa = 0; aa < NA; ++aa) {
          const int nt = NA * w + aa;
          f32x4 d1 = {0.f, 0.f, 0.f, 0.f}, d2 = d1;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            if (ks == 1 && tj < 2) continue;
            d1 = mfma16x16x32(bt[aa][ks], wt[ks], d1);
          }
#pragma unroll
          for (int kp = 0; kp < 2; ++kp) d2 = mfma16x16x32(ht[aa][kp], dt2[kp], d2);
          if (u < nv) {
            f32x4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = fmaf(eU[tj], d2[r], d1[r]);
            *reinterpret_cast<u16x4*>(a.dCpart + ((b * a.L + t0 + u) * a.H + h) * NS + 16 * nt + 4 * g4) =
                u16x4{f2bf(v[0]), f2bf(v[1]), f2bf(v[2]), f2bf(v[3])};
          }
        }
      }
    }

    // Every LDS tile of the block has been read once all waves are here; the
    // phase below reads only per-token scalars and partial sums, which no
    // other wave writes before the next block's dx phase, so waves 1-3 go on
    // to stage the next block meanwhile.
    __syncthreads();

    // ---- log-decay gradient -> ddt, dA (wave 0, lane = token)
    if (w == 0) {
      const int k = lane;
      float rowT = 0.f, colT = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rowT += sm.rowT4[k >> 4][i][k & 15];
        colT += sm.colT4[k >> 4][i][k & 15];
      }
      const float toff = sm.E[k] * (sm.toffp[0][k] + sm.toffp[1][k] + sm.toffp[2][k] + sm.toffp[3][k]);
      const float dph = sm.dphip[0][k] + sm.dphip[1][k] + sm.dphip[2][k] + sm.dphip[3][k];
      const float uu = sm.up[0][k] + sm.up[1][k] + sm.up[2][k] + sm.up[3][k];
      const float uprev = fast_exp2(sm.cum[kBQ - 1]) * (DISC == kBwdBilinear ? sm.sg[kBQ - 1] : 1.f) *
                          (sm.uprevp[0] + sm.uprevp[1] + sm.uprevp[2] + sm.uprevp[3]);
      // reverse inclusive prefix sum dlam_k = sum_{j >= k} dcum_j, where the
      // last token's dcum also carries uprev + sum(uu): that term enters every
      // dlam_k, so it is added after the scan, and the two scans run side by side
      const float dcum = rowT - colT + toff - uu;
      const float usum = wave_sum(uu);
      const float incl = wave_incl_sum(dcum);
      const float total = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), 63));
      const float dlam = (total - incl + dcum) + (uprev + usum);
      const float dtv = sm.dtv[k], ek = sm.ek[k], ph = sm.phi[k];
      float ddt = 0.f, dAk = 0.f;
      if (DISC == kBwdGla) {
        // phi is constant: the log-gate gradient goes out per 64-column slice
        if (k < nv) a.dgpart[(b * a.L + t0 + k) * a.H + h] = dlam;
      } else if (DISC == kBwdDirac) {   // phi = 1: no input-factor term
        ddt = dlam * Ah;
        dAk = dlam * dtv;
      } else if (DISC == kBwdEuler) {
        ddt = dlam * Ah + dph;
        dAk = dlam * dtv;
      } else if (DISC == kBwdBilinear) {
        // dlam is the gradient wrt ln|e|: d ln|e| / dl = 1 / ((1 - l/2)(1 + l/2));
        // dphi/ddt = r^2, dphi/dA = dt^2 r^2 / 2 with r = 1 / (1 - l/2)
        const float lam = dtv * Ah;
        const float r = __builtin_amdgcn_rcpf(1.f - 0.5f * lam);
        const float dln = r * __builtin_amdgcn_rcpf(1.f + 0.5f * lam);
        const float gl = isfinite(dln) ? dlam * dln : 0.f;
        ddt = fmaf(gl, Ah, dph * r * r);
        dAk = fmaf(gl, dtv, dph * 0.5f * dtv * dtv * r * r);
      } else {
        const float lam = dtv * Ah;
        const float dphidA = fabsf(lam) < 1e-3f
                                 ? dtv * dtv * fmaf(lam, fmaf(lam, 1.f / 8.f, 1.f / 3.f), 0.5f)
                                 : (dtv * ek - ph) * invA;
        ddt = fmaf(dlam, Ah, dph * ek);
        dAk = fmaf(dlam, dtv, dph * dphidA);
      }
      if (DISC != kBwdGla) {
        if (k < nv) a.ddt[(b * a.L + t0 + k) * a.H + h] = f2bf(ddt);
        dA_acc += k < nv ? dAk : 0.f;   // per token; summed over the wave at the end
      }
    }
  }
  dA_acc = wave_sum(dA_acc);
  if (tid == 0) a.dApart[(b * a.H + h) * a.nseg + sg] = dA_acc;
  // own slots: wave 0 may still be reading uprevp in the last block's decay phase
  if (lane == 0) sm.ddp[w] = dD_acc;
  __syncthreads();
  if (tid == 0) a.dDpart[(b * a.H + h) * a.nseg + sg] = sm.ddp[0] + sm.ddp[1] + sm.ddp[2] + sm.ddp[3];
}

// ---------------------------------------------------------------------------
// reduce: dB, dC over the heads of each group (fixed order); dA, dD over
// (batch, segment) per head.
// ---------------------------------------------------------------------------
// The first nblk_bc blocks: dB, dC, one thread per 8 consecutive n of a
// (b, t, group) row, heads summed in order.  The blocks after them: dA, dD,
// one wave per head; lane l sums partials l, l + 64, ... in order and the
// wave adds the 64 lane sums in a fixed pattern.
__device__ __forceinline__ void reduce_bc_block(const BwdArgs& a, int64_t blk) {
  {
    const int64_t n8 = a.N / 8;
    const int64_t total = a.B * a.L * a.G * n8;
    const int64_t idx = blk * 256 + threadIdx.x;
    if (idx >= total) return;
    const int64_t hpg = a.H / a.G;
    const int64_t c8 = idx % n8;
    const int64_t g = (idx / n8) % a.G;
    const int64_t bt = idx / (n8 * a.G);     // b * L + t
    const int64_t hstride = a.N;   // heads innermost
    const uint16_t* pb = a.dBpart + (bt * a.H + g * hpg) * a.N + 8 * c8;
    const uint16_t* pc = a.dCpart + (bt * a.H + g * hpg) * a.N + 8 * c8;
    float sb[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, sc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int64_t k = 0; k < hpg; ++k) {
      const u16x8 vb = *reinterpret_cast<const u16x8*>(pb + k * hstride);
      const u16x8 vc = *reinterpret_cast<const u16x8*>(pc + k * hstride);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        sb[r] += bf2f(vb[r]);
        sc[r] += bf2f(vc[r]);
      }
    }
    const int64_t o = (bt * a.G + g) * a.N + 8 * c8;
    u16x8 ob, oc;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      ob[r] = f2bf(sb[r]);
      oc[r] = f2bf(sc[r]);
    }
    *reinterpret_cast<u16x8*>(a.dBm + o) = ob;
    *reinterpret_cast<u16x8*>(a.dCm + o) = oc;
  }
}

__global__ __launch_bounds__(256) void ssd_bwd_reduce_kernel(BwdArgs a, int64_t nblk_bc) {
  if (blockIdx.x < nblk_bc) {
    reduce_bc_block(a, blockIdx.x);
    return;
  }
  if (a.dA == nullptr) return;
  const int lane = threadIdx.x & 63;
  const int64_t hh = (blockIdx.x - nblk_bc) * 4 + (threadIdx.x >> 6);
  if (hh >= a.H) return;   // whole waves leave together
  float sa = 0.f, sd = 0.f;
  for (int64_t i = lane; i < a.B * a.nseg; i += 64) {
    const int64_t bb = i / a.nseg, sgi = i % a.nseg;
    sa += a.dApart[(bb * a.H + hh) * a.nseg + sgi];
    sd += a.dDpart[(bb * a.H + hh) * a.nseg + sgi];
  }
  sa = wave_sum(sa);
  sd = wave_sum(sd);
  if (lane == 0) {
    a.dA[hh] = sa;
    if (a.dD != nullptr) a.dD[hh] = sd;
  }
}

// GLA: dg = (sum of the per-slice log-gate gradients) / g, fixed order.
__device__ __forceinline__ void gla_dg_block(const BwdArgs& a, int64_t blk) {
  const int64_t idx = blk * 256 + threadIdx.x;   // (b L + t) G + grp
  if (idx >= a.B * a.L * a.G) return;
  const int64_t grp = idx % a.G, bt = idx / a.G;
  const int64_t hpg = a.H / a.G;
  float s = 0.f;
  for (int64_t hh = grp * hpg; hh < (grp + 1) * hpg; ++hh) s += a.dgpart[bt * a.H + hh];
  a.dg[idx] = f2bf(s / bf2f(a.dt[idx]));
}

__global__ __launch_bounds__(256) void gla_bwd_dg_kernel(BwdArgs a) { gla_dg_block(a, blockIdx.x); }

// One launch running two independent jobs side by side: gloc of a batch
// slice (latency bound) and the reductions of the slice before it (bandwidth
// bound: dB, dC over heads, and for GLA the gate gradient).  They touch
// disjoint buffers: gloc writes the segment adjoints, the reductions read
// the partials the previous slice's main kernel wrote.  Work ids go through
// the XCD remap first, then the reduction blocks are spread evenly among the
// gloc workgroups (id f is reduction block floor(f nr / total) when that
// floor steps at f, else gloc workgroup f - floor(f nr / total)).
template <int MODE, int NS>
__global__ __launch_bounds__(256) void ssd_bwd_gloc_reduce_kernel(BwdArgs gl, BwdArgs rd,
                                                                  int64_t n_red, int64_t n_dg) {
  const int64_t total = gridDim.x;
  const int64_t nr = n_red + n_dg;
  const int64_t f = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t r_lo = f * nr / total, r_hi = (f + 1) * nr / total;
  if (r_hi > r_lo) {
    if (r_lo < n_red) reduce_bc_block(rd, r_lo);
    else gla_dg_block(rd, r_lo - n_red);
    return;
  }
  gloc_body<MODE, NS>(gl, f - r_lo);
}

// Empty input (B * L == 0): dA = dD = 0 and dh0 = dh_last (or 0).
__global__ __launch_bounds__(256) void ssd_bwd_empty_kernel(float* dA, float* dD, float* dh0,
                                                            const float* dh_last, int64_t H,
                                                            int64_t nstate) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < H) {
    if (dA != nullptr) dA[i] = 0.f;
    if (dD != nullptr) dD[i] = 0.f;
  }
  if (dh0 != nullptr && i < nstate) dh0[i] = dh_last != nullptr ? dh_last[i] : 0.f;
}

hipError_t launch_ssd_bwd_empty(float* dA, float* dD, float* dh0, const float* dh_last, int64_t H,
                                int64_t nstate, hipStream_t stream) {
  const int64_t n = (nstate > H ? nstate : H);
  hipLaunchKernelGGL(ssd_bwd_empty_kernel, dim3((n + 255) / 256 > 0 ? (n + 255) / 256 : 1), dim3(256),
                     0, stream, dA, dD, dh0, dh_last, H, nstate);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
static inline int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }

struct WsLayout {
  int64_t dB, dC, g, lam, dA, dD, dg, total;
};

// The launches run over slices of bs batch rows: the per-token and per-state
// partials in the workspace are sized for one slice, so the workspace stays
// bounded as B grows.  By default a slice holds at least 1024 workgroups of
// the main kernel (four per CU), or the whole batch.
static int64_t bwd_slice(int64_t B, int64_t L, int64_t H, int64_t seg) {
  const int64_t per_row = H * ((L + seg - 1) / seg);
  const int64_t bs = (1024 + per_row - 1) / per_row;
  return bs < B ? bs : B;
}

// H: heads of 64 columns (for GLA, H * V / 64).  dA and dD partials cover
// the whole batch; everything else one slice of bs rows.
static WsLayout ws_layout(int64_t B, int64_t L, int64_t H, int64_t N, int64_t seg, bool gla,
                          int64_t bs) {
  const int64_t nseg = (L + seg - 1) / seg;
  WsLayout w;
  int64_t o = 0;
  w.dB = o; o = align256(o + H * bs * L * N * 2);
  w.dC = o; o = align256(o + H * bs * L * N * 2);
  w.g = o; o = align256(o + nseg * bs * H * kBP * N * 4);
  w.lam = o; o = align256(o + nseg * bs * H * 4);
  w.dA = o; o = align256(o + B * H * nseg * 4);
  w.dD = o; o = align256(o + B * H * nseg * 4);
  w.dg = o; o = align256(o + (gla ? H * bs * L * 4 : 0));
  w.total = o;
  return w;
}

// The largest slice (at most the default one) whose layout fits in ws_bytes;
// 0 when not even one row fits.
static int64_t bwd_slice_fit(int64_t B, int64_t L, int64_t H, int64_t N, int64_t seg, bool gla,
                             size_t ws_bytes) {
  for (int64_t bs = bwd_slice(B, L, H, seg); bs >= 1; --bs)
    if (static_cast<size_t>(ws_layout(B, L, H, N, seg, gla, bs).total) <= ws_bytes) return bs;
  return 0;
}

size_t ssd_bwd_workspace(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                         int64_t seg, bool smallest) {
  (void)G;
  if (P != kBP || seg > 256 || B * L == 0) return 0;
  const int64_t bs = smallest ? 1 : bwd_slice(B, L, H, seg);
  return static_cast<size_t>(ws_layout(B, L, H, N, seg, false, bs).total);
}

size_t gla_bwd_workspace(int64_t B, int64_t L, int64_t H, int64_t K, int64_t V, int64_t seg,
                         bool smallest) {
  if (V % kBP != 0 || seg > 256 || B * L == 0) return 0;
  const int64_t Hs = H * (V / kBP);
  const int64_t bs = smallest ? 1 : bwd_slice(B, L, Hs, seg);
  return static_cast<size_t>(ws_layout(B, L, Hs, K, seg, true, bs).total);
}

bool ssd_bwd_supported(int64_t P, int64_t N, int64_t seg) {
  return P == kBP && (N == 64 || N == 128) && seg >= 64 && seg <= 256 && seg % 64 == 0;
}

template <int MODE, int NS>
static void launch_main(const BwdArgs& a, int64_t nwg, int nbs, hipStream_t s) {
  if (nbs == 1) hipLaunchKernelGGL((ssd_bwd_main_kernel<MODE, NS, 1>), dim3(nwg), dim3(256), 0, s, a);
  else if (nbs == 2) hipLaunchKernelGGL((ssd_bwd_main_kernel<MODE, NS, 2>), dim3(nwg), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((ssd_bwd_main_kernel<MODE, NS, 4>), dim3(nwg), dim3(256), 0, s, a);
}

// The launches on filled-in args: per slice of batch rows gloc, gcombine,
// main and the dB/dC reduction (plus the gate reduction for GLA), each on
// pointers advanced to the slice's first row; then dA, dD over the batch.
template <int MODE>
static hipError_t launch_bwd(BwdArgs a, void* ws, size_t ws_bytes, hipStream_t stream) {
  const int64_t bs = bwd_slice_fit(a.B, a.L, a.H, a.N, a.seg, MODE == kBwdGla, ws_bytes);
  if (bs < 1) return hipErrorInvalidValue;   // the entry points check the size first
  const WsLayout lay = ws_layout(a.B, a.L, a.H, a.N, a.seg, MODE == kBwdGla, bs);
  char* base = static_cast<char*>(ws);
  a.dBpart = reinterpret_cast<uint16_t*>(base + lay.dB);
  a.dCpart = reinterpret_cast<uint16_t*>(base + lay.dC);
  a.gseg = reinterpret_cast<float*>(base + lay.g);
  a.lam = reinterpret_cast<float*>(base + lay.lam);
  a.dApart = reinterpret_cast<float*>(base + lay.dA);
  a.dDpart = reinterpret_cast<float*>(base + lay.dD);
  a.dgpart = reinterpret_cast<float*>(base + lay.dg);
  a.nseg = (a.L + a.seg - 1) / a.seg;
  a.ckB = a.B;
  const int64_t PN = kBP * a.N;
  const int nbs = static_cast<int>(a.seg / kBQ);
  // blocks of the reductions of slice r: dB, dC over heads; GLA's gate gradient
  auto n_red = [](const BwdArgs& r) { return (r.B * r.L * r.G * (r.N / 8) + 255) / 256; };
  auto n_dg = [](const BwdArgs& r) { return MODE == kBwdGla ? (r.B * r.L * r.G + 255) / 256 : int64_t(0); };
  BwdArgs prev = a;      // the slice whose reductions are still to run
  bool pending = false;
  for (int64_t b0 = 0; b0 < a.B; b0 += bs) {
    BwdArgs s = a;
    s.B = (a.B - b0) < bs ? (a.B - b0) : bs;
    const int64_t xr = b0 * a.L * a.H * kBP;   // x, dy, dx rows of the slice
    const int64_t gr = b0 * a.L;               // tokens before the slice
    const int64_t st = b0 * a.H * PN;          // state elements before the slice
    s.x += xr; s.dy += xr; s.dx += xr;
    s.dt += gr * (MODE == kBwdGla ? a.G : a.H);
    if (s.ddt != nullptr) s.ddt += gr * a.H;
    s.Bm += gr * a.G * a.N; s.Cm += gr * a.G * a.N;
    s.dBm += gr * a.G * a.N; s.dCm += gr * a.G * a.N;
    if (s.dg != nullptr) s.dg += gr * a.G;
    s.ckpt += st;
    if (s.h0 != nullptr) s.h0 += st;
    if (s.dh_last != nullptr) s.dh_last += st;
    if (s.dh0 != nullptr) s.dh0 += st;
    s.dApart += b0 * a.H * a.nseg;
    s.dDpart += b0 * a.H * a.nseg;
    const int64_t nwg = s.B * s.H * s.nseg;
    if (!pending) {
      if (s.N == 128) hipLaunchKernelGGL((ssd_bwd_gloc_kernel<MODE, 128>), dim3(nwg), dim3(256), 0, stream, s);
      else hipLaunchKernelGGL((ssd_bwd_gloc_kernel<MODE, 64>), dim3(nwg), dim3(256), 0, stream, s);
    } else {   // this slice's gloc beside the previous slice's reductions
      const int64_t nr = n_red(prev), nd = n_dg(prev);
      const dim3 grid(static_cast<unsigned>(nwg + nr + nd));
      if (s.N == 128)
        hipLaunchKernelGGL((ssd_bwd_gloc_reduce_kernel<MODE, 128>), grid, dim3(256), 0, stream, s, prev, nr, nd);
      else
        hipLaunchKernelGGL((ssd_bwd_gloc_reduce_kernel<MODE, 64>), grid, dim3(256), 0, stream, s, prev, nr, nd);
    }
    hipLaunchKernelGGL(ssd_bwd_gcombine_kernel<MODE>, dim3((s.B * s.H * PN + 255) / 256), dim3(256), 0,
                       stream, s, PN);
    if (s.N == 128) launch_main<MODE, 128>(s, nwg, nbs, stream);
    else launch_main<MODE, 64>(s, nwg, nbs, stream);
    prev = s;
    pending = true;
  }
  if (pending) {   // the last slice's reductions
    const int64_t nr = n_red(prev);
    hipLaunchKernelGGL(ssd_bwd_reduce_kernel, dim3(nr), dim3(256), 0, stream, prev, nr);
    if (MODE == kBwdGla) hipLaunchKernelGGL(gla_bwd_dg_kernel, dim3(n_dg(prev)), dim3(256), 0, stream, prev);
  }
  if (a.dA != nullptr)
    hipLaunchKernelGGL(ssd_bwd_reduce_kernel, dim3((a.H + 3) / 4), dim3(256), 0, stream, a, int64_t(0));
  return hipGetLastError();
}

hipError_t launch_ssd_bwd(int disc, const void* x, const void* dt, const float* A, const void* Bm,
                          const void* Cm, const float* Dskip, const float* h0, const float* ckpt,
                          const void* dy,
                          const float* dh_last, void* dx, void* ddt, float* dA, void* dBm,
                          void* dCm, float* dD, float* dh0, void* ws, size_t ws_bytes,
                          int64_t B, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                          int64_t seg, hipStream_t stream) {
  (void)P;
  if (B * L == 0) return hipSuccess;
  BwdArgs a = {};
  a.x = static_cast<const uint16_t*>(x); a.dt = static_cast<const uint16_t*>(dt); a.A = A;
  a.Bm = static_cast<const uint16_t*>(Bm); a.Cm = static_cast<const uint16_t*>(Cm);
  a.Dskip = Dskip; a.ckpt = ckpt; a.dy = static_cast<const uint16_t*>(dy); a.dh_last = dh_last;
  a.h0 = h0;
  a.dx = static_cast<uint16_t*>(dx); a.ddt = static_cast<uint16_t*>(ddt); a.dA = dA;
  a.dBm = static_cast<uint16_t*>(dBm); a.dCm = static_cast<uint16_t*>(dCm); a.dD = dD; a.dh0 = dh0;
  a.B = B; a.L = L; a.H = H; a.G = G; a.N = N; a.seg = seg;
  // disc holds the public discretisation code (ZOH 0, Euler 1, bilinear 2, dirac 3)
  if (disc == kBwdEuler) return launch_bwd<kBwdEuler>(a, ws, ws_bytes, stream);
  if (disc == kBwdDirac) return launch_bwd<kBwdDirac>(a, ws, ws_bytes, stream);
  if (disc == 2) return launch_bwd<kBwdBilinear>(a, ws, ws_bytes, stream);
  return launch_bwd<kBwdZoh>(a, ws, ws_bytes, stream);
}

hipError_t launch_gla_bwd(const void* q, const void* k, const void* v, const void* g,
                          const float* ckpt, const void* dout, const float* dS_last, void* dq,
                          void* dk, void* dv, void* dg, float* dS0, void* ws, size_t ws_bytes,
                          int64_t B, int64_t L, int64_t H, int64_t K, int64_t V, int64_t seg,
                          hipStream_t stream) {
  if (B * L == 0) return hipSuccess;
  BwdArgs a = {};
  a.x = static_cast<const uint16_t*>(v); a.dt = static_cast<const uint16_t*>(g); a.A = nullptr;
  a.Bm = static_cast<const uint16_t*>(k); a.Cm = static_cast<const uint16_t*>(q);
  a.Dskip = nullptr; a.ckpt = ckpt; a.dy = static_cast<const uint16_t*>(dout); a.dh_last = dS_last;
  a.dx = static_cast<uint16_t*>(dv); a.ddt = nullptr; a.dA = nullptr;
  a.dBm = static_cast<uint16_t*>(dk); a.dCm = static_cast<uint16_t*>(dq); a.dD = nullptr; a.dh0 = dS0;
  a.dg = static_cast<uint16_t*>(dg);
  a.B = B; a.L = L; a.H = H * (V / kBP); a.G = H; a.N = K; a.seg = seg;
  return launch_bwd<kBwdGla>(a, ws, ws_bytes, stream);
}

}  // namespace lr
