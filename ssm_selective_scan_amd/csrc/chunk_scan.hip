// chunk_scan.hip — chunked forward scan for Mamba-2 SSD and GLA on MFMA.
//
// Both recurrences have a scalar decay per (token, head) and a rank-1 write:
//   SSD ("mlx-recurrence" post, ssd_scan, state [B, H, Dh, N]):
//       h <- e_t h + phi_t x_t B_t^T,   y_t = h C_t + D x_t
//   GLA ("mlx-recurrence" post, gla_scan, state [B, H, Dh, Dh]):
//       S <- g_t S + k_t v_t^T,         o_t = S^T q_t
// With the roles x <-> v, B <-> k, C <-> q, phi = 1 and log-decay log2(g) for
// GLA, one kernel serves both.  Notation below is SSD's: the state is
// h[p][n] (p < P columns written by x, n < N rows read by C).
//
// One workgroup (4 waves) owns one (batch, head, 64-wide slice of p) and walks
// the sequence in 64-token blocks in a single launch.  Per block, with cum
// the inclusive prefix sum of the log2-decays inside the block (a DPP wave
// scan) and decays always formed as 2^(cum_t - cum_s) of differences:
//   M[t][s]  = (C_t . B_s) 2^(cum_t - cum_s) phi_s  for s <= t, else 0
//   y_t      = 2^cum_t (C_t . h_prev) + sum_s M[t][s] x_s + D x_t
//   h_next   = 2^cum_end h_prev + sum_s 2^(cum_end - cum_s) phi_s x_s B_s^T
// The four contractions (C B^T, M X, C h, B_w^T X) run on
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation; the state h stays in
// MFMA accumulator registers for the whole sequence (wave w owns columns
// p in [16w, 16w+16) for all n), so it never goes to memory except for the
// optional checkpoints and the final state.  Inputs are staged through LDS
// in k-contiguous layouts (B also transposed and pre-scaled for the state
// update; x transposed), and the decayed mask M goes through LDS so every
// wave can use it for its p columns.
#include "common.hpp"

namespace lr {

constexpr int kCQ = 64;    // tokens per block
constexpr int kCPS = 64;   // p columns per workgroup
constexpr int kLdT = kCQ + 8;  // leading dim of token-contiguous LDS tiles

enum { kModeSsdZoh = 0, kModeSsdEuler = 1, kModeGla = 2 };

struct ChunkFwdArgs {
  const uint16_t* x;    // SSD x / GLA v      [B, L, H, P]
  const uint16_t* gate; // SSD dt / GLA g     [B, L, H]
  const float* A;       // SSD only           [H]
  const uint16_t* Bm;   // SSD B / GLA k      [B, L, G, N] / [B, L, H, K]
  const uint16_t* Cm;   // SSD C / GLA q
  const float* Dskip;   // SSD only, may be null
  const float* h0;      // may be null
  uint16_t* y;          // [B, L, H, P]
  float* h_last;        // may be null
  float* ckpt;          // SSD only, may be null
  int64_t B, L, H, P, G, seg;
  int64_t bc_row;       // elements between consecutive tokens of Bm/Cm
  int64_t st_p, st_n;   // state strides of p and n (SSD: N, 1; GLA: 1, V)
};

template <int NS>
struct ChunkLds {
  static constexpr int kLdN = NS + 8;
  uint16_t Cs[kCQ * kLdN];     // C[t][n]
  uint16_t Bs[kCQ * kLdN];     // B[s][n]
  uint16_t BwT[NS * kLdT];     // B[s][n] 2^(cum_end - cum_s) phi_s, as [n][s]
  uint16_t XT[kCPS * kLdT];    // x[s][p], as [p][s]
  uint16_t Ms[kCQ * kLdT];     // M[t][s]
  float cum[kCQ];
  float phi[kCQ];
};

template <int MODE, int NS>
__global__ __launch_bounds__(256) void chunk_fwd_kernel(ChunkFwdArgs g) {
  constexpr int NT = NS / 16;     // 16-row tiles of n
  constexpr int NK = NS / 32;     // 32-wide k steps over n
  constexpr int kLdN = ChunkLds<NS>::kLdN;
  __shared__ ChunkLds<NS> sm;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int g4 = lane >> 4, c16 = lane & 15;

  const int64_t nps = g.P / kCPS;
  const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t ps = wid % nps;
  const int64_t bh = wid / nps;
  const int64_t h = bh % g.H;
  const int64_t b = bh / g.H;
  const int64_t grp = (MODE == kModeGla) ? h : h / (g.H / g.G);
  const int64_t xrow = g.H * g.P;               // elements between tokens of x / y
  const int64_t xoff = h * g.P + ps * kCPS;     // this workgroup's columns
  const int64_t bcoff = grp * NS;
  const float Ah = (MODE == kModeGla) ? 0.f : g.A[h];
  const float Dh = (MODE == kModeGla || g.Dskip == nullptr) ? 0.f : g.Dskip[h];

  // state accumulators: hacc[nt] holds h[n = 16 nt + 4 g4 + r][p = 16 w + c16]
  f32x4 hacc[NT];
  const int64_t sbase = (b * g.H + h) * g.P * NS;
  const int64_t pcol = ps * kCPS + 16 * w + c16;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t n = 16 * nt + 4 * g4 + r;
      hacc[nt][r] = g.h0 ? g.h0[sbase + pcol * g.st_p + n * g.st_n] : 0.f;
    }
  }

  const int64_t nblk = (g.L + kCQ - 1) / kCQ;

  // Register staging of one block: C and B rows (NS/32 16-byte chunks of each
  // per thread), x (2 chunks per thread, lanes walk tokens) and the gate
  // (wave 0, lane = token).  The next block's loads are issued as soon as
  // the current block is in LDS, so their latency overlaps the MFMA work.
  constexpr int kCB = (kCQ * (NS / 8)) / 256;
  constexpr int kXC = (kCQ * (kCPS / 8)) / 256;
  u16x8 creg[kCB], breg[kCB], xreg[kXC];
  uint16_t greg = 0;
  int nv_next = 0;
  auto prefetch = [&](int64_t blk) {
    const int64_t t0 = blk * kCQ;
    const int nv = static_cast<int>((g.L - t0) < kCQ ? (g.L - t0) : kCQ);
    nv_next = nv;
#pragma unroll
    for (int k = 0; k < kCB; ++k) {
      const int idx = tid + 256 * k;
      const int r = idx / (NS / 8), c = idx % (NS / 8);
      creg[k] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      breg[k] = creg[k];
      if (r < nv) {
        const int64_t off = (b * g.L + t0 + r) * g.bc_row + bcoff + 8 * c;
        creg[k] = *reinterpret_cast<const u16x8*>(g.Cm + off);
        breg[k] = *reinterpret_cast<const u16x8*>(g.Bm + off);
      }
    }
#pragma unroll
    for (int k = 0; k < kXC; ++k) {
      const int idx = tid + 256 * k;
      const int s = idx & 63, c = idx >> 6;
      xreg[k] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (s < nv) xreg[k] = *reinterpret_cast<const u16x8*>(g.x + (b * g.L + t0 + s) * xrow + xoff + 8 * c);
    }
    if (w == 0 && lane < nv) greg = g.gate[(b * g.L + t0 + lane) * g.H + h];
  };
  if (nblk > 0) prefetch(0);

  for (int64_t blk = 0; blk < nblk; ++blk) {
    const int64_t t0 = blk * kCQ;
    const int nv = nv_next;

    if (g.ckpt != nullptr && (t0 % g.seg) == 0) {
      float* cp = g.ckpt + ((t0 / g.seg) * g.B * g.H) * g.P * NS + sbase;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        *reinterpret_cast<f32x4*>(cp + pcol * NS + 16 * nt + 4 * g4) = hacc[nt];
    }

    // ---- per-token decay and input scale (wave 0, lane = token)
    if (w == 0) {
      const bool ok = lane < nv;
      float l2, ph;
      if (MODE == kModeGla) {
        const float gv = ok ? bf2f(greg) : 1.f;
        l2 = fast_log2(gv);
        ph = ok ? 1.f : 0.f;
      } else {
        const float dtv = ok ? bf2f(greg) : 0.f;
        const float lam = dtv * Ah;
        l2 = lam * kLog2e;
        if (MODE == kModeSsdEuler) {
          ph = dtv;
        } else {
          const float ser = dtv * fmaf(lam, fmaf(lam, fmaf(lam, 1.f / 24.f, 1.f / 6.f), 0.5f), 1.f);
          ph = fabsf(lam) < 0.1f ? ser : (fast_exp2(l2) - 1.f) / Ah;
        }
      }
      sm.cum[lane] = wave_incl_sum(l2);
      sm.phi[lane] = ph;
    }
    // ---- staged registers -> LDS: C, B row-major; x transposed XT[p][s]
#pragma unroll
    for (int k = 0; k < kCB; ++k) {
      const int idx = tid + 256 * k;
      const int r = idx / (NS / 8), c = idx % (NS / 8);
      *reinterpret_cast<u16x8*>(sm.Cs + r * kLdN + 8 * c) = creg[k];
      *reinterpret_cast<u16x8*>(sm.Bs + r * kLdN + 8 * c) = breg[k];
    }
#pragma unroll
    for (int k = 0; k < kXC; ++k) {
      const int idx = tid + 256 * k;
      const int s = idx & 63, c = idx >> 6;
#pragma unroll
      for (int i = 0; i < 8; ++i) sm.XT[(8 * c + i) * kLdT + s] = xreg[k][i];
    }
    __syncthreads();
    if (blk + 1 < nblk) prefetch(blk + 1);

    const float cum_end = sm.cum[kCQ - 1];
    // ---- B scaled by 2^(cum_end - cum_s) phi_s, transposed: BwT[n][s]
    for (int idx = tid; idx < kCQ * (NS / 8); idx += 256) {
      const int s = idx & 63, c = idx >> 6;
      const float ws = fast_exp2(cum_end - sm.cum[s]) * sm.phi[s];
      const u16x8 v = *reinterpret_cast<const u16x8*>(sm.Bs + s * kLdN + 8 * c);
#pragma unroll
      for (int i = 0; i < 8; ++i) sm.BwT[(8 * c + i) * kLdT + s] = f2bf(bf2f(v[i]) * ws);
    }
    // ---- decayed causal mask M[t][s]; 12 tiles of 16x16 (3 per wave):
    //      (t-tile, s-tile) with s-tile <= t-tile, plus the all-zero tiles
    //      (0,1) and (2,3) that complete the 32-wide k steps of M X.
    {
      const int ti_tab[12] = {0, 0, 1, 1, 2, 2, 2, 2, 3, 3, 3, 3};
      const int si_tab[12] = {0, 1, 0, 1, 0, 1, 2, 3, 0, 1, 2, 3};
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        const int ti = ti_tab[3 * w + q], si = si_tab[3 * w + q];
        const int t = 16 * ti + c16;           // this lane's column of Z^T
        const int s0 = 16 * si + 4 * g4;       // this lane's 4 rows of Z^T
        u16x4 out = {0, 0, 0, 0};
        if (si <= ti) {
          f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < NK; ++kk)
            z = mfma16x16x32(lds_tile(sm.Bs, kLdN, 16 * si, 32 * kk, lane),
                             lds_tile(sm.Cs, kLdN, 16 * ti, 32 * kk, lane), z);
          const float ct = sm.cum[t];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int s = s0 + r;
            const float m = (s <= t) ? z[r] * fast_exp2(ct - sm.cum[s]) * sm.phi[s] : 0.f;
            out[r] = f2bf(m);
          }
        }
        *reinterpret_cast<u16x4*>(sm.Ms + t * kLdT + s0) = out;
      }
    }
    __syncthreads();

    // ---- y = 2^cum_t (C_t . h_prev) + M X + D x
    f32x4 yacc[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) yacc[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const bf16x8 hb = pack_dd(hacc[2 * kk], hacc[2 * kk + 1]);
#pragma unroll
      for (int ti = 0; ti < 4; ++ti)
        yacc[ti] = mfma16x16x32(lds_tile_perm(sm.Cs, kLdN, 16 * ti, 32 * kk, lane), hb, yacc[ti]);
    }
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) yacc[ti][r] *= fast_exp2(sm.cum[16 * ti + 4 * g4 + r]);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks == 1 && ti < 2) continue;
        yacc[ti] = mfma16x16x32(lds_tile(sm.Ms, kLdT, 16 * ti, 32 * ks, lane),
                                lds_tile(sm.XT, kLdT, 16 * w, 32 * ks, lane), yacc[ti]);
      }
    }
    {
      const int p = 16 * w + c16;
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        const int tb = 16 * ti + 4 * g4;
        const u16x4 xv = *reinterpret_cast<const u16x4*>(sm.XT + p * kLdT + tb);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (tb + r < nv) {
            const float v = yacc[ti][r] + Dh * bf2f(xv[r]);
            g.y[(b * g.L + t0 + tb + r) * xrow + xoff + p] = f2bf(v);
          }
        }
      }
    }

    // ---- h_next = 2^cum_end h_prev + Bw^T X
    {
      const float dec = fast_exp2(cum_end);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        hacc[nt] *= dec;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          hacc[nt] = mfma16x16x32(lds_tile(sm.BwT, kLdT, 16 * nt, 32 * ks, lane),
                                  lds_tile(sm.XT, kLdT, 16 * w, 32 * ks, lane), hacc[nt]);
      }
    }
    __syncthreads();
  }

  if (g.h_last != nullptr) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t n = 16 * nt + 4 * g4 + r;
        g.h_last[sbase + pcol * g.st_p + n * g.st_n] = hacc[nt][r];
      }
  }
}

template <int MODE, int NS>
static hipError_t launch_chunk(const ChunkFwdArgs& a, hipStream_t stream) {
  const int64_t nwg = a.B * a.H * (a.P / kCPS);
  hipLaunchKernelGGL((chunk_fwd_kernel<MODE, NS>), dim3(static_cast<unsigned>(nwg)), dim3(256),
                     0, stream, a);
  return hipGetLastError();
}

hipError_t launch_ssd_fwd(int disc, const void* x, const void* dt, const float* A, const void* Bm,
                          const void* Cm, const float* Dskip, const float* h0, void* y,
                          float* h_last, float* ckpt, int64_t B, int64_t L, int64_t H, int64_t P,
                          int64_t G, int64_t N, int64_t seg, hipStream_t stream) {
  ChunkFwdArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.gate = static_cast<const uint16_t*>(dt);
  a.A = A;
  a.Bm = static_cast<const uint16_t*>(Bm);
  a.Cm = static_cast<const uint16_t*>(Cm);
  a.Dskip = Dskip;
  a.h0 = h0;
  a.y = static_cast<uint16_t*>(y);
  a.h_last = h_last;
  a.ckpt = seg > 0 ? ckpt : nullptr;
  a.B = B; a.L = L; a.H = H; a.P = P; a.G = G; a.seg = seg > 0 ? seg : 1;
  a.bc_row = G * N;
  a.st_p = N; a.st_n = 1;
  if (N == 128) return disc == 1 ? launch_chunk<kModeSsdEuler, 128>(a, stream)
                                 : launch_chunk<kModeSsdZoh, 128>(a, stream);
  return disc == 1 ? launch_chunk<kModeSsdEuler, 64>(a, stream)
                   : launch_chunk<kModeSsdZoh, 64>(a, stream);
}

hipError_t launch_gla_fwd(const void* q, const void* k, const void* v, const void* gate,
                          const float* S0, void* o, float* S_last, int64_t B, int64_t L,
                          int64_t H, int64_t K, int64_t V, hipStream_t stream) {
  ChunkFwdArgs a;
  a.x = static_cast<const uint16_t*>(v);
  a.gate = static_cast<const uint16_t*>(gate);
  a.A = nullptr;
  a.Bm = static_cast<const uint16_t*>(k);
  a.Cm = static_cast<const uint16_t*>(q);
  a.Dskip = nullptr;
  a.h0 = S0;
  a.y = static_cast<uint16_t*>(o);
  a.h_last = S_last;
  a.ckpt = nullptr;
  a.B = B; a.L = L; a.H = H; a.P = V; a.G = H; a.seg = 1;
  a.bc_row = H * K;
  a.st_p = 1; a.st_n = V;
  if (K == 128) return launch_chunk<kModeGla, 128>(a, stream);
  return launch_chunk<kModeGla, 64>(a, stream);
}

}  // namespace lr
