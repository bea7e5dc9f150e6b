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
//   h_next   = 2^cum_end h_prev + sum_s B_s (2^(cum_end - cum_s) phi_s x_s)^T
// The contractions run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
// y is computed transposed (rows p, columns t): the state accumulators are
// then directly the A operand of h_prev C^T, each lane ends with four
// consecutive p of one token (one 8-byte store), and D x is folded into the
// diagonal of M (y_t = sum_s (M[t][s] + D delta_ts) x_s + ...).
// The state h stays in accumulator registers for the whole sequence (wave w
// owns columns p in [16w, 16w+16) for all n); it goes to memory only for the
// optional checkpoints and the final state.  The 10 causal C B^T tiles of
// the decayed mask M are split over the waves and shared through LDS.
// Every input tile sits in LDS exactly as it lies in memory (token rows):
// operands whose contraction runs over tokens (x in M X, B and the
// decay-weighted x in the state update) are read with gfx950's transposing
// LDS read, so staging is a plain 16-byte copy.  One LDS buffer (66 KB):
// block k+1, loaded from HBM into registers during block k, is written into
// it once block k is done.  Row pitches are
// chosen per tile for its read pattern (see ChunkBuf).
//
// When the grid leaves CUs idle the sequence is cut into parts that run side
// by side.  The parts' end states from a zero start and their decay
// products come from a state-only pre-pass (SO); every part then folds those
// of the parts before it into its entering state with the combine
// (a2, b2) o (a1, b1) = (a2 a1, a2 b1 + b2) ("K-Search for MLX" blog,
// section "A 20x faster prefill", combine equation), applied to whole parts.
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace lr {

constexpr int kCQ = 64;        // tokens per block
constexpr int kCPS = 64;       // p columns per workgroup
constexpr int kLdM = kCQ + 8;  // pitch of M[t][s] (36 words: conflict-free 16-byte reads)

enum { kModeSsdZoh = 0, kModeSsdEuler = 1, kModeGla = 2, kModeSsdBilinear = 3, kModeSsdDirac = 4 };

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
  // Sequence split: part q covers blocks [q bpp, (q + 1) bpp).  part_state
  // [q][B][H][P][N] holds the state at the end of part q started from zero,
  // part_dec [q][B][H] the product of its decays (parts 0 .. nparts - 2).
  float* part_state;
  float* part_dec;
  int64_t nparts;       // parts of the sequence
  int64_t bpp;          // 64-token blocks per part
  int64_t grid_parts;   // parts covered by this launch (main: nparts, pre-pass: nparts - 1)
};

// One block of inputs in LDS, token-major.  Every row starts 16-byte
// aligned; pitches in 4-byte words are, mod 32:
//   Cs: 4  -> the 16-byte reads of C B^T are conflict-free
//   Bs: 8  -> the transposing reads of the state update are conflict-free
//   Xs, Xw: 8 (transposing reads only)
template <int NS>
struct ChunkBuf {
  static constexpr int kLdC = NS + 8;
  static constexpr int kLdB = NS + 16;
  static constexpr int kLdX = kCPS + 16;
  uint16_t Cs[kCQ * kLdC];     // C[t][n]
  uint16_t Bs[kCQ * kLdB];     // B[s][n]
  uint16_t Xs[kCQ * kLdX];     // x[s][p]
  uint16_t Xw[kCQ * kLdX];     // 2^(cum_end - cum_s) phi_s x[s][p]
  float cum[kCQ];
  float phi[kCQ];
  float sg[kCQ];               // bilinear only: sign of the decay product up to t
};

// Per-token log2-decay, input scale and (bilinear only) decay of one token.
// The bilinear decay (1 + l/2)/(1 - l/2) is negative for l < -2: its
// magnitude goes into the log2 sum and its sign into a parity scan.
template <int MODE>
__device__ __forceinline__ void chunk_scalars(uint16_t graw, bool ok, float Ah, float& l2, float& ph,
                                              float& ad) {
  ad = 1.f;
  if (MODE == kModeGla) {
    const float gv = ok ? bf2f(graw) : 1.f;
    l2 = fast_log2(gv);
    ph = ok ? 1.f : 0.f;
  } else if (MODE == kModeSsdBilinear) {
    const float dtv = ok ? bf2f(graw) : 0.f;
    const float r = __builtin_amdgcn_rcpf(1.f - 0.5f * dtv * Ah);
    ad = (1.f + 0.5f * dtv * Ah) * r;
    l2 = fmaxf(fast_log2(fabsf(ad)), -126.f);
    ph = dtv * r;
  } else if (MODE == kModeSsdDirac) {
    const float dtv = ok ? bf2f(graw) : 0.f;
    l2 = dtv * Ah * kLog2e;
    ph = ok ? 1.f : 0.f;
  } else {
    const float dtv = ok ? bf2f(graw) : 0.f;
    const float lam = dtv * Ah;
    l2 = lam * kLog2e;
    if (MODE == kModeSsdEuler) {
      ph = dtv;
    } else {
      const float ser = dtv * fmaf(lam, fmaf(lam, fmaf(lam, 1.f / 24.f, 1.f / 6.f), 0.5f), 1.f);
      ph = fabsf(lam) < 0.1f ? ser : (fast_exp2(l2) - 1.f) / Ah;
    }
  }
}

// SO (state only): the pre-pass of a split sequence; it skips C, the mask and
// the outputs and writes the part's end state and decay product.
template <int MODE, int NS, bool SO>
__global__ __launch_bounds__(256) void chunk_fwd_kernel(ChunkFwdArgs g) {
  constexpr int NT = NS / 16;     // 16-row tiles of n
  constexpr int NK = NS / 32;     // 32-wide k steps over n
  constexpr int kLdC = ChunkBuf<NS>::kLdC, kLdB = ChunkBuf<NS>::kLdB, kLdX = ChunkBuf<NS>::kLdX;
  // staged 16-byte chunks per thread: row = token, 8 columns per chunk
  constexpr int kRowCB = NS / 8, kRowX = kCPS / 8;
  constexpr int kCB = kCQ * kRowCB / 256;   // C, B
  constexpr int kXC = kCQ * kRowX / 256;    // x
  // One input buffer: the next block is staged after the current one is
  // done (66 KB of LDS).
  __shared__ ChunkBuf<NS> sm[1];
  __shared__ uint16_t Ms[SO ? 8 : kCQ * kLdM];   // M[t][s]

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int g4 = lane >> 4, c16 = lane & 15;

  const int64_t nps = g.P / kCPS;
  const int64_t wid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t part = wid % g.grid_parts;
  const int64_t ps = (wid / g.grid_parts) % nps;
  const int64_t bh = (wid / g.grid_parts) / nps;
  const int64_t h = bh % g.H;
  const int64_t b = bh / g.H;
  const int64_t grp = (MODE == kModeGla) ? h : h / (g.H / g.G);
  const int64_t xrow = g.H * g.P;               // elements between tokens of x / y
  const float Ah = (MODE == kModeGla) ? 0.f : g.A[h];
  const float Dh = (MODE == kModeGla || g.Dskip == nullptr) ? 0.f : g.Dskip[h];
  // per-thread base pointers (token 0 of this batch row, this workgroup's columns)
  const uint16_t* xb = g.x + b * g.L * xrow + h * g.P + ps * kCPS;
  uint16_t* yb = g.y + b * g.L * xrow + h * g.P + ps * kCPS;
  const uint16_t* Cb = g.Cm + b * g.L * g.bc_row + grp * NS;
  const uint16_t* Bb = g.Bm + b * g.L * g.bc_row + grp * NS;
  const uint16_t* gb = g.gate + b * g.L * g.H + h;

  // state accumulators: hacc[nt] holds h[n = 16 nt + 4 g4 + r][p = 16 w + c16]
  f32x4 hacc[NT];
  const int64_t sbase = (b * g.H + h) * g.P * NS;
  const int64_t pcol = ps * kCPS + 16 * w + c16;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t n = 16 * nt + 4 * g4 + r;
      hacc[nt][r] = (!SO && g.h0) ? g.h0[sbase + pcol * g.st_p + n * g.st_n] : 0.f;
    }
  }
  // the state entering this part: fold the earlier parts' end states with the
  // combine (h <- dec_q h + state_q), in order
  const int64_t pstride = g.B * g.H * g.P * NS;
  if (!SO) {
    for (int64_t q = 0; q < part; ++q) {
      const float dq = g.part_dec[q * g.B * g.H + b * g.H + h];
      const float* sq = g.part_state + q * pstride + sbase + pcol * NS + 4 * g4;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(sq + 16 * nt);
#pragma unroll
        for (int r = 0; r < 4; ++r) hacc[nt][r] = fmaf(dq, hacc[nt][r], v[r]);
      }
    }
  }

  const int64_t nblk_all = (g.L + kCQ - 1) / kCQ;
  const int64_t blk_lo = part * g.bpp;
  const int64_t nblk = (blk_lo + g.bpp < nblk_all) ? blk_lo + g.bpp : nblk_all;   // end block

  // ---- register staging of one block: chunk q = tid + 256 k is token
  // q / kRow, columns 8 (q % kRow) .. + 7 (consecutive lanes read consecutive
  // 16 bytes of a row; 32-bit offsets inside the block)
  u16x8 creg[kCB], breg[kCB], xreg[kXC];
  uint16_t greg = 0;
  // byte offsets from the block's first token (unsigned 32-bit: the loads
  // take the wave-uniform block base as their 64-bit address)
  uint32_t cboff[kCB], xoffl[kXC];
#pragma unroll
  for (int k = 0; k < kCB; ++k) {
    const int q = tid + 256 * k;
    cboff[k] = 2u * ((q / kRowCB) * static_cast<uint32_t>(g.bc_row) + 8 * (q % kRowCB));
  }
#pragma unroll
  for (int k = 0; k < kXC; ++k) {
    const int q = tid + 256 * k;
    xoffl[k] = 2u * ((q / kRowX) * static_cast<uint32_t>(xrow) + 8 * (q % kRowX));
  }
  auto ld16 = [](const uint16_t* base, uint32_t off) {
    return *reinterpret_cast<const u16x8*>(reinterpret_cast<const char*>(base) + off);
  };
  auto prefetch = [&](int64_t blk) {
    const int64_t t0 = blk * kCQ;
    const int nv = static_cast<int>((g.L - t0) < kCQ ? (g.L - t0) : kCQ);
    const uint16_t* cblk = Cb + t0 * g.bc_row;
    const uint16_t* bblk = Bb + t0 * g.bc_row;
    const uint16_t* xblk = xb + t0 * xrow;
    if (nv == kCQ) {   // full block: no bounds
#pragma unroll
      for (int k = 0; k < kCB; ++k) {
        if constexpr (!SO) creg[k] = ld16(cblk, cboff[k]);
        breg[k] = ld16(bblk, cboff[k]);
      }
#pragma unroll
      for (int k = 0; k < kXC; ++k) xreg[k] = ld16(xblk, xoffl[k]);
    } else {
#pragma unroll
      for (int k = 0; k < kCB; ++k) {
        const int row = (tid + 256 * k) / kRowCB;
        creg[k] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        breg[k] = creg[k];
        if (row < nv) {
          if constexpr (!SO) creg[k] = ld16(cblk, cboff[k]);
          breg[k] = ld16(bblk, cboff[k]);
        }
      }
#pragma unroll
      for (int k = 0; k < kXC; ++k) {
        const int row = (tid + 256 * k) / kRowX;
        xreg[k] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        if (row < nv) xreg[k] = ld16(xblk, xoffl[k]);
      }
    }
    greg = (lane < nv) ? gb[(t0 + lane) * g.H] : uint16_t(0);
  };

  // ---- registers -> LDS buffer for block blk (scalars from the gates every
  // wave holds, scan done redundantly per wave; lane = token)
  auto stage = [&](int64_t blk, ChunkBuf<NS>& bf) {
    const int64_t t0 = blk * kCQ;
    const int nv = static_cast<int>((g.L - t0) < kCQ ? (g.L - t0) : kCQ);
    float l2, ph, ad;
    chunk_scalars<MODE>(greg, lane < nv, Ah, l2, ph, ad);
    const float c = wave_incl_sum(l2);
    const float cend = __shfl(c, 63);
    float sgc = 1.f, sge = 1.f;
    if constexpr (MODE == kModeSsdBilinear) {
      const float nneg = wave_incl_sum(ad < 0.f ? 1.f : 0.f);
      sgc = (static_cast<int>(nneg) & 1) ? -1.f : 1.f;
      sge = __shfl(sgc, 63);
    }
    // weight of token `lane` in the state update
    const float wsc = fast_exp2(cend - c) * ph * (sgc * sge);
    if (w == 0) {
      bf.cum[lane] = c;
      bf.phi[lane] = ph;
      bf.sg[lane] = sgc;
    }
#pragma unroll
    for (int k = 0; k < kCB; ++k) {
      const int q = tid + 256 * k, row = q / kRowCB, col = 8 * (q % kRowCB);
      if constexpr (!SO) *reinterpret_cast<u16x8*>(bf.Cs + row * kLdC + col) = creg[k];
      *reinterpret_cast<u16x8*>(bf.Bs + row * kLdB + col) = breg[k];
    }
#pragma unroll
    for (int k = 0; k < kXC; ++k) {
      const int q = tid + 256 * k, row = q / kRowX, col = 8 * (q % kRowX);
      const float ws = __shfl(wsc, row);
      u16x8 xw;
#pragma unroll
      for (int i = 0; i < 8; ++i) xw[i] = f2bf(bf2f(xreg[k][i]) * ws);
      *reinterpret_cast<u16x8*>(bf.Xs + row * kLdX + col) = xreg[k];
      *reinterpret_cast<u16x8*>(bf.Xw + row * kLdX + col) = xw;
    }
  };

  if (blk_lo < nblk) {
    prefetch(blk_lo);
    stage(blk_lo, sm[0]);
    if (blk_lo + 1 < nblk) prefetch(blk_lo + 1);
  }
  __syncthreads();

  // checkpoint s (the state entering token s * seg) goes to ckpt + s * ck_step
  const int64_t ck_step = g.B * g.H * g.P * NS;
  float* ck_base = (!SO && g.ckpt != nullptr) ? g.ckpt + sbase + pcol * NS + 4 * g4 : nullptr;
  float dprod = 1.f;   // SO: product of the part's block decays
  // per-lane byte offset of this lane's 4 outputs of token c16 in a 16-token tile
  const uint32_t yoff = 2u * (static_cast<uint32_t>(c16) * static_cast<uint32_t>(xrow) + 16 * w + 4 * g4);

  for (int64_t blk = blk_lo; blk < nblk; ++blk) {
    ChunkBuf<NS>& cur = sm[0];
    const int64_t t0 = blk * kCQ;
    const int nv = static_cast<int>((g.L - t0) < kCQ ? (g.L - t0) : kCQ);

    if (ck_base != nullptr && t0 % g.seg == 0) {
      float* ck = ck_base + (t0 / g.seg) * ck_step;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) *reinterpret_cast<f32x4*>(ck + 16 * nt) = hacc[nt];
    }
    if constexpr (!SO) {

    // ---- decayed causal mask M[t][s]: 12 tiles of 16x16 (3 per wave), the
    //      10 with s-tile <= t-tile plus the all-zero (0,1) and (2,3) that
    //      complete the 32-wide k steps of M X
    {
      // Each wave's three tiles are fixed at compile time, so a C or B tile
      // that several of them share is read from LDS once per k step.
      auto tiles = [&](auto ta, auto sa, auto tb, auto sb, auto tc, auto sc) {
        constexpr int TI[3] = {decltype(ta)::value, decltype(tb)::value, decltype(tc)::value};
        constexpr int SI[3] = {decltype(sa)::value, decltype(sb)::value, decltype(sc)::value};
        f32x4 z[3];
#pragma unroll
        for (int q = 0; q < 3; ++q) z[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          bf16x8 cop[3], bop[3];
#pragma unroll
          for (int q = 0; q < 3; ++q) {
            if (SI[q] > TI[q]) continue;
            bool cre = false, bre = false;
#pragma unroll
            for (int r = 0; r < q; ++r) {
              if (SI[r] > TI[r]) continue;
              if (!cre && TI[r] == TI[q]) { cop[q] = cop[r]; cre = true; }
              if (!bre && SI[r] == SI[q]) { bop[q] = bop[r]; bre = true; }
            }
            if (!cre) cop[q] = lds_tile(cur.Cs, kLdC, 16 * TI[q], 32 * kk, lane);
            if (!bre) bop[q] = lds_tile(cur.Bs, kLdB, 16 * SI[q], 32 * kk, lane);
            z[q] = mfma16x16x32(bop[q], cop[q], z[q]);
          }
        }
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          const int ti = TI[q], si = SI[q];
          const int t = 16 * ti + c16;           // this lane's column of Z^T
          const int s0 = 16 * si + 4 * g4;       // this lane's 4 rows of Z^T
          u16x4 out = {0, 0, 0, 0};
          if (si <= ti) {
            const float ct = cur.cum[t];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int sr = s0 + r;
              // unconditional loads, then a select (no per-lane branches
              // around LDS reads; a non-finite value above the diagonal is discarded)
              float m = z[q][r] * fast_exp2(ct - cur.cum[sr]) * cur.phi[sr];
              if (MODE == kModeSsdBilinear) m *= cur.sg[t] * cur.sg[sr];
              m = (sr <= t) ? m : 0.f;
              if (sr == t) m += Dh;   // D x_t folded into the diagonal
              out[r] = f2bf(m);
            }
          }
          *reinterpret_cast<u16x4*>(Ms + t * kLdM + s0) = out;
        }
      };
      using I0 = std::integral_constant<int, 0>;
      using I1 = std::integral_constant<int, 1>;
      using I2 = std::integral_constant<int, 2>;
      using I3 = std::integral_constant<int, 3>;
      const int wu = __builtin_amdgcn_readfirstlane(w);   // wave-uniform branch
      // (t tile, s tile): 4 operand tiles per k step for waves 0-2, 2 for wave 3,
      // which also writes the zero tiles (0,1) and (2,3)
      if (wu == 0) tiles(I3{}, I0{}, I3{}, I1{}, I3{}, I2{});
      else if (wu == 1) tiles(I2{}, I0{}, I2{}, I1{}, I2{}, I2{});
      else if (wu == 2) tiles(I1{}, I0{}, I1{}, I1{}, I0{}, I0{});
      else tiles(I3{}, I3{}, I0{}, I1{}, I2{}, I3{});
    }
    __syncthreads();

    // ---- y^T[p][t] = 2^cum_t (h_prev C^T)[p][t] + (X^T M^T)[p][t]
    //      lane holds p = 16 w + 4 g4 + r, t = 16 ti + c16
    f32x4 yacc[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) yacc[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const bf16x8 hb = pack_dd(hacc[2 * kk], hacc[2 * kk + 1]);
#pragma unroll
      for (int ti = 0; ti < 4; ++ti)
        yacc[ti] = mfma16x16x32(hb, lds_tile_perm(cur.Cs, kLdC, 16 * ti, 32 * kk, lane), yacc[ti]);
    }
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      const int t = 16 * ti + c16;
      yacc[ti] *= (MODE == kModeSsdBilinear) ? fast_exp2(cur.cum[t]) * cur.sg[t] : fast_exp2(cur.cum[t]);
    }
    {
      const bf16x8 x0 = lds_tile_tr(cur.Xs, kLdX, 0, 16 * w, lane);
      const bf16x8 x1 = lds_tile_tr(cur.Xs, kLdX, 32, 16 * w, lane);
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        yacc[ti] = mfma16x16x32(x0, lds_tile(Ms, kLdM, 16 * ti, 0, lane), yacc[ti]);
        if (ti >= 2) yacc[ti] = mfma16x16x32(x1, lds_tile(Ms, kLdM, 16 * ti, 32, lane), yacc[ti]);
      }
    }
    {
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        char* yt = reinterpret_cast<char*>(yb + (t0 + 16 * ti) * xrow);
        if (16 * ti + c16 < nv) {
          const u16x4 v = {f2bf(yacc[ti][0]), f2bf(yacc[ti][1]), f2bf(yacc[ti][2]), f2bf(yacc[ti][3])};
          *reinterpret_cast<u16x4*>(yt + yoff) = v;
        }
      }
    }

    }   // !SO

    // ---- h_next = 2^cum_end h_prev + B^T (decay-weighted x)
    {
      const float dec = (MODE == kModeSsdBilinear) ? fast_exp2(cur.cum[kCQ - 1]) * cur.sg[kCQ - 1]
                                                   : fast_exp2(cur.cum[kCQ - 1]);
      const bf16x8 xw0 = lds_tile_tr(cur.Xw, kLdX, 0, 16 * w, lane);
      const bf16x8 xw1 = lds_tile_tr(cur.Xw, kLdX, 32, 16 * w, lane);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        hacc[nt] *= dec;
        hacc[nt] = mfma16x16x32(lds_tile_tr(cur.Bs, kLdB, 0, 16 * nt, lane), xw0, hacc[nt]);
        hacc[nt] = mfma16x16x32(lds_tile_tr(cur.Bs, kLdB, 32, 16 * nt, lane), xw1, hacc[nt]);
      }
      dprod *= dec;
    }
    __syncthreads();
    // the next block into the buffer (every wave is done with it), the one
    // after into registers
    if (blk + 1 < nblk) {
      stage(blk + 1, sm[0]);
      if (blk + 2 < nblk) prefetch(blk + 2);
      __syncthreads();
    }
  }

  if constexpr (SO) {
    float* out = g.part_state + part * pstride + sbase + pcol * NS + 4 * g4;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) *reinterpret_cast<f32x4*>(out + 16 * nt) = hacc[nt];
    if (tid == 0) g.part_dec[part * g.B * g.H + b * g.H + h] = dprod;
    return;
  }
  if (g.h_last != nullptr && nblk == nblk_all) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t n = 16 * nt + 4 * g4 + r;
        g.h_last[sbase + pcol * g.st_p + n * g.st_n] = hacc[nt][r];
      }
  }
}

// Sequence split of the forward: when the grid leaves CUs idle (fewer than
// 256 workgroups, MI355X's CU count) the sequence is cut into parts of at
// least 8 blocks, up to 512 workgroups, each run by its own workgroups from
// the state the pre-pass and the fold give it.  A grid with a workgroup for
// every CU runs unsplit: a second workgroup on a CU adds only about a fifth
// to its throughput (every phase of a block slows down), less than the
// pre-pass costs.  Workspace: the parts' end states and decay products.
struct ChunkSplit { int64_t nblk, nparts, bpp, dec_off; size_t bytes; };
static ChunkSplit chunk_split(int64_t B, int64_t L, int64_t H, int64_t P, int64_t NS) {
  ChunkSplit sp;
  sp.nblk = (L + kCQ - 1) / kCQ;
  const int64_t nwg = B * H * (P / kCPS);
  int64_t want = nwg > 0 && nwg < 256 ? (512 + nwg - 1) / nwg : 1;
  const int64_t cap = sp.nblk / 8 > 1 ? sp.nblk / 8 : 1;
  if (want > cap) want = cap;
  if (want > 16) want = 16;
  if (want < 1) want = 1;
  sp.bpp = sp.nblk > 0 ? (sp.nblk + want - 1) / want : 1;
  sp.nparts = sp.nblk > 0 ? (sp.nblk + sp.bpp - 1) / sp.bpp : 1;
  const int64_t st = (sp.nparts - 1) * B * H * P * NS * 4;
  sp.dec_off = (st + 255) & ~int64_t(255);
  sp.bytes = sp.nparts > 1 ? static_cast<size_t>(sp.dec_off + (sp.nparts - 1) * B * H * 4) : 0;
  return sp;
}

size_t ssd_fwd_workspace(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N) {
  return chunk_split(B, L, H, P, N).bytes;
}
size_t gla_fwd_workspace(int64_t B, int64_t L, int64_t H, int64_t K, int64_t V) {
  return chunk_split(B, L, H, V, K).bytes;
}

template <int MODE, int NS>
static hipError_t launch_chunk(ChunkFwdArgs a, void* ws, size_t ws_bytes, hipStream_t stream) {
  const int64_t nwg = a.B * a.H * (a.P / kCPS);
  const ChunkSplit sp = chunk_split(a.B, a.L, a.H, a.P, NS);
  a.nparts = 1;
  a.bpp = sp.nblk > 0 ? sp.nblk : 1;
  a.part_state = nullptr;
  a.part_dec = nullptr;
  if (ws != nullptr && sp.nparts > 1 && ws_bytes >= sp.bytes) {
    a.nparts = sp.nparts;
    a.bpp = sp.bpp;
    a.part_state = static_cast<float*>(ws);
    a.part_dec = reinterpret_cast<float*>(static_cast<char*>(ws) + sp.dec_off);
    a.grid_parts = a.nparts - 1;   // pre-pass: the end states of parts 0 .. nparts - 2
    hipLaunchKernelGGL((chunk_fwd_kernel<MODE, NS, true>),
                       dim3(static_cast<unsigned>(nwg * a.grid_parts)), dim3(256), 0, stream, a);
  }
  a.grid_parts = a.nparts;
  hipLaunchKernelGGL((chunk_fwd_kernel<MODE, NS, false>),
                     dim3(static_cast<unsigned>(nwg * a.nparts)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_ssd_fwd(int disc, const void* x, const void* dt, const float* A, const void* Bm,
                          const void* Cm, const float* Dskip, const float* h0, void* y,
                          float* h_last, float* ckpt, int64_t B, int64_t L, int64_t H, int64_t P,
                          int64_t G, int64_t N, int64_t seg, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
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
  if (N == 128) {
    switch (disc) {
      case 1: return launch_chunk<kModeSsdEuler, 128>(a, ws, ws_bytes, stream);
      case 2: return launch_chunk<kModeSsdBilinear, 128>(a, ws, ws_bytes, stream);
      case 3: return launch_chunk<kModeSsdDirac, 128>(a, ws, ws_bytes, stream);
      default: return launch_chunk<kModeSsdZoh, 128>(a, ws, ws_bytes, stream);
    }
  }
  switch (disc) {
    case 1: return launch_chunk<kModeSsdEuler, 64>(a, ws, ws_bytes, stream);
    case 2: return launch_chunk<kModeSsdBilinear, 64>(a, ws, ws_bytes, stream);
    case 3: return launch_chunk<kModeSsdDirac, 64>(a, ws, ws_bytes, stream);
    default: return launch_chunk<kModeSsdZoh, 64>(a, ws, ws_bytes, stream);
  }
}

// ---------------------------------------------------------------------------
// Static scratch of lr_ssd_scan_noalloc: the sequence split's part states and
// decay products live in this file-scope device array instead of a caller
// workspace, so the call allocates nothing.  Each GPU the library runs on
// holds its own copy (16 MiB) until the process ends.  For N <= 128 the
// split never needs more: its parts times workgroups stay below 512, so the
// part states take at most 511 * 64 * 128 * 4 bytes plus 511 decays.
// Host code reaches the array only through the address hipGetSymbolAddress
// returns for the current device (the array's name is a host-side stand-in).
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch[kMaxScratchDevices];
}  // namespace

size_t ssd_noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

// Device address of `scratch` on the current device, looked up once per
// device (two threads racing on the first call store the same address).
hipError_t ssd_noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_gla_fwd(const void* q, const void* k, const void* v, const void* gate,
                          const float* S0, void* o, float* S_last, float* ckpt, int64_t B,
                          int64_t L, int64_t H, int64_t K, int64_t V, int64_t seg, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
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
  a.ckpt = seg > 0 ? ckpt : nullptr;   // [nseg][B][H][V][K]: the state transposed
  a.B = B; a.L = L; a.H = H; a.P = V; a.G = H; a.seg = seg > 0 ? seg : 1;
  a.bc_row = H * K;
  a.st_p = 1; a.st_n = V;
  if (K == 128) return launch_chunk<kModeGla, 128>(a, ws, ws_bytes, stream);
  return launch_chunk<kModeGla, 64>(a, ws, ws_bytes, stream);
}

}  // namespace lr
