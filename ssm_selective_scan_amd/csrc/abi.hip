// abi.hip — the extern "C" boundary of liblr (declared in include/lr.h).
//
// Each entry point validates every argument without touching the device
// (the shape and argument checks of the "mlx-recurrence" post's shared
// chassis), then launches its kernel(s) on the caller's stream and maps a
// launch failure to LR_E_HIP.  No allocation and no synchronisation; the only
// global state is the per-device address of lr_ssd_scan_noalloc's static
// scratch array (chunk_scan.hip).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <limits>

#include "lr.h"

#include "launch.hpp"

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 46;   // per tensor; keeps every index in int64
constexpr int64_t kMaxGrid = std::numeric_limits<int32_t>::max();
constexpr int64_t kMaxSelD = int64_t(1) << 24;   // channels of lr_selective_scan
// elements between consecutive tokens of a chunked-scan input (G*N, H*P; GLA
// H*K, H*V): the kernels address up to 64 token rows of one block with
// unsigned 32-bit byte offsets (126 * 2^25 + a row < 2^32)
constexpr int64_t kMaxChunkRow = int64_t(1) << 25;

// Checked product of non-negative sizes; false on overflow.
bool mul_ok(int64_t& acc, int64_t v) {
  if (v < 0) return false;
  if (v != 0 && acc > std::numeric_limits<int64_t>::max() / v) return false;
  acc *= v;
  return true;
}

bool elems_ok(std::initializer_list<int64_t> dims) {
  int64_t n = 1;
  for (int64_t d : dims)
    if (!mul_ok(n, d)) return false;
  return n <= kMaxElems;
}

// A token row of n1 * n2 elements that the chunked kernels can address.
bool row_ok(int64_t n1, int64_t n2) {
  int64_t n = 1;
  return mul_ok(n, n1) && mul_ok(n, n2) && n <= kMaxChunkRow;
}

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool all_aligned(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p != nullptr && !aligned(p)) return false;
  return true;
}

bool any_null(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p == nullptr) return true;
  return false;
}

lr_status hip_status(hipError_t e) { return e == hipSuccess ? LR_OK : LR_E_HIP; }

bool valid_io(int io) { return io == LR_F32 || io == LR_BF16; }
bool valid_disc(int d) {
  return d == LR_DISC_ZOH || d == LR_DISC_EULER || d == LR_DISC_BILINEAR || d == LR_DISC_DIRAC;
}

// Checks shared by the SSD forward and backward.
lr_status check_ssd_sizes(int io, int disc, int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                          int64_t N, int64_t chunk, int64_t seg) {
  if (!valid_io(io) || !valid_disc(disc)) return LR_E_DTYPE;
  if (B < 0 || L < 0 || H < 1 || P < 1 || G < 1 || N < 1 || chunk < 1 || seg < 0) return LR_E_SHAPE;
  if (H % G != 0) return LR_E_SHAPE;
  if (io != LR_BF16) return LR_E_UNSUPPORTED;
  if (P % 64 != 0 || (N != 64 && N != 128) || chunk % 64 != 0 || seg % 64 != 0)
    return LR_E_UNSUPPORTED;
  if (seg > 0 && seg % chunk != 0) return LR_E_SHAPE;   // segments are whole chunks
  if (!elems_ok({B, L, H, P}) || !elems_ok({B, L, G, N}) || !elems_ok({B, H, P, N}))
    return LR_E_OVERFLOW;
  if (!row_ok(G, N) || !row_ok(H, P)) return LR_E_UNSUPPORTED;
  int64_t nwg = 1;
  if (!mul_ok(nwg, B) || !mul_ok(nwg, H) || !mul_ok(nwg, P / 64) || nwg > kMaxGrid)
    return LR_E_OVERFLOW;
  if (seg > 0) {
    const int64_t nseg = (L + seg - 1) / seg;
    if (!elems_ok({nseg, B, H, P, N})) return LR_E_OVERFLOW;
  }
  return LR_OK;
}

}  // namespace

extern "C" {

const char* lr_status_string(int s) {
  switch (s) {
    case LR_OK: return "LR_OK: success";
    case LR_E_NULLPTR: return "LR_E_NULLPTR: a required pointer is NULL";
    case LR_E_SHAPE: return "LR_E_SHAPE: invalid or inconsistent sizes";
    case LR_E_DTYPE: return "LR_E_DTYPE: unknown dtype or discretisation";
    case LR_E_ALIGN: return "LR_E_ALIGN: a pointer is not 16-byte aligned";
    case LR_E_UNSUPPORTED: return "LR_E_UNSUPPORTED: size or dtype outside the compiled set";
    case LR_E_WORKSPACE: return "LR_E_WORKSPACE: workspace missing or too small";
    case LR_E_OVERFLOW: return "LR_E_OVERFLOW: sizes overflow the supported index range";
    case LR_E_HIP: return "LR_E_HIP: the HIP runtime reported an error";
    default: return "unknown lr_status";
  }
}

const char* lr_version(void) { return "liblr 0.1.0 gfx950"; }

lr_status lr_diag_scan(lr_dtype io, int64_t B, int64_t L, int64_t D, const void* a, const void* b,
                       const float* h0, void* h, float* h_last, void* stream) {
  if (!valid_io(io)) return LR_E_DTYPE;
  if (B < 0 || L < 0 || D < 1) return LR_E_SHAPE;
  if (!elems_ok({B, L, D})) return LR_E_OVERFLOW;
  int64_t nwg = 1;
  if (!mul_ok(nwg, B) || !mul_ok(nwg, (D + 15) / 16) || nwg > kMaxGrid) return LR_E_OVERFLOW;
  if (B * L > 0 && any_null({a, b, h})) return LR_E_NULLPTR;
  if (!all_aligned({a, b, h, h0, h_last})) return LR_E_ALIGN;
  if (B == 0) return LR_OK;
  auto s = static_cast<hipStream_t>(stream);
  return hip_status(io == LR_F32 ? lr::launch_diag_scan<float>(a, b, h0, h, h_last, B, L, D, s)
                                 : lr::launch_diag_scan<uint16_t>(a, b, h0, h, h_last, B, L, D, s));
}

lr_status lr_diag_scan_bwd(lr_dtype io, int64_t B, int64_t L, int64_t D, const void* a,
                           const void* h, const float* h0, const void* dh, const float* dh_last,
                           void* da, void* db, float* dh0, void* stream) {
  if (!valid_io(io)) return LR_E_DTYPE;
  if (B < 0 || L < 0 || D < 1) return LR_E_SHAPE;
  if (!elems_ok({B, L, D})) return LR_E_OVERFLOW;
  int64_t nwg = 1;
  if (!mul_ok(nwg, B) || !mul_ok(nwg, (D + 15) / 16) || nwg > kMaxGrid) return LR_E_OVERFLOW;
  if (B * L > 0 && any_null({a, h, dh, da, db})) return LR_E_NULLPTR;
  if (!all_aligned({a, h, h0, dh, dh_last, da, db, dh0})) return LR_E_ALIGN;
  if (B == 0) return LR_OK;
  auto s = static_cast<hipStream_t>(stream);
  return hip_status(io == LR_F32
                        ? lr::launch_diag_scan_bwd<float>(a, h, h0, dh, dh_last, da, db, dh0, B, L, D, s)
                        : lr::launch_diag_scan_bwd<uint16_t>(a, h, h0, dh, dh_last, da, db, dh0, B, L, D, s));
}

lr_status lr_selective_scan(lr_dtype io, lr_disc disc, int64_t B, int64_t L, int64_t D, int64_t N,
                            int64_t seg, const void* x, const void* dt, const float* A,
                            const void* Bm, const void* Cm, const float* Dskip, const float* h0,
                            void* y, float* h_last, float* ckpt, void* stream) {
  if (!valid_io(io) || !valid_disc(disc)) return LR_E_DTYPE;
  if (B < 0 || L < 0 || D < 1 || N < 1 || seg < 0) return LR_E_SHAPE;
  if (N > 64 || seg % 32 != 0) return LR_E_UNSUPPORTED;
  // tile offsets (64 tokens x D) are 32-bit in the kernels
  if (D > kMaxSelD) return LR_E_UNSUPPORTED;
  if (!elems_ok({B, L, D}) || !elems_ok({B, D, N}) || !elems_ok({D, N})) return LR_E_OVERFLOW;
  if (seg > 0 && !elems_ok({(L + seg - 1) / seg, B, D, N})) return LR_E_OVERFLOW;
  int64_t nwg = 1;   // 32 channels per workgroup in the smallest layout
  if (!mul_ok(nwg, B) || !mul_ok(nwg, (D + 31) / 32) || nwg > kMaxGrid) return LR_E_OVERFLOW;
  if (A == nullptr) return LR_E_NULLPTR;
  if (B * L > 0 && any_null({x, dt, Bm, Cm, y})) return LR_E_NULLPTR;
  if (B * L > 0 && seg > 0 && ckpt == nullptr) return LR_E_NULLPTR;
  if (!all_aligned({x, dt, A, Bm, Cm, Dskip, h0, y, h_last, ckpt})) return LR_E_ALIGN;
  if (B == 0) return LR_OK;
  auto s = static_cast<hipStream_t>(stream);
  const int n = static_cast<int>(N);
  float* ck = seg > 0 ? ckpt : nullptr;
  return hip_status(io == LR_F32
                        ? lr::launch_selective_scan<float>(disc, x, dt, A, Bm, Cm, Dskip, h0, y,
                                                           h_last, ck, B, L, D, n, seg, s)
                        : lr::launch_selective_scan<uint16_t>(disc, x, dt, A, Bm, Cm, Dskip, h0,
                                                              y, h_last, ck, B, L, D, n, seg, s));
}

size_t lr_selective_scan_bwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N,
                                             int64_t seg) {
  if (B < 0 || L < 0 || D < 1 || N < 1 || !lr::selective_bwd_supported(N, seg)) return 0;
  if (!elems_ok({B, L, D}) || !elems_ok({B, D, N})) return 0;
  return lr::selective_bwd_workspace(B, L, D, N);
}

lr_status lr_selective_scan_bwd(lr_dtype io, lr_disc disc, int64_t B, int64_t L, int64_t D,
                                int64_t N, int64_t seg, const void* x, const void* dt,
                                const float* A, const void* Bm, const void* Cm,
                                const float* Dskip, const float* ckpt, const void* dy,
                                const float* dh_last, void* dx, void* ddt, float* dA, void* dBm,
                                void* dCm, float* dD, float* dh0, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!valid_io(io) || !valid_disc(disc)) return LR_E_DTYPE;
  if (B < 0 || L < 0 || D < 1 || N < 1 || seg < 1) return LR_E_SHAPE;
  if (!lr::selective_bwd_supported(N, seg)) return LR_E_UNSUPPORTED;
  if (!elems_ok({B, L, D}) || !elems_ok({B, D, N}) || !elems_ok({D, N}) ||
      !elems_ok({(D + 63) / 64, B, L, N}) || !elems_ok({(L + seg - 1) / seg, B, D, N}))
    return LR_E_OVERFLOW;
  int64_t nwg = 1;
  if (!mul_ok(nwg, B) || !mul_ok(nwg, (D + 63) / 64) || nwg > kMaxGrid) return LR_E_OVERFLOW;
  if (A == nullptr || dA == nullptr) return LR_E_NULLPTR;
  if (B * L > 0 && any_null({x, dt, Bm, Cm, ckpt, dy, dx, ddt, dBm, dCm})) return LR_E_NULLPTR;
  if (!all_aligned({x, dt, A, Bm, Cm, Dskip, ckpt, dy, dh_last, dx, ddt, dA, dBm, dCm, dD, dh0,
                    workspace}))
    return LR_E_ALIGN;
  const size_t need = lr::selective_bwd_workspace(B, L, D, N);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return LR_E_WORKSPACE;
  auto s = static_cast<hipStream_t>(stream);
  return hip_status(io == LR_F32
                        ? lr::launch_selective_bwd<float>(disc, x, dt, A, Bm, Cm, Dskip, ckpt, dy,
                                                          dh_last, dx, ddt, dA, dBm, dCm, dD, dh0,
                                                          workspace, B, L, D, N, seg, s)
                        : lr::launch_selective_bwd<uint16_t>(disc, x, dt, A, Bm, Cm, Dskip, ckpt,
                                                             dy, dh_last, dx, ddt, dA, dBm, dCm, dD,
                                                             dh0, workspace, B, L, D, N, seg, s));
}

lr_status lr_ssd_scan(lr_dtype io, lr_disc disc, int64_t B, int64_t L, int64_t H, int64_t P,
                      int64_t G, int64_t N, int64_t chunk, int64_t seg, const void* x,
                      const void* dt, const float* A, const void* Bm, const void* Cm,
                      const float* Dskip, const float* h0, void* y, float* h_last, float* ckpt,
                      void* workspace, size_t workspace_bytes, void* stream) {
  lr_status st = check_ssd_sizes(io, disc, B, L, H, P, G, N, chunk, seg);
  if (st != LR_OK) return st;
  if (workspace != nullptr && workspace_bytes < lr::ssd_fwd_workspace(B, L, H, P, N))
    return LR_E_WORKSPACE;
  if (A == nullptr) return LR_E_NULLPTR;
  if (B * L > 0 && any_null({x, dt, Bm, Cm, y})) return LR_E_NULLPTR;
  if (seg > 0 && B * L > 0 && ckpt == nullptr) return LR_E_NULLPTR;
  if (!all_aligned({x, dt, A, Bm, Cm, Dskip, h0, y, h_last, ckpt, workspace})) return LR_E_ALIGN;
  if (B == 0) return LR_OK;
  return hip_status(lr::launch_ssd_fwd(disc, x, dt, A, Bm, Cm, Dskip, h0, y, h_last, ckpt, B, L,
                                       H, P, G, N, seg, workspace, workspace_bytes,
                                       static_cast<hipStream_t>(stream)));
}

lr_status lr_ssd_scan_noalloc(lr_dtype io, lr_disc disc, int64_t B, int64_t L, int64_t H,
                              int64_t P, int64_t G, int64_t N, int64_t chunk, int64_t seg,
                              const void* x, const void* dt, const float* A, const void* Bm,
                              const void* Cm, const float* Dskip, const float* h0, void* y,
                              float* h_last, float* ckpt, void* stream) {
  lr_status st = check_ssd_sizes(io, disc, B, L, H, P, G, N, chunk, seg);
  if (st != LR_OK) return st;
  const size_t need = lr::ssd_fwd_workspace(B, L, H, P, N);
  if (need > lr::ssd_noalloc_scratch_bytes()) return LR_E_WORKSPACE;
  if (A == nullptr) return LR_E_NULLPTR;
  if (B * L > 0 && any_null({x, dt, Bm, Cm, y})) return LR_E_NULLPTR;
  if (seg > 0 && B * L > 0 && ckpt == nullptr) return LR_E_NULLPTR;
  if (!all_aligned({x, dt, A, Bm, Cm, Dskip, h0, y, h_last, ckpt})) return LR_E_ALIGN;
  if (B == 0) return LR_OK;
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = lr::ssd_noalloc_scratch(&ws);
    if (e != hipSuccess) return LR_E_HIP;
  }
  return hip_status(lr::launch_ssd_fwd(disc, x, dt, A, Bm, Cm, Dskip, h0, y, h_last, ckpt, B, L,
                                       H, P, G, N, seg, ws, ws != nullptr ? need : 0,
                                       static_cast<hipStream_t>(stream)));
}

size_t lr_ssd_scan_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                                   int64_t N, int64_t chunk) {
  if (check_ssd_sizes(LR_BF16, LR_DISC_ZOH, B, L, H, P, G, N, chunk, 0) != LR_OK) return 0;
  return lr::ssd_fwd_workspace(B, L, H, P, N);
}

size_t lr_ssd_scan_bwd_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                                       int64_t N, int64_t chunk, int64_t seg) {
  if (check_ssd_sizes(LR_BF16, LR_DISC_ZOH, B, L, H, P, G, N, chunk, seg) != LR_OK || seg < 1 ||
      !lr::ssd_bwd_supported(P, N, seg))
    return 0;
  return lr::ssd_bwd_workspace(B, L, H, P, G, N, seg);
}

lr_status lr_ssd_scan_bwd(lr_dtype io, lr_disc disc, int64_t B, int64_t L, int64_t H, int64_t P,
                          int64_t G, int64_t N, int64_t chunk, int64_t seg, const void* x,
                          const void* dt, const float* A, const void* Bm, const void* Cm,
                          const float* Dskip, const float* h0, const float* ckpt, const void* dy,
                          const float* dh_last, void* dx, void* ddt, float* dA, void* dBm,
                          void* dCm, float* dD, float* dh0, void* workspace,
                          size_t workspace_bytes, void* stream) {
  lr_status st = check_ssd_sizes(io, disc, B, L, H, P, G, N, chunk, seg);
  if (st != LR_OK) return st;
  if (seg < 1) return LR_E_SHAPE;
  if (!lr::ssd_bwd_supported(P, N, seg)) return LR_E_UNSUPPORTED;
  if (A == nullptr || dA == nullptr) return LR_E_NULLPTR;
  if (B * L > 0 && any_null({x, dt, Bm, Cm, ckpt, dy, dx, ddt, dBm, dCm})) return LR_E_NULLPTR;
  if (!all_aligned({x, dt, A, Bm, Cm, Dskip, h0, ckpt, dy, dh_last, dx, ddt, dA, dBm, dCm, dD,
                    dh0, workspace}))
    return LR_E_ALIGN;
  // below the default size the backward runs in smaller batch slices
  const size_t need = lr::ssd_bwd_workspace(B, L, H, P, G, N, seg, true);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return LR_E_WORKSPACE;
  if (B * L == 0)
    return hip_status(lr::launch_ssd_bwd_empty(dA, dD, dh0, dh_last, H, B * H * P * N,
                                               static_cast<hipStream_t>(stream)));
  return hip_status(lr::launch_ssd_bwd(disc, x, dt, A, Bm, Cm, Dskip, h0, ckpt, dy, dh_last, dx, ddt,
                                       dA, dBm, dCm, dD, dh0, workspace, workspace_bytes, B, L, H,
                                       P, G, N, seg, static_cast<hipStream_t>(stream)));
}

// Checks shared by the GLA forward and backward.
static lr_status check_gla_sizes(int io, int64_t B, int64_t L, int64_t H, int64_t K, int64_t V,
                          int64_t chunk, int64_t seg) {
  if (!valid_io(io)) return LR_E_DTYPE;
  if (B < 0 || L < 0 || H < 1 || K < 1 || V < 1 || chunk < 1 || seg < 0) return LR_E_SHAPE;
  if (io != LR_BF16 || (K != 64 && K != 128) || V % 64 != 0 || chunk % 64 != 0 || seg % 64 != 0)
    return LR_E_UNSUPPORTED;
  if (seg > 0 && seg % chunk != 0) return LR_E_SHAPE;   // segments are whole chunks
  if (!elems_ok({B, L, H, K}) || !elems_ok({B, L, H, V}) || !elems_ok({B, H, K, V}))
    return LR_E_OVERFLOW;
  if (!row_ok(H, K) || !row_ok(H, V)) return LR_E_UNSUPPORTED;
  int64_t nwg = 1;
  if (!mul_ok(nwg, B) || !mul_ok(nwg, H) || !mul_ok(nwg, V / 64) || nwg > kMaxGrid)
    return LR_E_OVERFLOW;
  if (seg > 0) {
    const int64_t nseg = (L + seg - 1) / seg;
    if (!elems_ok({nseg, B, H, K, V})) return LR_E_OVERFLOW;
    if (!mul_ok(nwg, nseg) || nwg > kMaxGrid) return LR_E_OVERFLOW;
  }
  return LR_OK;
}

lr_status lr_gla_scan(lr_dtype io, int64_t B, int64_t L, int64_t H, int64_t K, int64_t V,
                      int64_t chunk, int64_t seg, const void* q, const void* k, const void* v,
                      const void* g, const float* S0, void* o, float* S_last, float* ckpt,
                      void* workspace, size_t workspace_bytes, void* stream) {
  const lr_status st = check_gla_sizes(io, B, L, H, K, V, chunk, seg);
  if (st != LR_OK) return st;
  if (workspace != nullptr && workspace_bytes < lr::gla_fwd_workspace(B, L, H, K, V))
    return LR_E_WORKSPACE;
  if (B * L > 0 && any_null({q, k, v, g, o})) return LR_E_NULLPTR;
  if (B * L > 0 && seg > 0 && ckpt == nullptr) return LR_E_NULLPTR;
  if (!all_aligned({q, k, v, g, S0, o, S_last, ckpt, workspace})) return LR_E_ALIGN;
  if (B == 0) return LR_OK;
  return hip_status(lr::launch_gla_fwd(q, k, v, g, S0, o, S_last, seg > 0 ? ckpt : nullptr, B, L,
                                       H, K, V, seg, workspace, workspace_bytes,
                                       static_cast<hipStream_t>(stream)));
}

size_t lr_gla_scan_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t K, int64_t V,
                                   int64_t chunk) {
  if (check_gla_sizes(LR_BF16, B, L, H, K, V, chunk, 0) != LR_OK) return 0;
  return lr::gla_fwd_workspace(B, L, H, K, V);
}

size_t lr_gla_scan_bwd_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t K, int64_t V,
                                       int64_t chunk, int64_t seg) {
  if (check_gla_sizes(LR_BF16, B, L, H, K, V, chunk, seg) != LR_OK || !lr::ssd_bwd_supported(64, K, seg))
    return 0;
  return lr::gla_bwd_workspace(B, L, H, K, V, seg);
}

lr_status lr_gla_scan_bwd(lr_dtype io, int64_t B, int64_t L, int64_t H, int64_t K, int64_t V,
                          int64_t chunk, int64_t seg, const void* q, const void* k, const void* v,
                          const void* g, const float* ckpt, const void* dout,
                          const float* dS_last, void* dq, void* dk, void* dv, void* dg,
                          float* dS0, void* workspace, size_t workspace_bytes, void* stream) {
  const lr_status st = check_gla_sizes(io, B, L, H, K, V, chunk, seg);
  if (st != LR_OK) return st;
  if (seg < 1) return LR_E_SHAPE;
  if (!lr::ssd_bwd_supported(64, K, seg)) return LR_E_UNSUPPORTED;
  if (B * L > 0 && any_null({q, k, v, g, ckpt, dout, dq, dk, dv, dg})) return LR_E_NULLPTR;
  if (!all_aligned({q, k, v, g, ckpt, dout, dS_last, dq, dk, dv, dg, dS0, workspace}))
    return LR_E_ALIGN;
  const size_t need = lr::gla_bwd_workspace(B, L, H, K, V, seg, true);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return LR_E_WORKSPACE;
  if (B * L == 0) {
    if (dS0 == nullptr || B == 0) return LR_OK;
    return hip_status(lr::launch_ssd_bwd_empty(nullptr, nullptr, dS0, dS_last, 0, B * H * K * V,
                                               static_cast<hipStream_t>(stream)));
  }
  return hip_status(lr::launch_gla_bwd(q, k, v, g, ckpt, dout, dS_last, dq, dk, dv, dg, dS0,
                                       workspace, workspace_bytes, B, L, H, K, V, seg,
                                       static_cast<hipStream_t>(stream)));
}

lr_status lr_rotlru_scan(lr_dtype io, int64_t B, int64_t L, int64_t D, const void* r,
                         const void* theta, const void* u, const float* h0, void* h,
                         float* h_last, void* stream) {
  if (!valid_io(io)) return LR_E_DTYPE;
  if (B < 0 || L < 0 || D < 2 || D % 2 != 0) return LR_E_SHAPE;
  if (!elems_ok({B, L, D})) return LR_E_OVERFLOW;
  int64_t nwg = 1;
  if (!mul_ok(nwg, B) || !mul_ok(nwg, (D / 2 + 15) / 16) || nwg > kMaxGrid) return LR_E_OVERFLOW;
  if (B * L > 0 && any_null({r, theta, u, h})) return LR_E_NULLPTR;
  if (!all_aligned({r, theta, u, h0, h, h_last})) return LR_E_ALIGN;
  if (B == 0) return LR_OK;
  auto s = static_cast<hipStream_t>(stream);
  return hip_status(io == LR_F32 ? lr::launch_rotlru_scan<float>(r, theta, u, h0, h, h_last, B, L, D, s)
                                 : lr::launch_rotlru_scan<uint16_t>(r, theta, u, h0, h, h_last, B, L, D, s));
}

lr_status lr_rotlru_scan_bwd(lr_dtype io, int64_t B, int64_t L, int64_t D, const void* r,
                             const void* theta, const void* h, const float* h0, const void* dh,
                             const float* dh_last, void* dr, void* dtheta, void* du, float* dh0,
                             void* stream) {
  if (!valid_io(io)) return LR_E_DTYPE;
  if (B < 0 || L < 0 || D < 2 || D % 2 != 0) return LR_E_SHAPE;
  if (!elems_ok({B, L, D})) return LR_E_OVERFLOW;
  int64_t nwg = 1;
  if (!mul_ok(nwg, B) || !mul_ok(nwg, (D / 2 + 15) / 16) || nwg > kMaxGrid) return LR_E_OVERFLOW;
  if (B * L > 0 && any_null({r, theta, h, dh, dr, dtheta, du})) return LR_E_NULLPTR;
  if (!all_aligned({r, theta, h, h0, dh, dh_last, dr, dtheta, du, dh0})) return LR_E_ALIGN;
  if (B == 0) return LR_OK;
  auto s = static_cast<hipStream_t>(stream);
  return hip_status(io == LR_F32
                        ? lr::launch_rotlru_scan_bwd<float>(r, theta, h, h0, dh, dh_last, dr, dtheta,
                                                            du, dh0, B, L, D, s)
                        : lr::launch_rotlru_scan_bwd<uint16_t>(r, theta, h, h0, dh, dh_last, dr,
                                                               dtheta, du, dh0, B, L, D, s));
}

// ---------------------------------------------------------------- steps
lr_status lr_diag_step(lr_dtype io, int64_t B, int64_t D, const void* a, const void* b, float* h,
                       void* out, void* stream) {
  if (!valid_io(io)) return LR_E_DTYPE;
  if (B < 0 || D < 1) return LR_E_SHAPE;
  if (!elems_ok({B, D}) || (B * D + 255) / 256 > kMaxGrid) return LR_E_OVERFLOW;
  if (B > 0 && any_null({a, b, h})) return LR_E_NULLPTR;
  if (!all_aligned({a, b, h, out})) return LR_E_ALIGN;
  if (B == 0) return LR_OK;
  auto s = static_cast<hipStream_t>(stream);
  return hip_status(io == LR_F32 ? lr::launch_diag_step<float>(a, b, h, out, B * D, s)
                                 : lr::launch_diag_step<uint16_t>(a, b, h, out, B * D, s));
}

lr_status lr_selective_step(lr_dtype io, lr_disc disc, int64_t B, int64_t D, int64_t N,
                            const void* x, const void* dt, const float* A, const void* Bm,
                            const void* Cm, const float* Dskip, float* h, void* y, void* stream) {
  if (!valid_io(io) || !valid_disc(disc)) return LR_E_DTYPE;
  if (B < 0 || D < 1 || N < 1) return LR_E_SHAPE;
  if (N > 64) return LR_E_UNSUPPORTED;
  if (!elems_ok({B, D, 64}) || (B * D * 64 + 255) / 256 > kMaxGrid) return LR_E_OVERFLOW;
  if (A == nullptr) return LR_E_NULLPTR;
  if (B > 0 && any_null({x, dt, Bm, Cm, h, y})) return LR_E_NULLPTR;
  if (!all_aligned({x, dt, A, Bm, Cm, Dskip, h, y})) return LR_E_ALIGN;
  if (B == 0) return LR_OK;
  auto s = static_cast<hipStream_t>(stream);
  const int n = static_cast<int>(N);
  return hip_status(io == LR_F32
                        ? lr::launch_selective_step<float>(disc, x, dt, A, Bm, Cm, Dskip, h, y, B, D, n, s)
                        : lr::launch_selective_step<uint16_t>(disc, x, dt, A, Bm, Cm, Dskip, h, y, B, D, n, s));
}

lr_status lr_ssd_step(lr_dtype io, lr_disc disc, int64_t B, int64_t H, int64_t P, int64_t G,
                      int64_t N, const void* x, const void* dt, const float* A, const void* Bm,
                      const void* Cm, const float* Dskip, float* h, void* y, void* stream) {
  if (!valid_io(io) || !valid_disc(disc)) return LR_E_DTYPE;
  if (B < 0 || H < 1 || P < 1 || G < 1 || N < 1 || H % G != 0) return LR_E_SHAPE;
  if (io != LR_BF16 || (N != 64 && N != 128)) return LR_E_UNSUPPORTED;
  if (!elems_ok({B, H, P, N}) || (B * H * P * 4 + 255) / 256 > kMaxGrid) return LR_E_OVERFLOW;
  if (A == nullptr) return LR_E_NULLPTR;
  if (B > 0 && any_null({x, dt, Bm, Cm, h, y})) return LR_E_NULLPTR;
  if (!all_aligned({x, dt, A, Bm, Cm, Dskip, h, y})) return LR_E_ALIGN;
  if (B == 0) return LR_OK;
  return hip_status(lr::launch_ssd_step(disc, x, dt, A, Bm, Cm, Dskip, h, y, B, H, P, G, N,
                                        static_cast<hipStream_t>(stream)));
}

lr_status lr_gla_step(lr_dtype io, int64_t B, int64_t H, int64_t K, int64_t V, const void* q,
                      const void* k, const void* v, const void* g, float* S, void* o,
                      void* stream) {
  if (!valid_io(io)) return LR_E_DTYPE;
  if (B < 0 || H < 1 || K < 1 || V < 1) return LR_E_SHAPE;
  if (io != LR_BF16 || V % 64 != 0) return LR_E_UNSUPPORTED;
  if (!elems_ok({B, H, K, V})) return LR_E_OVERFLOW;
  int64_t nwg = 1;
  if (!mul_ok(nwg, B) || !mul_ok(nwg, H) || !mul_ok(nwg, V / 64) || nwg > kMaxGrid)
    return LR_E_OVERFLOW;
  if (B > 0 && any_null({q, k, v, g, S, o})) return LR_E_NULLPTR;
  if (!all_aligned({q, k, v, g, S, o})) return LR_E_ALIGN;
  if (B == 0) return LR_OK;
  return hip_status(lr::launch_gla_step(q, k, v, g, S, o, B, H, K, V,
                                        static_cast<hipStream_t>(stream)));
}

}  // extern "C"
