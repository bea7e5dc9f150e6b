// launch.hpp — host entry points of the kernel files, called by the C ABI
// (abi.hip): one declaration per launcher or size query, defined in the
// .hip file of its kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace lr {
template <typename T>
hipError_t launch_diag_scan(const void* a, const void* b, const float* h0, void* h,
                            float* h_last, int64_t B, int64_t L, int64_t D, hipStream_t stream);
template <typename T>
hipError_t launch_diag_scan_bwd(const void* a, const void* h, const float* h0, const void* dh,
                                const float* dh_last, void* da, void* db, float* dh0, int64_t B,
                                int64_t L, int64_t D, hipStream_t stream);
template <typename T>
hipError_t launch_selective_scan(int disc, const void* x, const void* dt, const float* A,
                                 const void* Bm, const void* Cm, const float* Dskip,
                                 const float* h0, void* y, float* h_last, float* ckpt, int64_t B,
                                 int64_t L, int64_t D, int N, int64_t seg, hipStream_t stream);
bool selective_bwd_supported(int64_t N, int64_t seg);
size_t selective_bwd_workspace(int64_t B, int64_t L, int64_t D, int64_t N);
template <typename T>
hipError_t launch_selective_bwd(int disc, const void* x, const void* dt, const float* A,
                                const void* Bm, const void* Cm, const float* Dskip,
                                const float* ckpt, const void* dy, const float* dh_last, void* dx,
                                void* ddt, float* dA, void* dBm, void* dCm, float* dD, float* dh0,
                                void* ws, int64_t B, int64_t L, int64_t D, int64_t N, int64_t seg,
                                hipStream_t stream);
hipError_t launch_ssd_fwd(int disc, const void* x, const void* dt, const float* A, const void* Bm,
                          const void* Cm, const float* Dskip, const float* h0, void* y,
                          float* h_last, float* ckpt, int64_t B, int64_t L, int64_t H, int64_t P,
                          int64_t G, int64_t N, int64_t seg, void* ws, size_t ws_bytes,
                          hipStream_t stream);
hipError_t launch_gla_fwd(const void* q, const void* k, const void* v, const void* gate,
                          const float* S0, void* o, float* S_last, float* ckpt, int64_t B,
                          int64_t L, int64_t H, int64_t K, int64_t V, int64_t seg, void* ws,
                          size_t ws_bytes, hipStream_t stream);
size_t ssd_fwd_workspace(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N);
size_t ssd_noalloc_scratch_bytes();
hipError_t ssd_noalloc_scratch(void** out);
size_t gla_fwd_workspace(int64_t B, int64_t L, int64_t H, int64_t K, int64_t V);
// Backward workspaces: the default size, or (smallest) the one for slices of
// one batch row, below which the backward cannot run.
size_t gla_bwd_workspace(int64_t B, int64_t L, int64_t H, int64_t K, int64_t V, int64_t seg,
                         bool smallest = false);
hipError_t launch_gla_bwd(const void* q, const void* k, const void* v, const void* g,
                          const float* ckpt, const void* dout, const float* dS_last, void* dq,
                          void* dk, void* dv, void* dg, float* dS0, void* ws, size_t ws_bytes,
                          int64_t B, int64_t L, int64_t H, int64_t K, int64_t V, int64_t seg,
                          hipStream_t stream);
size_t ssd_bwd_workspace(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                         int64_t seg, bool smallest = false);
bool ssd_bwd_supported(int64_t P, int64_t N, int64_t seg);
hipError_t launch_ssd_bwd_empty(float* dA, float* dD, float* dh0, const float* dh_last, int64_t H,
                                int64_t nstate, hipStream_t stream);
hipError_t launch_ssd_bwd(int disc, const void* x, const void* dt, const float* A, const void* Bm,
                          const void* Cm, const float* Dskip, const float* h0, const float* ckpt,
                          const void* dy,
                          const float* dh_last, void* dx, void* ddt, float* dA, void* dBm,
                          void* dCm, float* dD, float* dh0, void* ws, size_t ws_bytes,
                          int64_t B, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                          int64_t seg, hipStream_t stream);
template <typename T>
hipError_t launch_rotlru_scan(const void* r, const void* theta, const void* u, const float* h0,
                              void* h, float* h_last, int64_t B, int64_t L, int64_t D,
                              hipStream_t stream);
template <typename T>
hipError_t launch_rotlru_scan_bwd(const void* r, const void* theta, const void* h, const float* h0,
                                  const void* dh, const float* dh_last, void* dr, void* dtheta,
                                  void* du, float* dh0, int64_t B, int64_t L, int64_t D,
                                  hipStream_t stream);
template <typename T>
hipError_t launch_diag_step(const void* a, const void* b, float* h, void* out, int64_t n,
                            hipStream_t s);
template <typename T>
hipError_t launch_selective_step(int disc, const void* x, const void* dt, const float* A,
                                 const void* Bm, const void* Cm, const float* Dskip, float* h,
                                 void* y, int64_t B, int64_t D, int N, hipStream_t s);
hipError_t launch_ssd_step(int disc, const void* x, const void* dt, const float* A, const void* Bm,
                           const void* Cm, const float* Dskip, float* h, void* y, int64_t B,
                           int64_t H, int64_t P, int64_t G, int64_t N, hipStream_t s);
hipError_t launch_gla_step(const void* q, const void* k, const void* v, const void* g, float* S,
                           void* o, int64_t B, int64_t H, int64_t K, int64_t V, hipStream_t s);
}  // namespace lr
