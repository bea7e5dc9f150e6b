/*
 * lr.h — C ABI of liblr, fused linear-recurrence scans for AMD MI355X (gfx950).
 *
 * Every scan evaluates the first-order linear recurrence
 *     h_t = a_t (.) h_{t-1} + b_t
 * whose steps compose under the associative (not commutative) combine
 *     (a2, b2) o (a1, b1) = (a2 a1, a2 b1 + b2)
 * (IBM Research blog "K-Search for MLX", section "A 20x faster prefill: the
 * Mamba SSM kernel", recurrence and combine equations).  Each forward scan is
 * one kernel launch over the whole sequence ("mlx-recurrence" post, Apple
 * Developer Forums thread 840535, opening paragraphs).
 *
 * Conventions for every entry point
 *   - All calls are asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL means the default stream).  The library never synchronises.
 *   - Tensor pointers are DEVICE pointers, dense, contiguous and row-major in
 *     exactly the shapes given in the comments (token-major [B, L, ...]).
 *     They must be 16-byte aligned.  No strides.
 *   - `io` is the element type of every per-token tensor and per-token
 *     gradient.  A, Dskip, states (h0, h_last, ckpt, S0, S_last) and the
 *     parameter gradients (dA, dD, dh0) are always float32.
 *   - Ownership: the caller owns every buffer.  The library allocates no
 *     memory and keeps no per-call state; scratch memory is a caller-provided
 *     workspace whose size comes from a query function.  The one exception,
 *     lr_ssd_scan_noalloc, uses a static device array of the library instead.
 *   - Sizes: B and L may be 0 (empty input: nothing is computed; outputs that
 *     carry a state receive the initial state).  Feature sizes must be > 0.
 *   - Errors: each call validates all arguments BEFORE touching the device.
 *     On failure it returns a non-zero lr_status and writes nothing.  Launch
 *     failures map to LR_E_HIP.  Faults inside a kernel surface at the
 *     caller's next synchronisation.  No C++ exception crosses the ABI.  The
 *     library is thread-safe: its only global state is the per-device address
 *     of lr_ssd_scan_noalloc's static array, set once per device.
 *   - Determinism: results are bitwise identical across runs for a fixed
 *     build, shape and input (no floating-point atomics anywhere).
 */
#ifndef LR_H_
#define LR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of per-token tensors.  The LR_*_RANGE_* enumerators are not
 * valid arguments: they make every int32 value a value of the type, so an
 * out-of-range code from the caller is rejected (LR_E_DTYPE) with defined
 * behaviour in the C++ implementation. */
typedef enum {
  LR_F32 = 0, LR_BF16 = 1,
  LR_DTYPE_RANGE_MIN = INT32_MIN, LR_DTYPE_RANGE_MAX = INT32_MAX
} lr_dtype;

/* Discretisation of a continuous-time decay A over a step dt ("lrnnx: A
 * library for Linear RNNs", Key Contributions 2-3, which name ZOH, bilinear
 * and dirac among the schemes of its fused kernels; the pages give no
 * formulas).  Readings used here, with l = dt*A:
 *   LR_DISC_ZOH:      abar = exp(l),                bbar = expm1(l)/A * B  (= dt*B at A=0)
 *   LR_DISC_EULER:    abar = exp(l),                bbar = dt * B
 *   LR_DISC_BILINEAR: abar = (1 + l/2) / (1 - l/2), bbar = dt / (1 - l/2) * B  (Tustin)
 *   LR_DISC_DIRAC:    abar = exp(l),                bbar = B  (the input is an
 *                     impulse of area x at the sample: no dt factor)           */
typedef enum {
  LR_DISC_ZOH = 0, LR_DISC_EULER = 1, LR_DISC_BILINEAR = 2, LR_DISC_DIRAC = 3,
  LR_DISC_RANGE_MIN = INT32_MIN, LR_DISC_RANGE_MAX = INT32_MAX   /* not valid arguments */
} lr_disc;

typedef enum {
  LR_OK = 0,
  LR_E_NULLPTR = 1,     /* a required pointer is NULL                        */
  LR_E_SHAPE = 2,       /* a size is negative/zero where it must be > 0, or
                           sizes are inconsistent (e.g. H % G != 0)          */
  LR_E_DTYPE = 3,       /* unknown lr_dtype or lr_disc value                  */
  LR_E_ALIGN = 4,       /* a pointer is not 16-byte aligned                   */
  LR_E_UNSUPPORTED = 5, /* a size or dtype outside the compiled set           */
  LR_E_WORKSPACE = 6,   /* workspace missing or smaller than required         */
  LR_E_OVERFLOW = 7,    /* a size product overflows int64 / exceeds limits    */
  LR_E_HIP = 8          /* the HIP runtime reported an error at launch        */
} lr_status;

/* Static, NUL-terminated description of a status code. */
const char* lr_status_string(int status);
/* Library version string, e.g. "liblr 0.1.0 gfx950". */
const char* lr_version(void);

/* ---------------------------------------------------------------------------
 * Diagonal recurrence (RG-LRU-style; "mlx-recurrence" post, rglru_scan,
 * state [B, D]).  The decay a and input b are given directly.
 *     h[b,t,d] = a[b,t,d] * h[b,t-1,d] + b[b,t,d],   h[b,-1,:] = h0 (or 0)
 *   io:     LR_F32 or LR_BF16 (a, b, h); state arithmetic is fp32.
 *   a, b:   [B, L, D] io          h: [B, L, D] io (every step is written)
 *   h0:     [B, D] fp32 or NULL   h_last: [B, D] fp32 or NULL
 * Supported: any B >= 0, L >= 0, D >= 1.
 * ------------------------------------------------------------------------- */
lr_status lr_diag_scan(lr_dtype io, int64_t B, int64_t L, int64_t D,
                       const void* a, const void* b, const float* h0,
                       void* h, float* h_last, void* stream);

/* ---------------------------------------------------------------------------
 * Backward of lr_diag_scan for the loss
 *     sum_t <dh[b,t,:], h[b,t,:]> + <dh_last[b,:], h[b,L-1,:]>
 * (reverse-time adjoint of the recurrence above: g_{L-1} = dh_{L-1} + dh_last,
 * g_t = a_{t+1} g_{t+1} + dh_t; then db_t = g_t, da_t = g_t h_{t-1} with
 * h_{-1} = h0, and dh0 = a_0 g_0).  The forward already writes every state,
 * so nothing is recomputed: h is the forward's output.
 *   a, h, dh: [B, L, D] io    h0, dh_last: [B, D] fp32 or NULL (= 0)
 *   da, db:   [B, L, D] io    dh0: [B, D] fp32 or NULL; dh0 = dh_last at L = 0
 * Supported: as lr_diag_scan.
 * ------------------------------------------------------------------------- */
lr_status lr_diag_scan_bwd(lr_dtype io, int64_t B, int64_t L, int64_t D,
                           const void* a, const void* h, const float* h0,
                           const void* dh, const float* dh_last, void* da,
                           void* db, float* dh0, void* stream);

/* ---------------------------------------------------------------------------
 * Rotational LRU ("mlx-recurrence" post, rotlru_scan: complex-diagonal
 * recurrence, magnitude gate, per-step rotation of two-dimensional channel
 * pairs, state [B, D] as interleaved pairs).  With z = h[2i] + i h[2i+1]:
 *     z_t = r_t (cos theta_t + i sin theta_t) z_{t-1} + (u_t[2i] + i u_t[2i+1])
 * (reading: the gate scales, theta rotates, the input pair is added).
 *   r, theta: [B, L, D/2] io (gate, angle in radians)    u, h: [B, L, D] io
 *   h0, h_last: [B, D] fp32 or NULL.  State arithmetic is fp32.
 * Supported: any B, L >= 0; D >= 2 and even.
 * ------------------------------------------------------------------------- */
lr_status lr_rotlru_scan(lr_dtype io, int64_t B, int64_t L, int64_t D,
                         const void* r, const void* theta, const void* u,
                         const float* h0, void* h, float* h_last, void* stream);

/* ---------------------------------------------------------------------------
 * Backward of lr_rotlru_scan (the post's rotlru_scan kernel has a forward and
 * a backward) for the loss
 *     sum_t <dh[b,t,:], h[b,t,:]> + <dh_last[b,:], h_last[b,:]>.
 * In complex form per pair (G_t = gradient w.r.t. z_t, real + i imaginary):
 * G_{L-1} = dh_{L-1} + dh_last, G_t = conj(a_{t+1}) G_{t+1} + dh_t; then
 * du_t = G_t, and with q = G_t conj(e^{i theta_t} z_{t-1}) (z_{-1} = h0):
 * dr_t = Re q, dtheta_t = r_t Im q; dh0 = conj(a_0) G_0.  h is the forward's
 * output; nothing is recomputed.
 *   r, theta: [B, L, D/2] io     h, dh: [B, L, D] io
 *   h0, dh_last: [B, D] fp32 or NULL (= 0)
 *   dr, dtheta: [B, L, D/2] io   du: [B, L, D] io
 *   dh0: [B, D] fp32 or NULL; dh0 = dh_last at L = 0
 * Supported: as lr_rotlru_scan.
 * ------------------------------------------------------------------------- */
lr_status lr_rotlru_scan_bwd(lr_dtype io, int64_t B, int64_t L, int64_t D,
                             const void* r, const void* theta, const void* h,
                             const float* h0, const void* dh, const float* dh_last,
                             void* dr, void* dtheta, void* du, float* dh0,
                             void* stream);

/* ---------------------------------------------------------------------------
 * Mamba-1 selective scan with ZOH (or Euler) discretisation and a fused
 * readout ("lrnnx: A library for Linear RNNs", Key Contributions 3: fused
 * scan + output projection; the hidden state never reaches memory).
 *     e = exp(dt[b,t,d] A[d,n]),  phi = expm1(dt A)/A (ZOH) or dt (Euler)
 *     h[b,d,n] <- e h[b,d,n] + phi Bm[b,t,n] x[b,t,d]
 *     y[b,t,d]  = sum_n Cm[b,t,n] h[b,d,n] + Dskip[d] x[b,t,d]
 *   x, dt:  [B, L, D] io     Bm, Cm: [B, L, N] io     y: [B, L, D] io
 *   A:      [D, N] fp32      Dskip:  [D] fp32 or NULL (treated as 0)
 *   h0:     [B, D, N] fp32 or NULL    h_last: [B, D, N] fp32 or NULL
 * dt is the step itself (> 0 expected; no bias or softplus is applied).
 *   seg:    0, or a multiple of 32: then ckpt[s] receives the state entering
 *           token s*seg (ckpt[0] = h0 or 0); ckpt: [ceil(L/seg), B, D, N]
 *           fp32, required iff seg > 0 (consumed by lr_selective_scan_bwd).
 * Supported: 1 <= N <= 64, 1 <= D <= 2^24 (LR_E_UNSUPPORTED beyond).
 * ------------------------------------------------------------------------- */
lr_status lr_selective_scan(lr_dtype io, lr_disc disc, int64_t B, int64_t L,
                            int64_t D, int64_t N, int64_t seg, const void* x,
                            const void* dt, const float* A, const void* Bm,
                            const void* Cm, const float* Dskip,
                            const float* h0, void* y, float* h_last,
                            float* ckpt, void* stream);

/* Workspace bytes needed by lr_selective_scan_bwd (0 on invalid or
 * unsupported sizes): fp32 partial sums of dB and dC per 64-channel tile, of
 * dA and dD per batch row, and the recomputed state every 16 tokens of the
 * segment being processed. */
size_t lr_selective_scan_bwd_workspace_bytes(int64_t B, int64_t L, int64_t D,
                                             int64_t N, int64_t seg);

/* ---------------------------------------------------------------------------
 * Backward of lr_selective_scan with segment checkpoint-and-recompute
 * ("mlx-recurrence" post: segment checkpoints in the forward, recompute in
 * the backward).  Gradients of  loss = sum(dy * y) + <dh_last, h_last>  with
 * respect to x, dt, A, Bm, Cm, Dskip and h0.
 *   ckpt:   the checkpoints written by lr_selective_scan with the same seg.
 *   dy:     [B, L, D] io        dh_last: [B, D, N] fp32 or NULL (= 0)
 *   dx, ddt: [B, L, D] io       dBm, dCm: [B, L, N] io
 *   dA: [D, N] fp32    dD: [D] fp32 or NULL    dh0: [B, D, N] fp32 or NULL
 *   workspace: device memory of at least lr_selective_scan_bwd_workspace_bytes().
 * Supported: 1 <= N <= 64; seg a multiple of 32 with 32 <= seg <= 256.
 * ------------------------------------------------------------------------- */
lr_status lr_selective_scan_bwd(lr_dtype io, lr_disc disc, int64_t B,
                                int64_t L, int64_t D, int64_t N, int64_t seg,
                                const void* x, const void* dt, const float* A,
                                const void* Bm, const void* Cm,
                                const float* Dskip, const float* ckpt,
                                const void* dy, const float* dh_last, void* dx,
                                void* ddt, float* dA, void* dBm, void* dCm,
                                float* dD, float* dh0, void* workspace,
                                size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Mamba-2 head-wise SSD scan ("mlx-recurrence" post, ssd_scan, state
 * [B, H, Dh, N]; Dh is called P here).  G groups share B/C: head h reads
 * group h / (H/G).  A and Dskip are per head, dt per (b, t, h).
 *     e = exp(dt[b,t,h] A[h]),  phi as in lr_selective_scan
 *     h[b,h,p,n] <- e h + phi x[b,t,h,p] Bm[b,t,g,n]
 *     y[b,t,h,p]  = sum_n Cm[b,t,g,n] h[b,h,p,n] + Dskip[h] x[b,t,h,p]
 *   x, y: [B, L, H, P] io    dt: [B, L, H] io    Bm, Cm: [B, L, G, N] io
 *   A: [H] fp32    Dskip: [H] fp32 or NULL    h0, h_last: [B, H, P, N] fp32
 *   chunk: the caller's chunk length; any multiple of 64.  The kernel always
 *          evaluates the intra-chunk quadratic form on 64-token blocks and
 *          carries the exact state between blocks, so the result does not
 *          depend on chunk beyond rounding.
 *   seg:   0, or a multiple of 64: then ckpt[s] receives the state ENTERING
 *          token s*seg (ckpt[0] = h0 or 0) for s = 0 .. ceil(L/seg)-1 —
 *          the segment checkpoints consumed by lr_ssd_scan_bwd.
 *   ckpt:  [ceil(L/seg), B, H, P, N] fp32; required iff seg > 0.  seg must
 *          be a multiple of chunk (segments are whole chunks): LR_E_SHAPE.
 *   workspace: optional, see lr_ssd_scan_workspace_bytes (NULL: one pass).
 * Supported: io = LR_BF16 only (the contractions run on bf16 MFMA; fp32 I/O
 * returns LR_E_UNSUPPORTED); P % 64 == 0; N in {64, 128}; H % G == 0;
 * G*N and H*P at most 2^25 (the kernels address 64 token rows with 32-bit
 * byte offsets; LR_E_UNSUPPORTED beyond).
 * Deliberate additions to the plain scan signature: seg/ckpt (the segment
 * checkpoints of the training path) and the optional workspace.
 * ------------------------------------------------------------------------- */
lr_status lr_ssd_scan(lr_dtype io, lr_disc disc, int64_t B, int64_t L,
                      int64_t H, int64_t P, int64_t G, int64_t N,
                      int64_t chunk, int64_t seg, const void* x,
                      const void* dt, const float* A, const void* Bm,
                      const void* Cm, const float* Dskip, const float* h0,
                      void* y, float* h_last, float* ckpt, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Optional workspace of lr_ssd_scan (0 when the sizes are invalid or when
 * the call does not split the sequence).  With too few (batch, head) pairs
 * to fill the GPU (fewer than 256 workgroups of one (batch, head, 64
 * columns of P) each, one per CU of an MI355X), the forward cuts the
 * sequence into parts run side by side: a first launch computes each part's end state from zero and its
 * decay product into the workspace (the (a, b) combine of the "K-Search
 * for MLX" blog, section "A 20x faster prefill", applied to whole parts),
 * and the main launch folds them into the state entering every part.
 *   workspace == NULL: single pass, same results up to rounding.
 *   workspace != NULL with fewer bytes than this: LR_E_WORKSPACE.
 * The caller owns the workspace; its contents are scratch. */
size_t lr_ssd_scan_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t P,
                                   int64_t G, int64_t N, int64_t chunk);

/* ---------------------------------------------------------------------------
 * lr_ssd_scan for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and kernels as lr_ssd_scan with an "auto" workspace, but
 * the sequence split's scratch (the parts' end states and decay products)
 * lives in a static 16 MiB device array of the library, one per GPU, held
 * until the process ends.  No workspace argument; the call allocates
 * nothing and issues no memset.  Arguments, layouts and errors as
 * lr_ssd_scan; LR_E_WORKSPACE if a split would need more than the static
 * array (for N <= 128 the split needs at most ~16.7 MB, so every accepted
 * size fits).  Nothing in the array has to start at zero: each call writes
 * the scratch it reads.  Every call on one GPU shares that GPU's array, so
 * calls that overlap in time on one GPU (other streams, other threads) race
 * on it: order them on one stream.
 * ------------------------------------------------------------------------- */
lr_status lr_ssd_scan_noalloc(lr_dtype io, lr_disc disc, int64_t B, int64_t L,
                              int64_t H, int64_t P, int64_t G, int64_t N,
                              int64_t chunk, int64_t seg, const void* x,
                              const void* dt, const float* A, const void* Bm,
                              const void* Cm, const float* Dskip,
                              const float* h0, void* y, float* h_last,
                              float* ckpt, void* stream);

/* Workspace bytes needed by lr_ssd_scan_bwd for these sizes (0 on invalid
 * sizes).  The workspace holds per-head partial sums of dB and dC (bf16)
 * and the adjoint state at segment boundaries (fp32) for one slice of batch
 * rows (the backward runs slice by slice; a slice holds the smallest number
 * of rows that gives 1024 (head, segment) work items, or the whole batch),
 * plus per-segment partials of dA, dD (fp32) for the whole batch. */
size_t lr_ssd_scan_bwd_workspace_bytes(int64_t B, int64_t L, int64_t H,
                                       int64_t P, int64_t G, int64_t N,
                                       int64_t chunk, int64_t seg);

/* ---------------------------------------------------------------------------
 * Backward of lr_ssd_scan with segment checkpoint-and-recompute
 * ("mlx-recurrence" post: the training path stores segment checkpoints in
 * the forward and recomputes inside each segment in the backward).
 * Gradients of  loss = sum(dy * y) + <dh_last, h_last>  with respect to
 * x, dt, A, Bm, Cm, Dskip and h0.
 *   ckpt:    the checkpoints written by lr_ssd_scan with the same seg.
 *   h0:      [B, H, P, N] fp32 or NULL: the forward's initial state; when
 *            given, segment 0 starts from it instead of ckpt[0] (the two are
 *            equal for checkpoints written by lr_ssd_scan with this h0).
 *   dy:      [B, L, H, P] io      dh_last: [B, H, P, N] fp32 or NULL (= 0)
 *   dx:      [B, L, H, P] io      ddt: [B, L, H] io
 *   dBm, dCm: [B, L, G, N] io (summed over the heads of each group)
 *   dA: [H] fp32    dD: [H] fp32 or NULL    dh0: [B, H, P, N] fp32 or NULL
 *   workspace: device memory of lr_ssd_scan_bwd_workspace_bytes() bytes;
 *            a smaller one makes the backward run in smaller batch slices
 *            (same results), down to one row per slice, for which
 *            lr_ssd_scan_bwd_workspace_bytes(1, L, ...)
 *            + 8 (B - 1) H ceil(L / seg) + 512 bytes suffice; below the
 *            one-row size: LR_E_WORKSPACE.
 * Supported: as lr_ssd_scan, with P == 64 and seg in {64, 128, 192, 256};
 * every disc, bilinear with negative decays included (their signs are
 * tracked as in the forward).
 * ------------------------------------------------------------------------- */
lr_status lr_ssd_scan_bwd(lr_dtype io, lr_disc disc, int64_t B, int64_t L,
                          int64_t H, int64_t P, int64_t G, int64_t N,
                          int64_t chunk, int64_t seg, const void* x,
                          const void* dt, const float* A, const void* Bm,
                          const void* Cm, const float* Dskip, const float* h0,
                          const float* ckpt, const void* dy,
                          const float* dh_last, void* dx, void* ddt,
                          float* dA, void* dBm, void* dCm, float* dD,
                          float* dh0, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ---------------------------------------------------------------------------
 * Gated linear attention with a scalar forget gate and an outer-product
 * write ("mlx-recurrence" post, gla_scan, state [B, H, Dh, Dh], read here as
 * [B, H, K, V]).
 *     S[b,h] <- g[b,t,h] S[b,h] + k[b,t,h] v[b,t,h]^T
 *     o[b,t,h] = S[b,h]^T q[b,t,h]
 *   q, k: [B, L, H, K] io    v, o: [B, L, H, V] io    g: [B, L, H] io, in (0, 1]
 *   S0, S_last: [B, H, K, V] fp32 or NULL
 *   chunk: any multiple of 64 (same meaning as in lr_ssd_scan).
 *   seg:   0, or a multiple of 64 and of chunk: then ckpt[s] receives the
 *          state entering token s*seg, TRANSPOSED: ckpt is
 *          [ceil(L/seg), B, H, V, K] fp32 (required iff seg > 0; consumed by
 *          lr_gla_scan_bwd).  The transposed layout is the kernel's own
 *          register order of the state (value columns outermost), which the
 *          backward reads back directly; S0 and S_last keep [B, H, K, V].
 *   workspace: optional, as in lr_ssd_scan (see lr_gla_scan_workspace_bytes).
 * No extra scaling of q is applied.
 * Supported: io = LR_BF16 only (bf16 MFMA; fp32 I/O returns
 * LR_E_UNSUPPORTED); K in {64, 128}; V % 64 == 0; H*K and H*V at most 2^25
 * (32-bit row offsets, as in lr_ssd_scan).
 * ------------------------------------------------------------------------- */
lr_status lr_gla_scan(lr_dtype io, int64_t B, int64_t L, int64_t H, int64_t K,
                      int64_t V, int64_t chunk, int64_t seg, const void* q,
                      const void* k, const void* v, const void* g,
                      const float* S0, void* o, float* S_last, float* ckpt,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Optional workspace of lr_gla_scan: as lr_ssd_scan_workspace_bytes. */
size_t lr_gla_scan_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t K,
                                   int64_t V, int64_t chunk);

/* Workspace bytes needed by lr_gla_scan_bwd (0 on invalid sizes): partial
 * sums of dk, dq (bf16) and of the log-gate gradient (fp32) per 64 columns
 * of v, and the adjoint state at segment boundaries (fp32), for one slice of
 * batch rows as in lr_ssd_scan_bwd_workspace_bytes. */
size_t lr_gla_scan_bwd_workspace_bytes(int64_t B, int64_t L, int64_t H,
                                       int64_t K, int64_t V, int64_t chunk,
                                       int64_t seg);

/* ---------------------------------------------------------------------------
 * Backward of lr_gla_scan with segment checkpoint-and-recompute (same
 * training path as lr_ssd_scan_bwd).  Gradients of
 *     loss = sum(dout * o) + <dS_last, S_last>
 * with respect to q, k, v, g and S0.
 *   ckpt:  written by lr_gla_scan with the same seg.
 *   dout:  [B, L, H, V] io      dS_last: [B, H, K, V] fp32 or NULL (= 0)
 *   dq, dk: [B, L, H, K] io     dv: [B, L, H, V] io     dg: [B, L, H] io
 *   dS0:   [B, H, K, V] fp32 or NULL
 *   workspace: device memory of lr_gla_scan_bwd_workspace_bytes() bytes;
 *            smaller down to one-row batch slices as in lr_ssd_scan_bwd
 *            (lr_gla_scan_bwd_workspace_bytes(1, L, ...)
 *            + 8 (B - 1) H (V / 64) ceil(L / seg) + 512 bytes suffice).
 * Supported: as lr_gla_scan, with seg in {64, 128, 192, 256}.
 * ------------------------------------------------------------------------- */
lr_status lr_gla_scan_bwd(lr_dtype io, int64_t B, int64_t L, int64_t H,
                          int64_t K, int64_t V, int64_t chunk, int64_t seg,
                          const void* q, const void* k, const void* v,
                          const void* g, const float* ckpt, const void* dout,
                          const float* dS_last, void* dq, void* dk, void* dv,
                          void* dg, float* dS0, void* workspace,
                          size_t workspace_bytes, void* stream);

/* ===========================================================================
 * Single-token steps (decode).  "lrnnx: A library for Linear RNNs" gives
 * every layer a step method for autoregressive generation, checked against
 * the parallel and recurrent modes, and runs the decode loop under graph
 * capture.  Each call advances the caller's fp32 state h (or S) by one token
 * IN PLACE and writes the token's output; T calls reproduce the matching
 * scan over T tokens.  The calls allocate nothing, never synchronise and
 * issue no memset, so a loop of them can be captured into a HIP graph.
 * Same conventions as above; shapes are the scan's with the L axis removed.
 * ======================================================================== */

/* h = a (.) h + b;  out = h (io; may be NULL).
 *   a, b, out: [B, D] io    h: [B, D] fp32 in/out */
lr_status lr_diag_step(lr_dtype io, int64_t B, int64_t D, const void* a,
                       const void* b, float* h, void* out, void* stream);

/* One token of lr_selective_scan.
 *   x, dt, y: [B, D] io    Bm, Cm: [B, N] io    A: [D, N]    Dskip: [D] or NULL
 *   h: [B, D, N] fp32 in/out.  Supported: 1 <= N <= 64. */
lr_status lr_selective_step(lr_dtype io, lr_disc disc, int64_t B, int64_t D,
                            int64_t N, const void* x, const void* dt,
                            const float* A, const void* Bm, const void* Cm,
                            const float* Dskip, float* h, void* y,
                            void* stream);

/* One token of lr_ssd_scan.
 *   x, y: [B, H, P] io    dt: [B, H] io    Bm, Cm: [B, G, N] io
 *   A: [H]    Dskip: [H] or NULL    h: [B, H, P, N] fp32 in/out.
 * Supported: io = LR_BF16; N in {64, 128}; H % G == 0. */
lr_status lr_ssd_step(lr_dtype io, lr_disc disc, int64_t B, int64_t H,
                      int64_t P, int64_t G, int64_t N, const void* x,
                      const void* dt, const float* A, const void* Bm,
                      const void* Cm, const float* Dskip, float* h, void* y,
                      void* stream);

/* One token of lr_gla_scan.
 *   q, k: [B, H, K] io    v, o: [B, H, V] io    g: [B, H] io
 *   S: [B, H, K, V] fp32 in/out.  Supported: io = LR_BF16; V % 64 == 0. */
lr_status lr_gla_step(lr_dtype io, int64_t B, int64_t H, int64_t K, int64_t V,
                      const void* q, const void* k, const void* v,
                      const void* g, float* S, void* o, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LR_H_ */
