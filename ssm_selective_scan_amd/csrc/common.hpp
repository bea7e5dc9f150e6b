// common.hpp — device primitives shared by the liblr kernels (gfx950, wave64).
//
//  * bf16 <-> fp32 conversion (round to nearest even)
//  * wave64 inclusive scans through DPP: a plain sum scan (log-decay segment
//    sums) and the (a, b)-pair scan of the associative combine
//        (a2, b2) o (a1, b1) = (a2 a1, a2 b1 + b2)
//    (IBM Research blog "K-Search for MLX", section "A 20x faster prefill:
//    the Mamba SSM kernel", combine equation)
//  * MFMA 16x16x32 bf16 operand helpers
//  * (host) the compute-unit count of the current device
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace lr {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- bf16 / io
__device__ __forceinline__ float bf2f(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}
// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// I/O element types: float (LR_F32) or uint16_t holding bf16 bits (LR_BF16).
template <typename T> struct Io;
template <> struct Io<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
  __device__ __forceinline__ static float cvt(float v) { return v; }
};
template <> struct Io<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t* p) { return bf2f(*p); }
  __device__ __forceinline__ static void store(uint16_t* p, float v) { *p = f2bf(v); }
  __device__ __forceinline__ static float cvt(uint16_t v) { return bf2f(v); }
};

// CPL consecutive elements of T as loaded: fp32 words, or bf16 values packed
// in 32-bit words.  Scans keep loaded elements raw and convert them (vcvt)
// only once every load of a segment has been issued: memory loads retire in
// order, so a conversion next to its load would make the wave wait for that
// load, and all earlier ones, before issuing the next.
template <typename T, int CPL> struct VRaw { float v[CPL]; };
template <> struct VRaw<uint16_t, 1> { uint16_t v; };
template <> struct VRaw<uint16_t, 2> { uint32_t v; };
template <> struct VRaw<uint16_t, 4> { uint2 v; };

template <typename T, int CPL>
__device__ __forceinline__ VRaw<T, CPL> vload_raw(const T* p) {
  VRaw<T, CPL> r;
  if constexpr (sizeof(T) == 4) {
    if constexpr (CPL == 1) {
      r.v[0] = *p;
    } else if constexpr (CPL == 2) {
      const float2 x = *reinterpret_cast<const float2*>(p);
      r.v[0] = x.x; r.v[1] = x.y;
    } else {
      const float4 x = *reinterpret_cast<const float4*>(p);
      r.v[0] = x.x; r.v[1] = x.y; r.v[2] = x.z; r.v[3] = x.w;
    }
  } else if constexpr (CPL == 1) {
    r.v = *p;
  } else if constexpr (CPL == 2) {
    r.v = *reinterpret_cast<const uint32_t*>(p);
  } else {
    r.v = *reinterpret_cast<const uint2*>(p);
  }
  return r;
}
// x as one element of T, unconverted (exact in bf16 for the 0 and 1 used here)
template <typename T> __device__ __forceinline__ T raw_of(float x) {
  if constexpr (sizeof(T) == 4) return x;
  else return static_cast<T>(f2bf(x));
}
// every element equal to x
template <typename T, int CPL>
__device__ __forceinline__ VRaw<T, CPL> vfill_raw(float x) {
  VRaw<T, CPL> r;
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int k = 0; k < CPL; ++k) r.v[k] = x;
  } else {
    const uint32_t b = f2bf(x);
    if constexpr (CPL == 1) r.v = static_cast<uint16_t>(b);
    else if constexpr (CPL == 2) r.v = b | (b << 16);
    else r.v = uint2{b | (b << 16), b | (b << 16)};
  }
  return r;
}
template <typename T, int CPL>
__device__ __forceinline__ void vcvt(const VRaw<T, CPL>& r, float (&v)[CPL]) {
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int k = 0; k < CPL; ++k) v[k] = r.v[k];
  } else if constexpr (CPL == 1) {
    v[0] = bf2f(r.v);
  } else if constexpr (CPL == 2) {
    v[0] = bf2f(static_cast<uint16_t>(r.v)); v[1] = bf2f(static_cast<uint16_t>(r.v >> 16));
  } else {
    v[0] = bf2f(static_cast<uint16_t>(r.v.x)); v[1] = bf2f(static_cast<uint16_t>(r.v.x >> 16));
    v[2] = bf2f(static_cast<uint16_t>(r.v.y)); v[3] = bf2f(static_cast<uint16_t>(r.v.y >> 16));
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ------------------------------------------------------------------ DPP scans
// dpp_ctrl encodings (GCN/CDNA): row_shr:n = 0x110+n, wave_shr:1 = 0x138,
// row_bcast:15 = 0x142, row_bcast:31 = 0x143.  A lane whose DPP source is
// invalid, or whose row is masked off, keeps `old`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float old, float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src),
                                                    CTRL, ROW_MASK, 0xf, false));
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_incl_sum(float v) {
  v += dpp_f<0x111, 0xf>(0.f, v);
  v += dpp_f<0x112, 0xf>(0.f, v);
  v += dpp_f<0x114, 0xf>(0.f, v);
  v += dpp_f<0x118, 0xf>(0.f, v);
  v += dpp_f<0x142, 0xa>(0.f, v);
  v += dpp_f<0x143, 0xc>(0.f, v);
  return v;
}

// One step of the pair scan: combine the lane's pair (later) with the pair
// received from an earlier lane; lanes without a source receive (1, 0), the
// identity of the combine.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void pair_step(float& a, float& b) {
  float pa = dpp_f<CTRL, ROW_MASK>(1.f, a);
  float pb = dpp_f<CTRL, ROW_MASK>(0.f, b);
  b = fmaf(a, pb, b);
  a = a * pa;
}

// Inclusive scan of (a, b) pairs over the 64 lanes (lane 0 is earliest):
// on return lane i holds (a_i ... a_0, h_i) with h the recurrence from 0.
__device__ __forceinline__ void wave_incl_pair_scan(float& a, float& b) {
  pair_step<0x111, 0xf>(a, b);
  pair_step<0x112, 0xf>(a, b);
  pair_step<0x114, 0xf>(a, b);
  pair_step<0x118, 0xf>(a, b);
  pair_step<0x142, 0xa>(a, b);
  pair_step<0x143, 0xc>(a, b);
}

// Shift a value one lane up across the whole wave (lane 0 receives `fill`).
__device__ __forceinline__ float wave_shr1(float v, float fill) {
  return dpp_f<0x138, 0xf>(fill, v);
}

// ----------------------------------------------------------------------- MFMA
// v_mfma_f32_16x16x32_bf16:  D[16x16] += A[16x32] * B[32x16]
//   A operand: lane l holds A[l % 16][8 (l / 16) + j], j = 0..7
//   B operand: lane l holds B[8 (l / 16) + j][l % 16]
//   D:         lane l holds D[4 (l / 16) + r][l % 16], r = 0..3
// Only the pairing of (lane group, slot) between A and B matters for the
// product, so any k-permutation applied to both operands is allowed.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u16x8 v) { return __builtin_bit_cast(bf16x8, v); }

// 16x32 operand tile from LDS stored [row][k] (k contiguous, leading dim ld
// elements, ld % 8 == 0): rows row0.., k-block k0.
__device__ __forceinline__ bf16x8 lds_tile(const uint16_t* base, int ld, int row0, int k0, int lane) {
  const uint16_t* p = base + (row0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4);
  return as_bf16x8(*reinterpret_cast<const u16x8*>(p));
}

// Same, with the k-permutation that matches two D tiles used as the other
// operand: slot j < 4 <-> k0 + 4 g + j, slot j >= 4 <-> k0 + 16 + 4 g + j - 4.
__device__ __forceinline__ bf16x8 lds_tile_perm(const uint16_t* base, int ld, int row0, int k0, int lane) {
  const uint16_t* p = base + (row0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4);
  u16x4 lo = *reinterpret_cast<const u16x4*>(p);
  u16x4 hi = *reinterpret_cast<const u16x4*>(p + 16);
  u16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return as_bf16x8(v);
}

// 16x32 operand tile from LDS stored [k][m] (m contiguous, leading dim ld,
// ld % 4 == 0): operand index m0 + (lane & 15), k-block k0.  Uses gfx950's
// transposing LDS read ds_read_b64_tr_b16: inside each group of 16 lanes, lane
// i receives element j of the 8-byte chunk addressed by lane 4 j + i / 4, at
// position i % 4.  Lane m of group g therefore addresses row k0 + 8 g + m / 4
// (then + 4 for the second half), columns m0 + 4 (m % 4) .. + 3, and ends up
// with column m0 + (lane & 15), rows k0 + 8 g + 0..7.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;
__device__ __forceinline__ bf16x8 lds_tile_tr(const uint16_t* base, int ld, int k0, int m0, int lane) {
  const int g = lane >> 4, m = lane & 15;
  const uint16_t* p = base + (k0 + 8 * g + (m >> 2)) * ld + m0 + 4 * (m & 3);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(p + 4 * ld));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Two fp32 D tiles (k rows 0-15 and 16-31 of a 32-k block) -> one bf16
// operand with the permutation of lds_tile_perm.
__device__ __forceinline__ bf16x8 pack_dd(f32x4 lo, f32x4 hi) {
  u16x8 v = {f2bf(lo[0]), f2bf(lo[1]), f2bf(lo[2]), f2bf(lo[3]),
             f2bf(hi[0]), f2bf(hi[1]), f2bf(hi[2]), f2bf(hi[3])};
  return as_bf16x8(v);
}

// Compute units of the current device (0 if the query fails), cached per
// device after the first call.
inline int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 0;
  }
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      (void)hipGetLastError();
      v = -1;
    }
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v > 0 ? v : 0;
}

// blockIdx -> logical work id such that consecutive logical ids run on the
// same XCD (the dispatcher hands workgroups to the 8 XCDs round-robin).
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
  const int x = bid & 7;
  const int per = nwg >> 3, rem = nwg & 7;
  return x * per + (x < rem ? x : rem) + (bid >> 3);
}

}  // namespace lr
