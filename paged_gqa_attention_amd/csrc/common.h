// Device helpers shared by the gfx950 attention kernels: storage-dtype
// conversions, cross-lane reductions and MFMA fragment types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// storage types; FP8 is OCP e4m3fn, BF8 is OCP e5m2
enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_FP8 = 3, DT_BF8 = 4 };

template <int DT> struct DtInfo;
template <> struct DtInfo<DT_F32>  { static constexpr int bytes = 4; };
template <> struct DtInfo<DT_F16>  { static constexpr int bytes = 2; };
template <> struct DtInfo<DT_BF16> { static constexpr int bytes = 2; };
template <> struct DtInfo<DT_FP8>  { static constexpr int bytes = 1; };
template <> struct DtInfo<DT_BF8>  { static constexpr int bytes = 1; };

__host__ __device__ constexpr bool is8bit(int dt) { return dt == DT_FP8 || dt == DT_BF8; }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kPage = 16;

// ---- 16-byte global loads ------------------------------------------------------
// The pointers are cast to the global address space: a pointer built from a
// fragment table entry is otherwise generic, and generic (flat) loads also
// count on the LDS counter, so every wait for an LDS read would wait for
// them too.

typedef const __attribute__((address_space(1))) u32x4 gu32x4;
typedef const __attribute__((address_space(1))) u32x2 gu32x2;

__device__ __forceinline__ u32x4 ld16(const void *p) {
  return *(gu32x4 *)p;
}
__device__ __forceinline__ u32x2 ld8(const void *p) {
  return *(gu32x2 *)p;
}
// a store through a global address space pointer (not a flat store)
template <typename T>
__device__ __forceinline__ void gstore(void *p, T v) {
  *(__attribute__((address_space(1))) T *)p = v;
}
// Non-temporal loads, for data a kernel reads exactly once (the K/V a decode
// partition streams): they do not allocate in the caches, which measured
// 6.1 against 5.4 TB/s for the paged decode stream on MI355X.
__device__ __forceinline__ u32x4 ld16_nt(const void *p) {
  return __builtin_nontemporal_load((gu32x4 *)p);
}
__device__ __forceinline__ u32x2 ld8_nt(const void *p) {
  return __builtin_nontemporal_load((gu32x2 *)p);
}
// A non-temporal 16-byte load at base + off through a buffer resource of
// `bytes` bytes (base wave-uniform): with bytes = 0 it returns zeros without
// a memory access, so a load that may be past the end needs no branch (the
// compiler then counts the loads in flight exactly).  Data format 32 bits in
// the resource's fourth word, as raw buffer loads require.
__device__ __forceinline__ u32x4 ld16_nt_buf(const void *base, uint32_t off, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void *ub = (void *)(uintptr_t)(((uint64_t)hi << 32) | lo);
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2));
}

// ---- page addressing ---------------------------------------------------------------

// Address of the (page pid, head) tile of a pool.  Contiguous pools:
// base_head + pid * page_bytes, base_head = pool base + head offset.  With a
// fragment table (frags != null) page pid is page (pid & (2^shift - 1)) of
// fragment pid >> shift, whose device address the table holds.  pid must be
// wave-uniform: the table entry is read with a scalar load.
__device__ __forceinline__ const char *page_addr(const char *base_head, const uint64_t *frags,
                                                 int shift, int64_t pid, int64_t page_bytes,
                                                 int64_t head_bytes) {
  if (frags) {
    typedef const __attribute__((address_space(4))) uint64_t cu64;
    const uint64_t f = ((cu64 *)frags)[pid >> shift];
    return reinterpret_cast<const char *>(f) + head_bytes +
           (pid & ((int64_t(1) << shift) - 1)) * page_bytes;
  }
  return base_head + pid * page_bytes;
}

// the same for a per-lane page id (vector load of the table entry)
__device__ __forceinline__ char *page_addr_lane(char *base_head, const uint64_t *frags, int shift,
                                                int64_t pid, int64_t page_bytes,
                                                int64_t head_bytes) {
  if (frags)
    return reinterpret_cast<char *>(frags[pid >> shift]) + head_bytes +
           (pid & ((int64_t(1) << shift) - 1)) * page_bytes;
  return base_head + pid * page_bytes;
}

// ---- storage -> FP32 -------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2, w)[0];
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2, w)[1];
}
// Two 8-bit codes of type KV (bytes 0,1 of w if !HI, else 2,3) to FP32,
// exact.  e4m3fn and e5m2 values are all representable in FP32, bf16 and
// f16, so every conversion below is exact.
template <int KV, bool HI>
__device__ __forceinline__ f32x2 e8x2_to_f32(uint32_t w) {
  if constexpr (KV == DT_BF8) return __builtin_amdgcn_cvt_pk_f32_bf8(w, HI);
  else return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}
// two codes to a packed bf16 / f16 pair.  The scaled conversions take only the
// exponent of their FP32 scale operand (measured on gfx950): with 1.0 they are
// plain exact conversions.
template <int KV, bool HI>
__device__ __forceinline__ uint32_t e8x2_to_bf16x2(uint32_t w) {
  if constexpr (KV == DT_BF8)
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HI));
  else
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
template <int KV, bool HI>
__device__ __forceinline__ uint32_t e8x2_to_f16x2(uint32_t w) {
  if constexpr (KV == DT_BF8)
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, HI));
  else
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}
// to the 16-bit MFMA/dot operand type (f16 if F16 else bf16)
template <int KV, bool F16, bool HI>
__device__ __forceinline__ uint32_t e8x2_to_16(uint32_t w) {
  if constexpr (F16) return e8x2_to_f16x2<KV, HI>(w);
  else return e8x2_to_bf16x2<KV, HI>(w);
}

// element e of a 16-byte chunk of dtype DT, to FP32
template <int DT>
__device__ __forceinline__ float chunk_elem(const u32x4 &c, int e) {
  if constexpr (DT == DT_F32) {
    return __uint_as_float(c[e]);
  } else if constexpr (DT == DT_BF16) {
    uint32_t w = c[e >> 1];
    return (e & 1) ? bf16_hi(w) : bf16_lo(w);
  } else if constexpr (DT == DT_F16) {
    uint32_t w = c[e >> 1];
    return (e & 1) ? f16_hi(w) : f16_lo(w);
  } else {
    uint32_t w = c[e >> 2];
    f32x2 v = (e & 2) ? e8x2_to_f32<DT, true>(w) : e8x2_to_f32<DT, false>(w);
    return (e & 1) ? v[1] : v[0];
  }
}

// ---- FP32 -> storage ---------------------------------------------------------------

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 r;
  r[0] = (__bf16)a;  // RNE
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  f16x2 r;
  r[0] = (_Float16)a;
  r[1] = (_Float16)b;
  return __builtin_bit_cast(uint32_t, r);
}

template <int DT>
__device__ __forceinline__ void store_out(void *base, int64_t idx, float v) {
  if constexpr (DT == DT_F32) {
    reinterpret_cast<float *>(base)[idx] = v;
  } else if constexpr (DT == DT_BF16) {
    reinterpret_cast<__bf16 *>(base)[idx] = (__bf16)v;
  } else {
    reinterpret_cast<_Float16 *>(base)[idx] = (_Float16)v;
  }
}

// ---- 2-element dot products with FP32 accumulation --------------------------------

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c,
                                false);
}

// ---- cross-lane -----------------------------------------------------------------------

// DPP controls (GFX9 encoding)
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), CTRL, 0xF, 0xF,
                                                     false));
}

__device__ __forceinline__ float shfl_xor(float v, int m) {
  int lane = __lane_id();
  return __uint_as_float(__builtin_amdgcn_ds_bpermute((lane ^ m) << 2, __float_as_uint(v)));
}

// Reductions across the two 32-lane halves / the 16-lane quarters of a wave.
// v_permlane32_swap(x, x) returns (x[0:32], x[0:32]) and (x[32:64], x[32:64]);
// combining the two gives the pairwise result in every lane (gfx950).
__device__ __forceinline__ float max_xor32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 3-input maximum.  Plain code, not inline asm: its operands are often MFMA
// results, and the compiler inserts the wait states a VALU read of an MFMA
// result needs only for instructions it can see (it forms v_max3_f32 itself).
__device__ __forceinline__ float max3(float a, float b, float c) {
  return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}

}  // namespace pa
