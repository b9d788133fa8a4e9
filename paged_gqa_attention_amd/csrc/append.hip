// K/V append: writes the new K and V rows of each sequence into its pages of
// the paged pool, converting them to the storage type (Geramy/LSE README,
// "K/V storage": 16-bit and FP8 cache storage).
//
// Row i of sequence b (of n_new rows) lands at position p = L_b - n_new + i,
// L_b = min(seq_lens[b], capacity): page_table[b][p / 16], slot p % 16.  The
// stored value is src / scale (one IEEE single-precision division), rounded to
// the storage type to nearest, ties to even; F16/BF16 overflow to infinity,
// e4m3fn saturates at +-448, e5m2 saturates finite values at +-57344 and keeps
// infinities; NaN stays NaN.
//
// With per-vector scales (8-bit storage, template flag VS; Geramy/LSE README,
// "K/V storage": fp8 and bf8 caches with scales) the scale of each new K or V
// vector is amax / fmax (amax over its finite entries, fmax the format's
// largest finite value; 1 if that is 0): the threads of a token row reduce
// their maxima with lane exchanges, one of them stores the scale, and every
// element is divided by it before rounding.
//
// One workgroup owns the new slots of four consecutive pages of one (sequence,
// KV head): each thread converts 8 consecutive elements of a token row, stores
// them to the token-major K tile and stages the V codes in LDS; the
// token-minor V tiles are then written 16 bytes (one component's consecutive
// slots) per store.
#include "attn_internal.h"
#include "common.h"

namespace pa {

namespace {

constexpr int kAppendThreads = 256;
// pages (16 slots each) per workgroup: 4, or 2 at head_dim 256 (LDS staging)
template <int D> constexpr int append_pages() { return D >= 256 ? 2 : 4; }

__device__ __forceinline__ uint32_t enc_bf16(float y) {
  const uint32_t u = __float_as_uint(y);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;   // NaN
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;                                 // RNE
}

__device__ __forceinline__ uint32_t enc_f16(float y) {
  const uint32_t u = __float_as_uint(y);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7e00u;   // NaN
  const _Float16 h = (_Float16)y;                          // v_cvt_f16_f32: RNE, IEEE
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// OCP e4m3fn (bias 7, largest finite 448 = 0x7e), saturating
__device__ __forceinline__ uint32_t enc_e4m3(float y) {
  // the hardware conversion rounds to nearest even, subnormals included;
  // finite magnitudes above the largest code (and infinities) are clamped to
  // it first.  NaN is written as sign | 0x7f (the conversion sets other bits).
  const float c = __builtin_fabsf(y) > 448.f ? __builtin_copysignf(448.f, y) : y;
  const uint32_t code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xffu;
  return y != y ? (((__float_as_uint(y) >> 24) & 0x80u) | 0x7fu) : code;
}

// OCP e5m2 (bias 15, largest finite 57344 = 0x7b), finite values saturating,
// infinities kept; the same conversion scheme as e4m3fn
__device__ __forceinline__ uint32_t enc_e5m2(float y) {
  const float a = __builtin_fabsf(y);
  const float c = (a > 57344.f && a != __builtin_inff()) ? __builtin_copysignf(57344.f, y) : y;
  const uint32_t code = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c, c, 0, false) & 0xffu;
  return y != y ? (((__float_as_uint(y) >> 24) & 0x80u) | 0x7fu) : code;
}

template <int SRC>
__device__ __forceinline__ void load8(const char *p, float *x) {
  if constexpr (SRC == DT_F32) {
    const u32x4 a = ld16(p), b = ld16(p + 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) { x[e] = __uint_as_float(a[e]); x[4 + e] = __uint_as_float(b[e]); }
  } else {
    const u32x4 a = ld16(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (SRC == DT_BF16) {
        x[2 * e] = bf16_lo(a[e]);
        x[2 * e + 1] = bf16_hi(a[e]);
      } else {
        x[2 * e] = f16_lo(a[e]);
        x[2 * e + 1] = f16_hi(a[e]);
      }
    }
  }
}

template <int KVDT>
__device__ __forceinline__ uint32_t encode(float y) {
  if constexpr (KVDT == DT_F32) return __float_as_uint(y);
  else if constexpr (KVDT == DT_BF16) return enc_bf16(y);
  else if constexpr (KVDT == DT_F16) return enc_f16(y);
  else if constexpr (KVDT == DT_BF8) return enc_e5m2(y);
  else return enc_e4m3(y);
}

// largest finite value of an 8-bit storage type
template <int KVDT>
constexpr float fmax8() { return KVDT == DT_BF8 ? 57344.0f : 448.0f; }

// per-vector scale of the token row whose TPT threads (consecutive lanes,
// 8 values each) hold x: amax over the finite values / fmax, 1 if that is 0
template <int KVDT, int TPT>
__device__ __forceinline__ float vector_scale(const float *x) {
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float v = __builtin_fabsf(x[e]);
    m = v <= 3.402823466e38f ? __builtin_fmaxf(m, v) : m;   // NaN and inf do not count
  }
#pragma unroll
  for (int k = 1; k < TPT; k <<= 1) m = __builtin_fmaxf(m, shfl_xor(m, k));
  const float u = m / fmax8<KVDT>();
  return u == 0.f ? 1.f : u;
}

// 8 codes -> one store of 8 elements of the storage type
template <int KVDT>
__device__ __forceinline__ void store8(char *p, const uint32_t *c) {
  if constexpr (KVDT == DT_F32) {
    gstore<u32x4>(p, u32x4{c[0], c[1], c[2], c[3]});
    gstore<u32x4>(p + 16, u32x4{c[4], c[5], c[6], c[7]});
  } else if constexpr (is8bit(KVDT)) {
    u32x2 w;
    w[0] = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    w[1] = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
    gstore<u32x2>(p, w);
  } else {
    gstore<u32x4>(p, u32x4{c[0] | (c[1] << 16), c[2] | (c[3] << 16),
                           c[4] | (c[5] << 16), c[6] | (c[7] << 16)});
  }
}

// 16 bytes of codes (16 / element-size codes) -> one store
template <int KVDT>
__device__ __forceinline__ void store_vec(char *p, const uint32_t *c) {
  if constexpr (KVDT == DT_F32) {
    gstore<u32x4>(p, u32x4{c[0], c[1], c[2], c[3]});
  } else if constexpr (is8bit(KVDT)) {
    u32x4 w;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = c[4 * q] | (c[4 * q + 1] << 8) | (c[4 * q + 2] << 16) | (c[4 * q + 3] << 24);
    gstore<u32x4>(p, w);
  } else {
    gstore<u32x4>(p, u32x4{c[0] | (c[1] << 16), c[2] | (c[3] << 16),
                           c[4] | (c[5] << 16), c[6] | (c[7] << 16)});
  }
}

template <int KVDT>
__device__ __forceinline__ void store1(char *p, uint32_t c) {
  if constexpr (KVDT == DT_F32) gstore<uint32_t>(p, c);
  else if constexpr (is8bit(KVDT)) gstore<uint8_t>(p, (uint8_t)c);
  else gstore<uint16_t>(p, (uint16_t)c);
}

template <int KVDT, int SRC, int D, bool VS>
__global__ __launch_bounds__(kAppendThreads) void kv_append(AppendArgs a) {
  constexpr int ELT = DtInfo<KVDT>::bytes;
  constexpr int SELT = DtInfo<SRC>::bytes;
  constexpr int TPT = D / 8;                  // threads per token row (8 elements each)
  constexpr int NS = 16 * append_pages<D>();       // slots of this workgroup
  constexpr int VG = 16 / ELT;                // slots per 16-byte V store
  __shared__ uint32_t vstage[NS][D + 1];      // V codes [slot][component] (+1: no bank conflicts)

  const int g = blockIdx.y, b = blockIdx.z;
  const int L = min(a.lens[b], a.capacity);
  const int first = max(0, L - a.n_new);      // first position written
  if (first >= L) return;
  const int page0 = first / 16 + blockIdx.x * append_pages<D>();   // first logical page
  const int p0 = page0 * 16;
  if (p0 >= L) return;
  const int s_lo = max(first, p0) - p0, s_hi = min(L, p0 + NS) - p0;   // slots [s_lo, s_hi)
  const char *ksrc = reinterpret_cast<const char *>(a.k_src);
  const char *vsrc = reinterpret_cast<const char *>(a.v_src);
  const int32_t *pt = a.page_table + (int64_t)b * a.pt_stride;
  auto tile = [&](void *base, const uint64_t *frags, int64_t sp, int64_t sh, int slot) {
    const int64_t pid = pt[page0 + slot / 16];
    return page_addr_lane(reinterpret_cast<char *>(base) + (int64_t)g * sh * ELT, frags,
                          a.frag_shift, pid, sp * ELT, (int64_t)g * sh * ELT);
  };

  // phase 1: token rows -> K tiles (token-major) and V codes -> LDS
  for (int idx = threadIdx.x; idx < NS * TPT; idx += kAppendThreads) {
    const int slot = idx / TPT, part = idx % TPT;
    if (slot < s_lo || slot >= s_hi) continue;
    const int row = p0 + slot - (L - a.n_new);                      // source row index
    const int64_t off = ((int64_t)b * a.s_b + (int64_t)row * a.s_r + (int64_t)g * a.s_h + part * 8) * SELT;
    float xk[8], xv[8];
    load8<SRC>(ksrc + off, xk);
    load8<SRC>(vsrc + off, xv);
    float uk = a.k_scale, uv = a.v_scale;
    if constexpr (VS) {
      // a slot's TPT threads are consecutive lanes of one wave, all present
      uk = vector_scale<KVDT, TPT>(xk);
      uv = vector_scale<KVDT, TPT>(xv);
      if (part == 0) {
        const int64_t si = (int64_t)pt[page0 + slot / 16] * a.vs_sp + (int64_t)g * a.vs_sh + slot % 16;
        a.k_vs[si] = uk;
        a.v_vs[si] = uv;
      }
    }
    uint32_t ck[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ck[e] = encode<KVDT>(xk[e] / uk);
      vstage[slot][part * 8 + e] = encode<KVDT>(xv[e] / uv);
    }
    store8<KVDT>(tile(a.k, a.k_frag, a.k_sp, a.k_sh, slot) + ((int64_t)(slot % 16) * D + part * 8) * ELT, ck);
  }
  __syncthreads();
  // phase 2: V tiles (token-minor): 16 bytes (VG slots of one component) per
  // store where all of them are new, single elements at the edges
  for (int idx = threadIdx.x; idx < NS / VG * D; idx += kAppendThreads) {
    const int d = idx / (NS / VG), s0 = (idx % (NS / VG)) * VG;
    if (s0 + VG <= s_lo || s0 >= s_hi) continue;
    char *vt = tile(a.v, a.v_frag, a.v_sp, a.v_sh, s0) + ((int64_t)d * 16 + s0 % 16) * ELT;
    if (s0 >= s_lo && s0 + VG <= s_hi) {
      uint32_t c[16];
#pragma unroll
      for (int e = 0; e < VG; ++e) c[e] = vstage[s0 + e][d];
      store_vec<KVDT>(vt, c);
    } else {
      for (int e = 0; e < VG; ++e)
        if (s0 + e >= s_lo && s0 + e < s_hi) store1<KVDT>(vt + e * ELT, vstage[s0 + e][d]);
    }
  }
}

template <int KV, int SRC, bool VS>
hipError_t append_d(const AppendArgs &a, hipStream_t s) {
  auto grid = [&](int pages) { return dim3(((a.n_new + 15) / 16 + 1 + pages - 1) / pages, a.Hkv, a.B); };
  if (a.D == 64) hipLaunchKernelGGL((kv_append<KV, SRC, 64, VS>), grid(append_pages<64>()), dim3(kAppendThreads), 0, s, a);
  else if (a.D == 128) hipLaunchKernelGGL((kv_append<KV, SRC, 128, VS>), grid(append_pages<128>()), dim3(kAppendThreads), 0, s, a);
  else hipLaunchKernelGGL((kv_append<KV, SRC, 256, VS>), grid(append_pages<256>()), dim3(kAppendThreads), 0, s, a);
  return hipGetLastError();
}

template <int KV, bool VS>
hipError_t append_s(const AppendArgs &a, hipStream_t s) {
  switch (a.src_dtype) {
    case DT_F32: return append_d<KV, DT_F32, VS>(a, s);
    case DT_F16: return append_d<KV, DT_F16, VS>(a, s);
    default: return append_d<KV, DT_BF16, VS>(a, s);
  }
}

template <int KV>
hipError_t append_8(const AppendArgs &a, hipStream_t s) {
  return a.k_vs ? append_s<KV, true>(a, s) : append_s<KV, false>(a, s);
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs &a, hipStream_t s) {
  switch (a.kv_dtype) {
    case DT_F32: return append_s<DT_F32, false>(a, s);
    case DT_F16: return append_s<DT_F16, false>(a, s);
    case DT_BF16: return append_s<DT_BF16, false>(a, s);
    case DT_FP8: return append_8<DT_FP8>(a, s);
    default: return append_8<DT_BF8>(a, s);
  }
}

}  // namespace pa
