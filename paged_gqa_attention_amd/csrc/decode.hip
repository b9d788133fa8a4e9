// Paged decode / speculative-verify attention for gfx950.
//
// One workgroup (4 waves) owns one KV partition of one (sequence, KV head)
// and all the query rows that read that KV head: the G query heads of the
// group times the R verify rows (Geramy/LSE releases, v0.4.21: K/V reads
// shared across query heads and token rows).  Each wave walks pages of the
// partition, keeps an online-softmax state per row in FP32, the four waves
// are merged in LDS, and the partition's unnormalised output, running max and
// sum go to the workspace.  A second kernel merges the partitions with a
// log-sum-exp merge and adds the sink (Geramy/LSE releases, v0.4.19: one
// partial family and one merge family; v0.4.20: partitions from K/V table
// capacity, empty partitions skipped).
//
// Two partial kernels:
//   decode_valu  FP32 VALU arithmetic, up to 8 rows per workgroup.  Used for
//                single-row decode (HBM-bound, no matrix cores needed) and for
//                FP32 K/V.  Four lanes share a token for Q.K; lanes own value
//                components for P.V.
//   decode_mfma  bf16/f16 MFMA 16x16x32 for 16..64 rows (multi-row verify):
//                S^T = K.Q^T and O^T += V^T.P^T, so every lane's softmax row
//                matches its accumulator row and V tiles (token-minor pages)
//                load straight into MFMA operands.
// With per-vector scales (8-bit K/V, template flag VS) a token's K scale
// multiplies its scores and its V scale its softmax weights before P.V; the
// row sums use the unscaled weights.
#include <type_traits>

#include "attn_internal.h"
#include "common.h"

namespace pa {

// Page loops are emitted twice inside each partial kernel, once per
// addressing mode, so that the contiguous-pool loop carries no trace of the
// fragment lookup; one uniform branch per workgroup picks the loop.
using Contiguous = std::false_type;
using Fragmented = std::true_type;

constexpr int kWaves = 4;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ int uniform_int(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------------
// Intra-workgroup merge of the four waves' softmax states, then the partial
// write.  `m_w`/`l_w` are [kWaves][NR] in LDS, `acc` is [NR][D] in LDS.
// Each wave calls add_wave() in turn (deterministic order).
// ---------------------------------------------------------------------------------
template <int NR>
__device__ __forceinline__ void wave_scales(const float (*m_w)[NR], int wave, int r, float &M,
                                            float &f) {
  M = kNegInf;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = __builtin_fmaxf(M, m_w[w][r]);
  float Mu = (M == kNegInf) ? 0.f : M;
  f = fast_exp2(m_w[wave][r] - Mu);
}

// ==================================================================================
// Log-sum-exp merge of the partitions + sink, one wave per output row
// ==================================================================================
// Row rr of (sequence b, KV head kvh) from its Pl partials, partial k at
// workspace index base + k * stride.
template <int D>
__device__ __forceinline__ void merge_row(const DecodeArgs &a, int b, int kvh, int rr, int Pl,
                                          int64_t base, int64_t stride, int lane) {
  constexpr int DPL = D / 64;
  constexpr int CH = 8;                  // partitions whose outputs are loaded at once
  const int h = kvh * a.G + rr / a.R, i = rr % a.R;
  const float sink = a.sinks ? a.sinks[h] * kLog2e : kNegInf;

  float o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.f;
  float M = sink, zp = 0.f;
  // partitions in chunks of 64 for the statistics and CH for the outputs; all
  // loads of a chunk are issued before any of them is used
  for (int p0 = 0; p0 < Pl; p0 += 64) {
    const int pm = p0 + lane;
    const float mp = pm < Pl ? a.ws_ml[(base + pm * stride) * 2] : kNegInf;
    const float lp = pm < Pl ? a.ws_ml[(base + pm * stride) * 2 + 1] : 0.f;
    float Mc = mp;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) Mc = __builtin_fmaxf(Mc, shfl_xor(Mc, m));
    const float Mn = __builtin_fmaxf(M, Mc);
    if (Mn == kNegInf) continue;
    const float rescale = fast_exp2(M - Mn);   // earlier chunks (M = -inf: 0)
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] *= rescale;
    zp *= rescale;
    M = Mn;
    const float w = (mp == kNegInf) ? 0.f : fast_exp2(mp - M);
    zp += w * lp;
    const int cnt = min(64, Pl - p0);
    for (int q0 = 0; q0 < cnt; q0 += CH) {
      float ov[CH][DPL];
#pragma unroll
      for (int q = 0; q < CH; ++q) {
        const int qq = q0 + q < cnt ? q0 + q : cnt - 1;
        const float *op = a.ws_o + (base + (p0 + qq) * stride) * D;
#pragma unroll
        for (int e = 0; e < DPL; ++e) ov[q][e] = op[lane + 64 * e];
      }
#pragma unroll
      for (int q = 0; q < CH; ++q) {
        if (q0 + q < cnt) {
          const float wq = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(w), q0 + q));
#pragma unroll
          for (int e = 0; e < DPL; ++e) o[e] = __builtin_fmaf(wq, ov[q][e], o[e]);
        }
      }
    }
  }
  float Z = 0.f;
  if (M != kNegInf) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) zp += shfl_xor(zp, m);
    Z = zp + fast_exp2(sink - M);
  }
  const float inv = (M == kNegInf) ? 0.f : a.v_scale / Z;
  char *orow = reinterpret_cast<char *>(a.o);
  const int64_t obase = (int64_t)b * a.o_sb + (int64_t)i * a.o_sr + (int64_t)h * a.o_sh;
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    const float v = o[e] * inv;
    if (a.o_dtype == DT_F32) store_out<DT_F32>(orow, obase + lane + 64 * e, v);
    else if (a.o_dtype == DT_BF16) store_out<DT_BF16>(orow, obase + lane + 64 * e, v);
    else store_out<DT_F16>(orow, obase + lane + 64 * e, v);
  }
  if (a.lse && lane == 0) {
    const float lse = (M == kNegInf) ? kNegInf : (M + __builtin_log2f(Z)) * kLn2;
    a.lse[((int64_t)b * a.Hq + h) * a.R + i] = lse;
  }
}

// one workgroup of 4 waves per (4 rows, KV head, sequence)
template <int D>
__global__ __launch_bounds__(256) void decode_merge(DecodeArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rr = blockIdx.x * kWaves + wave, kvh = blockIdx.y, b = blockIdx.z;
  int Pl;
  int64_t base, stride;
  if (!a.sk) {
    const int T = decode_tokens(a);
    const int L = min(a.lens[b], a.capacity);
    Pl = (L + T - 1) / T;                     // live partitions
    base = (((int64_t)b * a.Hkv + kvh) * a.rows + rr) * a.P;
    stride = 1;
  } else {
    // sequence b's partitions are the head's slots qe_b .. qe_b + q_b - 1, as
    // its partition 0 recorded them (an empty sequence has none)
    const int L = min(a.lens[b], a.capacity);
    const int qe = L > 0 ? a.sk_tab[((int64_t)kvh * a.B + b) * 2] : 0;
    Pl = L > 0 ? a.sk_tab[((int64_t)kvh * a.B + b) * 2 + 1] : 0;
    base = ((int64_t)kvh * a.sk_wgs + qe) * a.sk_rbw + rr;
    stride = a.sk_rbw;
  }
  // rows past a sequence's own row count are not part of the output
  if (rr < a.rows && rr % a.R < seq_rows(a.rows_b, b, a.R))
    merge_row<D>(a, b, kvh, rr, Pl, base, stride, lane);
}

// ==================================================================================
// VALU partial kernel
// ==================================================================================
//
// Lane layout per page (16 tokens):
//   K: lane = 4*n + qq handles token n; its 16-byte chunks are (4c + qq) of the
//      token row, c < NL.  A quad holds one token; partial dot products are
//      summed over the quad with DPP.
//   V: the page's V tile [D][16] is read as 64-lane x 16-byte chunks
//      g = 64c + lane; chunk g is value row g / CPR, tokens (g % CPR) * EPC + e.
//   After the quad sum every lane knows all rows' scores of its token and
//   handles the softmax of rows r = qq + 4k.
template <int KVDT, int QDT, int D, int RB, bool VS>
__global__ __launch_bounds__(256) void decode_valu(DecodeArgs a) {
  constexpr int ELT = DtInfo<KVDT>::bytes;
  constexpr int NL = D * ELT / 64;   // 16-byte chunks per lane per page, for K and for V
  constexpr int EPC = 16 / ELT;      // elements per chunk
  constexpr int CPR = ELT;           // V chunks per value row (16 tokens * ELT bytes)
  constexpr int MR = RB / 4;         // softmax rows per lane
  constexpr int QW = (KVDT == DT_F32) ? 4 : (is8bit(KVDT) ? 8 : 4);  // Q words per K chunk
  // 8-bit V: P.V as 16-bit dot products, half the vector instructions of
  // FP32 FMAs, which bound this kernel at 8-bit K/V.  Every e4m3fn and e5m2
  // value is exact in f16 and in bf16, and the 16-bit products are exact in
  // FP32, so the only rounding added is that of the weights: to f16 with
  // per-tensor scales (2^-11 relative; the row sums use the same rounded
  // weights), to bf16 with per-vector scales, whose weight times V scale can
  // lie outside the f16 range (2^-9 relative).
  constexpr bool PV16 = is8bit(KVDT);

  // query rows of the workgroup, in the arithmetic's representation:
  // FP32 for FP32 K/V, else the 16-bit Q codes
  constexpr int QE = (KVDT == DT_F32) ? 4 : 2;
  __shared__ __attribute__((aligned(16))) char q_lds[RB * D * QE];
  __shared__ float p_lds[kWaves][PV16 ? 1 : 16][RB];
  __shared__ __attribute__((aligned(16))) uint16_t p16_lds[kWaves][PV16 ? RB : 1][16];
  __shared__ float alpha_lds[kWaves][RB];
  __shared__ float m_w[kWaves][RB];
  __shared__ float l_w[kWaves][RB];
  __shared__ float acc_lds[RB][D];

  const int lane = threadIdx.x & 63;
  const int wave = uniform_int(threadIdx.x >> 6);
  // this workgroup's tokens [t0, t1) of row block rb of (sequence b, KV head
  // kvh); partial row r of the block goes to workspace index pbase + r * pstride
  int b, kvh, rb, t0, t1;
  int64_t pbase, pstride;
  if (!a.sk) {
    // partition p: blockIdx (KV head * row blocks + row block, p, sequence)
    kvh = blockIdx.x / a.row_blocks;
    rb = blockIdx.x % a.row_blocks;
    const int p = blockIdx.y;
    b = blockIdx.z;
    const int Lb = min(a.lens[b], a.capacity);
    if (p * decode_tokens_lo(a, Lb) >= Lb) return;   // empty partition: the merge never reads it
    const int T = decode_tokens(a);
    t0 = p * T;
    if (t0 >= Lb) return;
    t1 = min(Lb, t0 + T);
    pbase = (((int64_t)b * a.Hkv + kvh) * a.rows + rb * RB) * a.P + p;
    pstride = a.P;
  } else {
    // balanced partitions (one row block): slot q / Hkv of KV head q % Hkv, in pages
    kvh = blockIdx.x % a.Hkv;
    rb = 0;
    const int slot = blockIdx.x / a.Hkv;
    SkPlan sp;
    if (!sk_plan(a, slot, sp)) return;
    int x0, x1, pp, qq;
    sk_part(sp, slot, b, pp, qq, x0, x1);
    if (pp == 0 && threadIdx.x == 0) {
      a.sk_tab[((int64_t)kvh * a.B + b) * 2] = slot;
      a.sk_tab[((int64_t)kvh * a.B + b) * 2 + 1] = qq;
    }
    const int Lb = min(a.lens[b], a.capacity);
    t0 = x0 * kPage;
    t1 = min(Lb, x1 * kPage);
    pbase = ((int64_t)kvh * a.sk_wgs + slot) * a.sk_rbw;
    pstride = 1;
  }
  const int L = min(a.lens[b], a.capacity);
  const int n = lane >> 2, qq = lane & 3;
  const int tg = lane % CPR;

  // ---- query rows of this block -> LDS ----
  for (int idx = threadIdx.x; idx < RB * D; idx += 256) {
    const int r = idx / D, d = idx % D;
    const int rr = rb * RB + r;
    const bool ok = rr < a.rows;
    const int h = kvh * a.G + (ok ? rr / a.R : 0);
    const int i = ok ? rr % a.R : 0;
    const int64_t qi = (int64_t)b * a.q_sb + (int64_t)i * a.q_sr + (int64_t)h * a.q_sh + d;
    if constexpr (KVDT == DT_F32) {
      float v;
      if constexpr (QDT == DT_F32) v = reinterpret_cast<const float *>(a.q)[qi];
      else if constexpr (QDT == DT_BF16)
        v = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(a.q)[qi] << 16);
      else v = (float)reinterpret_cast<const _Float16 *>(a.q)[qi];
      reinterpret_cast<float *>(q_lds)[idx] = ok ? v : 0.f;
    } else {
      const uint16_t v = reinterpret_cast<const uint16_t *>(a.q)[qi];
      reinterpret_cast<uint16_t *>(q_lds)[idx] = ok ? v : (uint16_t)0;
    }
  }
  __syncthreads();
  // the lane's Q words for row r and chunk c (QW 32-bit words)
  auto q_words = [&](int r, int c, uint32_t *w) {
    const int e0 = (4 * c + qq) * EPC;
    const char *src = q_lds + ((size_t)r * D + e0) * QE;
#pragma unroll
    for (int k = 0; k < QW; k += 4) {
      const u32x4 v = *reinterpret_cast<const u32x4 *>(src + 4 * k);
#pragma unroll
      for (int e = 0; e < 4; ++e) w[k + e] = v[e];
    }
  };
  // position of the rows this lane handles in the softmax: r = qq + 4k
  const int nrows = seq_rows(a.rows_b, b, a.R);   // rows of this sequence
  int pos_mine[MR];
#pragma unroll
  for (int k = 0; k < MR; ++k) {
    const int rr = rb * RB + qq + 4 * k;
    pos_mine[k] = (rr < a.rows && rr % a.R < nrows) ? L - nrows + rr % a.R : -1;
  }

  float m_run[MR], l_run[MR];
  float o[RB][NL];
#pragma unroll
  for (int k = 0; k < MR; ++k) { m_run[k] = kNegInf; l_run[k] = 0.f; }
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int c = 0; c < NL; ++c) o[r][c] = 0.f;

  const char *kbase = reinterpret_cast<const char *>(a.k) + (int64_t)kvh * a.k_sh * ELT;
  const char *vbase = reinterpret_cast<const char *>(a.v) + (int64_t)kvh * a.v_sh * ELT;
  const int32_t *pt = a.page_table + (int64_t)b * a.pt_stride;
  const int pg_end = (t1 + 15) >> 4;
  const int pg_first = (t0 >> 4) + wave;
  int pg = pg_first;

  // This wave's page ids (its k-th page is pg_first + 4k), 128 at a time,
  // loaded coalesced and broadcast per page; the next 128 are loaded when the
  // walk, which visits the pages in order, reaches them.
  int ids[2];
  int ids_k0 = 0;
  // The id loads are unconditional (indices clamped to the last page) and
  // waited for at once: a load under a branch, or one still in flight where
  // the walk's paths join, makes the compiler wait for every K/V load in
  // flight at the join (once per 128 pages here is all it costs).
  auto load_ids = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int hlf = 0; hlf < 2; ++hlf) {
      const int idx = pg_first + (k0 + 64 * hlf + lane) * kWaves;
      ids[hlf] = pt[min(idx, pg_end - 1)];
    }
    ids_k0 = k0;
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  };
  load_ids(0);
  auto page_id = [&](int page_idx) -> int64_t {
    int k = (page_idx - pg_first) / kWaves - ids_k0;
    if (k >= 128) {
      load_ids(ids_k0 + 128);
      k -= 128;
    }
    return k < 64 ? __builtin_amdgcn_readlane(ids[0], k) : __builtin_amdgcn_readlane(ids[1], k - 64);
  };

  // per-vector scales: lane n's token (the quad shares it)
  const float *ksbase = VS ? a.k_vs + (int64_t)kvh * a.vs_sh + n : nullptr;
  const float *vsbase = VS ? a.v_vs + (int64_t)kvh * a.vs_sh + n : nullptr;
  // A page past the walk's end is "loaded" through an empty buffer resource
  // (zeros, no memory access), so that the loop issues its loads
  // unconditionally and every page waits for its own loads only.
  auto load_page = [&](auto mode, int page_idx, u32x4 *kd, u32x4 *vd, float &ksd,
                       float &vsd) __attribute__((always_inline)) {
    const bool live = page_idx < pg_end;
    const int64_t pid = page_id(page_idx);
    const char *kp, *vp;
    if constexpr (decltype(mode)::value) {
      kp = page_addr(kbase, a.k_frag, a.frag_shift, pid, a.k_sp * ELT, (int64_t)kvh * a.k_sh * ELT);
      vp = page_addr(vbase, a.v_frag, a.frag_shift, pid, a.v_sp * ELT, (int64_t)kvh * a.v_sh * ELT);
    } else {
      kp = kbase + pid * a.k_sp * ELT;
      vp = vbase + pid * a.v_sp * ELT;
    }
    const uint32_t tile = live ? 16 * D * ELT : 0;   // bytes of a (page, head) tile
#pragma unroll
    for (int c = 0; c < NL; ++c) {
      // streamed once: non-temporal
      kd[c] = ld16_nt_buf(kp, n * (D * ELT) + qq * 16 + c * 64, tile);
      vd[c] = ld16_nt_buf(vp, lane * 16 + c * 1024, tile);
    }
    if constexpr (VS) {
      ksd = ksbase[pid * a.vs_sp];
      vsd = vsbase[pid * a.vs_sp];
    }
  };

  auto process_page = [&](const int pg, const u32x4 *kc, const u32x4 *vc, float ksc,
                          float vsc) __attribute__((always_inline)) {
    // ---- scores of this lane's token for all rows ----
    float s[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < NL; ++c) {
        uint32_t qw[QW];
        q_words(r, c, qw);
        if constexpr (KVDT == DT_F32) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(__uint_as_float(qw[e]),
                                                           __uint_as_float(kc[c][e]), acc);
        } else if constexpr (KVDT == DT_BF16) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = dot2_bf16(qw[e], kc[c][e], acc);
        } else if constexpr (KVDT == DT_F16) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = dot2_f16(qw[e], kc[c][e], acc);
        } else {  // 8-bit K -> 16-bit pairs of Q's type
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            uint32_t lo = e8x2_to_16<KVDT, QDT != DT_BF16, false>(kc[c][e]);
            uint32_t hi = e8x2_to_16<KVDT, QDT != DT_BF16, true>(kc[c][e]);
            if constexpr (QDT == DT_BF16) {
              acc = dot2_bf16(qw[2 * e], lo, acc);
              acc = dot2_bf16(qw[2 * e + 1], hi, acc);
            } else {
              acc = dot2_f16(qw[2 * e], lo, acc);
              acc = dot2_f16(qw[2 * e + 1], hi, acc);
            }
          }
        }
      }
      s[r] = acc;   // this lane's quarter of the dot product
    }
    // quad reduce-scatter: lane qq ends with the full score of row qq + 4k
    // (two exchange steps; no lane needs the other rows' totals)
    float mine[MR];
#pragma unroll
    for (int k = 0; k < MR; ++k) {
      const bool o1 = qq & 1, o2 = qq & 2;
      const float x0 = o1 ? s[4 * k + 1] : s[4 * k], y0 = o1 ? s[4 * k] : s[4 * k + 1];
      const float x1 = o1 ? s[4 * k + 3] : s[4 * k + 2], y1 = o1 ? s[4 * k + 2] : s[4 * k + 3];
      const float t0 = x0 + dpp<kDppQuadXor1>(y0);
      const float t1 = x1 + dpp<kDppQuadXor1>(y1);
      const float x = o2 ? t1 : t0, y = o2 ? t0 : t1;
      mine[k] = x + dpp<kDppQuadXor2>(y);
    }

    // ---- online softmax for this lane's rows ----
    const int tok = pg * 16 + n;
    const bool page_full = (pg * 16 + 16 <= t1);
    const float sc_tok = VS ? a.score_scale * ksc : a.score_scale;
    // a slot past the end may hold any scale: its weight is 0 and stays 0
    const float v_tok = (VS && tok < t1) ? vsc : 0.f;
#pragma unroll
    for (int k = 0; k < MR; ++k) {
      const float v = mine[k];
      const bool valid = tok < t1 && tok <= pos_mine[k];
      const float x = valid ? v * sc_tok : kNegInf;
      float mx = x;
      mx = __builtin_fmaxf(mx, dpp<kDppRowRor4>(mx));
      mx = __builtin_fmaxf(mx, dpp<kDppRowRor8>(mx));
      mx = max_xor32(max_xor16(mx));
      const float m_new = __builtin_fmaxf(m_run[k], mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[k] - m_use);
      float pv = fast_exp2(x - m_use);
      if constexpr (PV16 && VS) {
        p16_lds[wave][qq + 4 * k][n] = __builtin_bit_cast(uint16_t, (__bf16)(pv * v_tok));
      } else if constexpr (PV16) {
        const _Float16 ph = (_Float16)pv;
        p16_lds[wave][qq + 4 * k][n] = __builtin_bit_cast(uint16_t, ph);
        pv = (float)ph;
      } else {
        p_lds[wave][n][qq + 4 * k] = VS ? pv * v_tok : pv;
      }
      l_run[k] = l_run[k] * alpha + pv;
      m_run[k] = m_new;
      if (n == 0) alpha_lds[wave][qq + 4 * k] = alpha;
    }
    wave_lds_sync();

    // ---- O += P V for this lane's value rows and token group ----
    float al[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) al[r] = alpha_lds[wave][r];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int c = 0; c < NL; ++c) o[r][c] *= al[r];
    if constexpr (PV16) {
      // the lane's chunk is one value row over the page's 16 tokens: word i of
      // the 16-bit weights and of the converted values holds tokens 2i, 2i+1
      uint32_t pw[RB][8];
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const u32x4 w0 = *reinterpret_cast<const u32x4 *>(&p16_lds[wave][r][0]);
        const u32x4 w1 = *reinterpret_cast<const u32x4 *>(&p16_lds[wave][r][8]);
#pragma unroll
        for (int i = 0; i < 4; ++i) { pw[r][i] = w0[i]; pw[r][4 + i] = w1[i]; }
      }
      const int nv = page_full ? 16 : t1 - pg * 16;   // valid tokens of the page
#pragma unroll
      for (int c = 0; c < NL; ++c) {
        uint32_t vh[8];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          vh[2 * w] = e8x2_to_16<KVDT, !VS, false>(vc[c][w]);
          vh[2 * w + 1] = e8x2_to_16<KVDT, !VS, true>(vc[c][w]);
        }
        if (!page_full) {
          // slots past the end may hold anything, NaN included
#pragma unroll
          for (int i = 0; i < 8; ++i)
            vh[i] = 2 * i >= nv ? 0u : (2 * i + 1 >= nv ? (vh[i] & 0xffffu) : vh[i]);
        }
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
          for (int i = 0; i < 8; ++i)
            o[r][c] = VS ? dot2_bf16(pw[r][i], vh[i], o[r][c]) : dot2_f16(pw[r][i], vh[i], o[r][c]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const int t = tg * EPC + e;
        float pr[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) pr[r] = p_lds[wave][t][r];
        const bool tvalid = page_full || (pg * 16 + t < t1);
#pragma unroll
        for (int c = 0; c < NL; ++c) {
          float vv = chunk_elem<KVDT>(vc[c], e);
          vv = tvalid ? vv : 0.f;  // slots past the end may hold anything, NaN included
#pragma unroll
          for (int r = 0; r < RB; ++r) o[r][c] = __builtin_fmaf(pr[r], vv, o[r][c]);
        }
      }
    }
    wave_lds_sync();

  };

  // Two page buffers in ping-pong: while one page is processed the other's
  // loads stay in flight (no register copies, which would force a full wait).
  u32x4 kA[NL], vA[NL], kB[NL], vB[NL];
  float ksA = 1.f, vsA = 1.f, ksB = 1.f, vsB = 1.f;
  auto pages = [&](auto mode) __attribute__((always_inline)) {
    if (pg >= pg_end) return;
    load_page(mode, pg, kA, vA, ksA, vsA);
    load_page(mode, pg + kWaves, kB, vB, ksB, vsB);
    for (; pg < pg_end; pg += 2 * kWaves) {
      process_page(pg, kA, vA, ksA, vsA);
      load_page(mode, pg + 2 * kWaves, kA, vA, ksA, vsA);
      if (pg + kWaves < pg_end) process_page(pg + kWaves, kB, vB, ksB, vsB);
      load_page(mode, pg + 3 * kWaves, kB, vB, ksB, vsB);
    }
  };
  if (a.k_frag || a.v_frag) pages(Fragmented{});
  else pages(Contiguous{});

  // ---- wave totals: l over the 16 token lanes of a row, o over the token groups ----
#pragma unroll
  for (int k = 0; k < MR; ++k) {
    float l = l_run[k];
    l += dpp<kDppRowRor4>(l);
    l += dpp<kDppRowRor8>(l);
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    l_run[k] = l;
  }
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int c = 0; c < NL; ++c) {
      float v = o[r][c];
      if constexpr (CPR >= 2) v += dpp<kDppQuadXor1>(v);
      if constexpr (CPR >= 4) v += dpp<kDppQuadXor2>(v);
      o[r][c] = v;
    }
  if (n == 0) {
#pragma unroll
    for (int k = 0; k < MR; ++k) {
      m_w[wave][qq + 4 * k] = m_run[k];
      l_w[wave][qq + 4 * k] = l_run[k];
    }
  }
  __syncthreads();

  float f[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    float M;
    wave_scales<RB>(m_w, wave, r, M, f[r]);
  }
  for (int w = 0; w < kWaves; ++w) {
    if (wave == w && tg == 0) {
#pragma unroll
      for (int c = 0; c < NL; ++c) {
        const int dv = (64 * c + lane) / CPR;
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          const float v = f[r] * o[r][c];
          acc_lds[r][dv] = (w == 0) ? v : acc_lds[r][dv] + v;
        }
      }
    }
    __syncthreads();
  }

  // ---- partial write: rows of this block ----
  for (int idx = threadIdx.x; idx < RB * D; idx += 256) {
    const int r = idx / D, d = idx % D;
    const int rr = rb * RB + r;
    if (rr < a.rows) a.ws_o[(pbase + r * pstride) * D + d] = acc_lds[r][d];
  }
  if (threadIdx.x < RB) {
    const int r = threadIdx.x;
    const int rr = rb * RB + r;
    if (rr < a.rows) {
      float M = kNegInf;
      for (int w = 0; w < kWaves; ++w) M = __builtin_fmaxf(M, m_w[w][r]);
      const float Mu = (M == kNegInf) ? 0.f : M;
      float l = 0.f;
      for (int w = 0; w < kWaves; ++w) l += fast_exp2(m_w[w][r] - Mu) * l_w[w][r];
      const int64_t slot = pbase + r * pstride;
      a.ws_ml[slot * 2 + 0] = M;
      a.ws_ml[slot * 2 + 1] = l;
    }
  }
}

// ==================================================================================
// MFMA partial kernel (16..64 rows)
// ==================================================================================
//
// Per wave step: a page pair (32 tokens).  QK^T uses two 16x16x32 MFMAs per
// 32-element d chunk, `a` = 0, 1, whose A rows m = 4j + i take tokens
// 8j + 4a + i, so that after both the lane (n = row, j) holds the scores of
// the 8 consecutive tokens 8j..8j+7 - exactly the 8 key slots it supplies as
// the B operand (P^T) of the PV MFMA, whose A operand (V^T) is then a single
// 16-byte read of a token-minor V page.
template <int KVDT, int QDT>
struct MfmaT {
  static constexpr bool f16 = (KVDT == DT_F16) || (is8bit(KVDT) && QDT == DT_F16);
};

template <bool F16>
__device__ __forceinline__ f32x4 mfma16(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// d offset of the 8 elements lane group j supplies for 32-wide d chunk kc
template <int KVDT>
__device__ __forceinline__ int dchunk(int kc, int j) {
  if constexpr (is8bit(KVDT)) return 64 * (kc >> 1) + 16 * j + 8 * (kc & 1);
  else return 32 * kc + 8 * j;
}

template <int KVDT, int QDT, int D, int NB, bool VS>
__global__ __launch_bounds__(256) void decode_mfma(DecodeArgs a) {
  constexpr int ELT = DtInfo<KVDT>::bytes;
  constexpr bool F16 = MfmaT<KVDT, QDT>::f16;
  constexpr int KC = D / 32;           // 32-wide d chunks
  constexpr int MB = D / 16;           // 16-row value blocks
  constexpr int NR = 16 * NB;          // padded rows
  constexpr int KL = is8bit(KVDT) ? KC / 2 : KC;  // 16-byte K loads per `a`

  __shared__ float m_w[kWaves][NR];
  __shared__ float l_w[kWaves][NR];
  __shared__ float acc_lds[NR][D + 4];

  const int lane = threadIdx.x & 63;
  const int wave = uniform_int(threadIdx.x >> 6);
  // this workgroup's tokens [t0, t1) of (sequence b, KV head kvh), t0 a
  // multiple of 32; partial row r goes to workspace index pbase + r * pstride
  int b, kvh, t0, t1;
  int64_t pbase, pstride;
  if (!a.sk) {
    // partition p: blockIdx (KV head, p, sequence)
    kvh = blockIdx.x;
    const int p = blockIdx.y;
    b = blockIdx.z;
    const int Lb = min(a.lens[b], a.capacity);
    if (p * decode_tokens_lo(a, Lb) >= Lb) return;   // empty partition
    const int T = decode_tokens(a);
    t0 = p * T;
    if (t0 >= Lb) return;
    t1 = min(Lb, t0 + T);
    pbase = (((int64_t)b * a.Hkv + kvh) * a.rows) * a.P + p;
    pstride = a.P;
  } else {
    // balanced partitions: slot q / Hkv of KV head q % Hkv, in page pairs
    kvh = blockIdx.x % a.Hkv;
    const int slot = blockIdx.x / a.Hkv;
    SkPlan sp;
    if (!sk_plan(a, slot, sp)) return;
    int x0, x1, pp, qq;
    sk_part(sp, slot, b, pp, qq, x0, x1);
    if (pp == 0 && threadIdx.x == 0) {
      a.sk_tab[((int64_t)kvh * a.B + b) * 2] = slot;
      a.sk_tab[((int64_t)kvh * a.B + b) * 2 + 1] = qq;
    }
    const int Lb = min(a.lens[b], a.capacity);
    t0 = x0 * 32;
    t1 = min(Lb, x1 * 32);
    pbase = ((int64_t)kvh * a.sk_wgs + slot) * a.sk_rbw;
    pstride = 1;
  }
  const int L = min(a.lens[b], a.capacity);
  const int n = lane & 15, j = lane >> 4;

  // ---- Q^T fragments: B[k = d][n = row] ----
  u32x4 qf[NB][KC];
  const int nrows = seq_rows(a.rows_b, b, a.R);   // rows of this sequence
  int pos[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int rr = 16 * nb + n;
    const bool ok = rr < a.rows;
    const int h = kvh * a.G + (ok ? rr / a.R : 0);
    const int i = ok ? rr % a.R : 0;
    pos[nb] = (ok && i < nrows) ? L - nrows + i : -1;
    const char *qrow = reinterpret_cast<const char *>(a.q) +
                       ((int64_t)b * a.q_sb + (int64_t)i * a.q_sr + (int64_t)h * a.q_sh) * 2;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      u32x4 v = ld16(qrow + dchunk<KVDT>(kc, j) * 2);
      qf[nb][kc] = ok ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  f32x4 oacc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) oacc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[NB], l_run[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) { m_run[nb] = kNegInf; l_run[nb] = 0.f; }

  const char *kbase = reinterpret_cast<const char *>(a.k) + (int64_t)kvh * a.k_sh * ELT;
  const char *vbase = reinterpret_cast<const char *>(a.v) + (int64_t)kvh * a.v_sh * ELT;
  const int32_t *pt = a.page_table + (int64_t)b * a.pt_stride;
  const int pg_end = (t1 + 15) >> 4;
  const int pp_end = (t1 + 31) >> 5;
  const int pp_first = (t0 >> 5) + wave;
  int pp = pp_first;

  // Page ids of this wave's page pairs (pair k = pp_first + 4k), 64 pairs at
  // a time, loaded coalesced and broadcast per pair; the next 64 are loaded
  // when the walk, which visits the pairs in order, reaches them.
  int ids0, ids1;
  int ids_k0 = 0;
  // The id loads are unconditional (indices clamped to the last page) and
  // waited for at once: a load under a branch, or one still in flight where
  // the walk's paths join, makes the compiler wait for every K/V load in
  // flight at the join (once per 64 pairs here is all it costs).
  auto load_ids = [&](int k0) __attribute__((always_inline)) {
    const int ppi = pp_first + (k0 + lane) * kWaves;
    const int p0 = min(2 * ppi, pg_end - 1), p1 = min(2 * ppi + 1, pg_end - 1);
    ids0 = pt[p0];
    ids1 = pt[p1];
    ids_k0 = k0;
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  };
  load_ids(0);

  // K rows: A row m = n of MFMA `a` holds token 8*(n/4) + 4a + n%4 (page-pair local)
  // V rows: value row 16*mb + n, tokens 8*j .. 8*j+7 (page j/2, offset 8*(j&1))
  // Per-vector scales: the K and V scales of the lane's score tokens 8j .. 8j+7
  // (sd[0..1] K, sd[2..3] V).
  auto load_pair = [&](auto mode, int ppi, u32x4 (*kd)[KL], u32x4 *vd16, u32x2 *vd8,
                       f32x4 *sd) __attribute__((always_inline)) {
    int k = (ppi - pp_first) / kWaves - ids_k0;
    if (k >= 64) {
      load_ids(ids_k0 + 64);
      k -= 64;
    }
    const int64_t pid0 = __builtin_amdgcn_readlane(ids0, k);
    const int64_t pid1 = __builtin_amdgcn_readlane(ids1, k);
    // the pair's two page tiles of K and V (page ids are wave-uniform)
    const char *kpg0, *kpg1, *vpg0, *vpg1;
    if constexpr (decltype(mode)::value) {
      const int64_t kh = (int64_t)kvh * a.k_sh * ELT, vh = (int64_t)kvh * a.v_sh * ELT;
      kpg0 = page_addr(kbase, a.k_frag, a.frag_shift, pid0, a.k_sp * ELT, kh);
      kpg1 = page_addr(kbase, a.k_frag, a.frag_shift, pid1, a.k_sp * ELT, kh);
      vpg0 = page_addr(vbase, a.v_frag, a.frag_shift, pid0, a.v_sp * ELT, vh);
      vpg1 = page_addr(vbase, a.v_frag, a.frag_shift, pid1, a.v_sp * ELT, vh);
    } else {
      kpg0 = kbase + pid0 * a.k_sp * ELT;
      kpg1 = kbase + pid1 * a.k_sp * ELT;
      vpg0 = vbase + pid0 * a.v_sp * ELT;
      vpg1 = vbase + pid1 * a.v_sp * ELT;
    }
#pragma unroll
    for (int aa = 0; aa < 2; ++aa) {
      const int tok = 8 * (n >> 2) + 4 * aa + (n & 3);
      const char *kp = (tok < 16 ? kpg0 : kpg1) + (tok & 15) * (D * ELT);
#pragma unroll
      for (int u = 0; u < KL; ++u) {
        const int d0 = is8bit(KVDT) ? 64 * u + 16 * j : dchunk<KVDT>(u, j);
        kd[aa][u] = ld16_nt(kp + d0 * ELT);   // streamed once: non-temporal
      }
    }
    const int64_t pidv = (j >> 1) ? pid1 : pid0;
    const char *vp = ((j >> 1) ? vpg1 : vpg0) + (8 * (j & 1)) * ELT;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const char *row = vp + (int64_t)(16 * mb + n) * 16 * ELT;
      if constexpr (is8bit(KVDT)) vd8[mb] = ld8_nt(row);
      else vd16[mb] = ld16_nt(row);
    }
    if constexpr (VS) {
      const int64_t so = pidv * a.vs_sp + (int64_t)kvh * a.vs_sh + 8 * (j & 1);
      const f32x4 *kq = reinterpret_cast<const f32x4 *>(a.k_vs + so);
      const f32x4 *vq = reinterpret_cast<const f32x4 *>(a.v_vs + so);
      sd[0] = kq[0];
      sd[1] = kq[1];
      sd[2] = vq[0];
      sd[3] = vq[1];
    }
  };
  auto process_pair = [&](const int pp, const u32x4 (*kf)[KL], const u32x4 *vf16, const u32x2 *vf8,
                          const f32x4 *sd) __attribute__((always_inline)) {
    // ---- S^T = K Q^T ----
    f32x4 s[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int aa = 0; aa < 2; ++aa) s[nb][aa] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int aa = 0; aa < 2; ++aa) {
#pragma unroll
      for (int u = 0; u < KL; ++u) {
        if constexpr (is8bit(KVDT)) {
          // 16 8-bit codes -> two 8-element 16-bit fragments (chunks kc = 2u, 2u+1)
          u32x4 lo, hi;
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            const uint32_t x = kf[aa][u][w];
            const uint32_t y = kf[aa][u][w + 2];
            lo[2 * w] = e8x2_to_16<KVDT, F16, false>(x);
            lo[2 * w + 1] = e8x2_to_16<KVDT, F16, true>(x);
            hi[2 * w] = e8x2_to_16<KVDT, F16, false>(y);
            hi[2 * w + 1] = e8x2_to_16<KVDT, F16, true>(y);
          }
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            s[nb][aa] = mfma16<F16>(lo, qf[nb][2 * u], s[nb][aa]);
            s[nb][aa] = mfma16<F16>(hi, qf[nb][2 * u + 1], s[nb][aa]);
          }
        } else {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) s[nb][aa] = mfma16<F16>(kf[aa][u], qf[nb][u], s[nb][aa]);
        }
      }
    }

    // ---- online softmax: lane row 16*nb + n, tokens 8j .. 8j+7 ----
    const int tokb = pp * 32 + 8 * j;
    // score multipliers and V weights of the 8 tokens (per-vector scales); a
    // slot past the end may hold any scale: its weight is 0 and stays 0
    float sk[8], vw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sk[e] = VS ? a.score_scale * sd[e >> 2][e & 3] : a.score_scale;
      vw[e] = (VS && tokb + e < t1) ? sd[2 + (e >> 2)][e & 3] : 0.f;
    }
    u32x4 pf[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float x[8];
#pragma unroll
      for (int aa = 0; aa < 2; ++aa)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = tokb + 4 * aa + i;
          const bool valid = tok < t1 && tok <= pos[nb];
          x[4 * aa + i] = valid ? s[nb][aa][i] * sk[4 * aa + i] : kNegInf;
        }
      float mx = max3(x[0], x[1], x[2]);
      mx = max3(mx, x[3], x[4]);
      mx = max3(mx, x[5], x[6]);
      mx = __builtin_fmaxf(mx, x[7]);
      mx = max_xor32(max_xor16(mx));   // the row's 32 tokens: lanes n, n + 16, n + 32, n + 48
      const float m_new = __builtin_fmaxf(m_run[nb], mx);
      // rescale only when some row's maximum moved (otherwise the factor is 1)
      if (__builtin_amdgcn_ballot_w64(m_new > m_run[nb])) {
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run[nb] - m_use);
        l_run[nb] *= alpha;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) oacc[mb][nb] *= alpha;
        m_run[nb] = m_new;
      }
      const float m_use = (m_run[nb] == kNegInf) ? 0.f : m_run[nb];
      float pv[8], ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pv[e] = fast_exp2(x[e] - m_use);
        ps += pv[e];
      }
      l_run[nb] += ps;
      if constexpr (VS) {
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] *= vw[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pf[nb][e] = F16 ? pack_f16x2(pv[2 * e], pv[2 * e + 1]) : pack_bf16x2(pv[2 * e], pv[2 * e + 1]);
    }

    // ---- O^T += V^T P^T ----
    const bool tail = (pp * 32 + 32 > t1);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      u32x4 vfr;
      if constexpr (is8bit(KVDT)) {
        vfr[0] = e8x2_to_16<KVDT, F16, false>(vf8[mb][0]);
        vfr[1] = e8x2_to_16<KVDT, F16, true>(vf8[mb][0]);
        vfr[2] = e8x2_to_16<KVDT, F16, false>(vf8[mb][1]);
        vfr[3] = e8x2_to_16<KVDT, F16, true>(vf8[mb][1]);
      } else {
        vfr = vf16[mb];
      }
      if (tail) {  // value slots at or past the end may hold anything: zero them
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tk = tokb + 2 * e;
          uint32_t w = vfr[e];
          if (tk >= t1) w &= 0xffff0000u;
          if (tk + 1 >= t1) w &= 0x0000ffffu;
          vfr[e] = w;
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) oacc[mb][nb] = mfma16<F16>(vfr, pf[nb], oacc[mb][nb]);
    }

  };

  // two page-pair buffers in ping-pong (no register copies of in-flight loads)
  u32x4 kA[2][KL], kB[2][KL], kC[2][KL];
  u32x4 vA16[MB], vB16[MB], vC16[MB];
  u32x2 vA8[MB], vB8[MB], vC8[MB];
  f32x4 sA[4], sB[4], sC[4];
  // The steady-state loops issue every load unconditionally (the loop runs
  // only while all its pairs exist) so that the compiler can count the loads
  // in flight exactly: processing a pair waits for that pair's loads only,
  // while the later pairs' loads stay in flight.  The last pairs are handled
  // after the loop.
  constexpr int S = kWaves;
  auto pairs = [&](auto mode) __attribute__((always_inline)) {
    if constexpr (is8bit(KVDT) && NB == 2) {
      // 8-bit pairs carry half the bytes of 16-bit ones for the same
      // arithmetic: three pairs in flight per wave at 32 rows (at 64 rows
      // the third set would spill)
      if (pp + 5 * S < pp_end) {
        load_pair(mode, pp, kA, vA16, vA8, sA);
        load_pair(mode, pp + S, kB, vB16, vB8, sB);
        load_pair(mode, pp + 2 * S, kC, vC16, vC8, sC);
        do {
          process_pair(pp, kA, vA16, vA8, sA);
          load_pair(mode, pp + 3 * S, kA, vA16, vA8, sA);
          process_pair(pp + S, kB, vB16, vB8, sB);
          load_pair(mode, pp + 4 * S, kB, vB16, vB8, sB);
          process_pair(pp + 2 * S, kC, vC16, vC8, sC);
          load_pair(mode, pp + 5 * S, kC, vC16, vC8, sC);
          pp += 3 * S;
        } while (pp + 5 * S < pp_end);
      } else {
        if (pp < pp_end) load_pair(mode, pp, kA, vA16, vA8, sA);
        if (pp + S < pp_end) load_pair(mode, pp + S, kB, vB16, vB8, sB);
        if (pp + 2 * S < pp_end) load_pair(mode, pp + 2 * S, kC, vC16, vC8, sC);
      }
      // A, B, C hold pairs pp, pp + S, pp + 2S (those that exist); pairs up
      // to pp + 4S remain
      if (pp < pp_end) {
        process_pair(pp, kA, vA16, vA8, sA);
        if (pp + 3 * S < pp_end) load_pair(mode, pp + 3 * S, kA, vA16, vA8, sA);
      }
      if (pp + S < pp_end) {
        process_pair(pp + S, kB, vB16, vB8, sB);
        if (pp + 4 * S < pp_end) load_pair(mode, pp + 4 * S, kB, vB16, vB8, sB);
      }
      if (pp + 2 * S < pp_end) process_pair(pp + 2 * S, kC, vC16, vC8, sC);
      if (pp + 3 * S < pp_end) process_pair(pp + 3 * S, kA, vA16, vA8, sA);
      if (pp + 4 * S < pp_end) process_pair(pp + 4 * S, kB, vB16, vB8, sB);
    } else if constexpr (NB == 4 && D == 128) {
      // 64 rows at d 128: the accumulators and Q fragments leave room for one
      // pair in flight (a second register set spills to scratch)
      for (; pp < pp_end; pp += kWaves) {
        load_pair(mode, pp, kA, vA16, vA8, sA);
        process_pair(pp, kA, vA16, vA8, sA);
      }
    } else {
      if (pp + 3 * S < pp_end) {
        load_pair(mode, pp, kA, vA16, vA8, sA);
        load_pair(mode, pp + S, kB, vB16, vB8, sB);
        do {
          process_pair(pp, kA, vA16, vA8, sA);
          load_pair(mode, pp + 2 * S, kA, vA16, vA8, sA);
          process_pair(pp + S, kB, vB16, vB8, sB);
          load_pair(mode, pp + 3 * S, kB, vB16, vB8, sB);
          pp += 2 * S;
        } while (pp + 3 * S < pp_end);
      } else {
        if (pp < pp_end) load_pair(mode, pp, kA, vA16, vA8, sA);
        if (pp + S < pp_end) load_pair(mode, pp + S, kB, vB16, vB8, sB);
      }
      // A, B hold pairs pp, pp + S (those that exist); pairs up to pp + 2S remain
      if (pp < pp_end) {
        process_pair(pp, kA, vA16, vA8, sA);
        if (pp + 2 * S < pp_end) load_pair(mode, pp + 2 * S, kA, vA16, vA8, sA);
      }
      if (pp + S < pp_end) process_pair(pp + S, kB, vB16, vB8, sB);
      if (pp + 2 * S < pp_end) process_pair(pp + 2 * S, kA, vA16, vA8, sA);
    }
  };
  if (a.k_frag || a.v_frag) pairs(Fragmented{});
  else pairs(Contiguous{});

  // ---- wave totals ----
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float l = l_run[nb];
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    l_run[nb] = l;
  }
  if (j == 0) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      m_w[wave][16 * nb + n] = m_run[nb];
      l_w[wave][16 * nb + n] = l_run[nb];
    }
  }
  __syncthreads();
  float f[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float M;
    wave_scales<NR>(m_w, wave, 16 * nb + n, M, f[nb]);
  }
  for (int w = 0; w < kWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int d = 16 * mb + 4 * j + i, r = 16 * nb + n;
            const float v = f[nb] * oacc[mb][nb][i];
            acc_lds[r][d] = (w == 0) ? v : acc_lds[r][d] + v;
          }
    }
    __syncthreads();
  }

  for (int idx = threadIdx.x; idx < NR * D; idx += 256) {
    const int r = idx / D, d = idx % D;
    if (r < a.rows) a.ws_o[(pbase + r * pstride) * D + d] = acc_lds[r][d];
  }
  for (int r = threadIdx.x; r < NR; r += 256) {
    if (r < a.rows) {
      float M = kNegInf;
      for (int w = 0; w < kWaves; ++w) M = __builtin_fmaxf(M, m_w[w][r]);
      const float Mu = (M == kNegInf) ? 0.f : M;
      float l = 0.f;
      for (int w = 0; w < kWaves; ++w) l += fast_exp2(m_w[w][r] - Mu) * l_w[w][r];
      const int64_t slot = pbase + r * pstride;
      a.ws_ml[slot * 2 + 0] = M;
      a.ws_ml[slot * 2 + 1] = l;
    }
  }
}

// ==================================================================================
// Debug gather: K/V of one sequence through the page table, dequantised the
// way the kernels do it (8-bit codes through both the FP32 and the 16-bit
// routes; a disagreement between the two is reported as NaN), times the
// per-vector scale (VS) and then the per-tensor scale, in FP32.
// ==================================================================================
template <int KVDT, bool VS>
__global__ void debug_gather(const void *k, const void *v, int64_t k_sp, int64_t k_sh,
                             int64_t v_sp, int64_t v_sh, int Hkv, int D, float k_scale,
                             float v_scale, const float *k_vs, const float *v_vs, int64_t vs_sp,
                             int64_t vs_sh, const uint64_t *k_frag, const uint64_t *v_frag,
                             int frag_shift, const int32_t *pt, int seq_len, float *k_out,
                             float *v_out) {
  constexpr int ELT = DtInfo<KVDT>::bytes;
  const int64_t total = (int64_t)Hkv * seq_len * D;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int d = idx % D;
    const int t = (idx / D) % seq_len;
    const int g = idx / ((int64_t)D * seq_len);
    const int64_t pid = pt[t >> 4];
    // element offsets inside the (page, head) tiles, from the tiles' addresses
    const int64_t ki = (t & 15) * D + d;
    const int64_t vi = (int64_t)d * 16 + (t & 15);
    float kv[2];
    const int64_t src[2] = {ki, vi};
    char *kh = const_cast<char *>(reinterpret_cast<const char *>(k)) + (int64_t)g * k_sh * ELT;
    char *vh = const_cast<char *>(reinterpret_cast<const char *>(v)) + (int64_t)g * v_sh * ELT;
    const void *base[2] = {
        page_addr_lane(kh, k_frag, frag_shift, pid, k_sp * ELT, (int64_t)g * k_sh * ELT),
        page_addr_lane(vh, v_frag, frag_shift, pid, v_sp * ELT, (int64_t)g * v_sh * ELT)};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int64_t e = src[s];
      if constexpr (KVDT == DT_F32) {
        kv[s] = reinterpret_cast<const float *>(base[s])[e];
      } else if constexpr (KVDT == DT_BF16) {
        kv[s] = bf16_lo(reinterpret_cast<const uint16_t *>(base[s])[e]);
      } else if constexpr (KVDT == DT_F16) {
        kv[s] = f16_lo(reinterpret_cast<const uint16_t *>(base[s])[e]);
      } else {
        const uint32_t code = reinterpret_cast<const uint8_t *>(base[s])[e];
        const float a32 = e8x2_to_f32<KVDT, false>(code)[0];
        const float b16 = bf16_lo(e8x2_to_bf16x2<KVDT, false>(code));
        const float h16 = f16_lo(e8x2_to_f16x2<KVDT, false>(code));
        const bool agree = (__float_as_uint(a32) == __float_as_uint(b16)) &&
                           (__float_as_uint(a32) == __float_as_uint(h16));
        kv[s] = (agree || a32 != a32) ? a32 : __builtin_nanf("");
      }
    }
    if constexpr (VS) {
      const int64_t si = pid * vs_sp + g * vs_sh + (t & 15);
      kv[0] = kv[0] * k_vs[si];
      kv[1] = kv[1] * v_vs[si];
    }
    k_out[idx] = kv[0] * k_scale;
    v_out[idx] = kv[1] * v_scale;
  }
}

// ==================================================================================
// launchers
// ==================================================================================

bool decode_valu_supported(int kv, int qd, int D) {
  if (D != 64 && D != 128 && D != 256) return false;
  if (D == 256 && kv == DT_F32) return false;   // FP32 K/V: head_dim up to 128
  if (kv == DT_F32) return qd == DT_F32 || qd == DT_F16 || qd == DT_BF16;
  if (kv == DT_BF16) return qd == DT_BF16;
  if (kv == DT_F16) return qd == DT_F16;
  if (is8bit(kv)) return qd == DT_BF16 || qd == DT_F16;
  return false;
}

bool decode_mfma_supported(int kv, int qd, int D, int rows) {
  if (D != 64 && D != 128) return false;
  if (rows > 64) return false;
  if (kv == DT_BF16) return qd == DT_BF16;
  if (kv == DT_F16) return qd == DT_F16;
  if (is8bit(kv)) return qd == DT_BF16 || qd == DT_F16;
  return false;
}

template <int KV, int QD, int D, bool VS>
static hipError_t valu_rb(const DecodeArgs &a, hipStream_t s) {
  // KV heads of one page run side by side; the balanced split has one
  // workgroup per partial slot
  const dim3 grid = a.sk ? dim3(a.Hkv * a.sk_wgs) : dim3(a.Hkv * a.row_blocks, a.P, a.B);
  const int rb = (a.rows + a.row_blocks - 1) / a.row_blocks;
  const unsigned lds = a.sk ? (unsigned)a.sk_lds : 0u;
  if (rb <= 4) hipLaunchKernelGGL((decode_valu<KV, QD, D, 4, VS>), grid, dim3(256), lds, s, a);
  else hipLaunchKernelGGL((decode_valu<KV, QD, D, 8, VS>), grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int KV, int QD, bool VS>
static hipError_t valu_d(const DecodeArgs &a, hipStream_t s) {
  if (a.D == 64) return valu_rb<KV, QD, 64, VS>(a, s);
  if constexpr (KV != DT_F32) {
    if (a.D == 256) return valu_rb<KV, QD, 256, VS>(a, s);
  }
  return valu_rb<KV, QD, 128, VS>(a, s);
}

// 8-bit K/V: element format, Q type and per-vector scales
template <int KV>
static hipError_t valu_8(const DecodeArgs &a, hipStream_t s) {
  const bool vs = a.k_vs != nullptr;
  if (a.q_dtype == DT_BF16) return vs ? valu_d<KV, DT_BF16, true>(a, s) : valu_d<KV, DT_BF16, false>(a, s);
  return vs ? valu_d<KV, DT_F16, true>(a, s) : valu_d<KV, DT_F16, false>(a, s);
}

hipError_t launch_decode_valu(const DecodeArgs &a, hipStream_t s) {
  switch (a.kv_dtype) {
    case DT_F32:
      if (a.q_dtype == DT_F32) return valu_d<DT_F32, DT_F32, false>(a, s);
      if (a.q_dtype == DT_BF16) return valu_d<DT_F32, DT_BF16, false>(a, s);
      return valu_d<DT_F32, DT_F16, false>(a, s);
    case DT_BF16: return valu_d<DT_BF16, DT_BF16, false>(a, s);
    case DT_F16: return valu_d<DT_F16, DT_F16, false>(a, s);
    case DT_FP8: return valu_8<DT_FP8>(a, s);
    default: return valu_8<DT_BF8>(a, s);
  }
}

template <int KV, int QD, int D, bool VS>
static hipError_t mfma_nb(const DecodeArgs &a, hipStream_t s) {
  const dim3 grid = a.sk ? dim3(a.Hkv * a.sk_wgs) : dim3(a.Hkv, a.P, a.B);
  const int nb = (a.rows + 15) / 16;
  const unsigned lds = a.sk ? (unsigned)a.sk_lds : 0u;
  switch (nb) {
    case 1: hipLaunchKernelGGL((decode_mfma<KV, QD, D, 1, VS>), grid, dim3(256), lds, s, a); break;
    case 2: hipLaunchKernelGGL((decode_mfma<KV, QD, D, 2, VS>), grid, dim3(256), lds, s, a); break;
    default: hipLaunchKernelGGL((decode_mfma<KV, QD, D, 4, VS>), grid, dim3(256), lds, s, a); break;
  }
  return hipGetLastError();
}

template <int KV, int QD, bool VS>
static hipError_t mfma_d(const DecodeArgs &a, hipStream_t s) {
  return a.D == 64 ? mfma_nb<KV, QD, 64, VS>(a, s) : mfma_nb<KV, QD, 128, VS>(a, s);
}

template <int KV>
static hipError_t mfma_8(const DecodeArgs &a, hipStream_t s) {
  const bool vs = a.k_vs != nullptr;
  if (a.q_dtype == DT_BF16) return vs ? mfma_d<KV, DT_BF16, true>(a, s) : mfma_d<KV, DT_BF16, false>(a, s);
  return vs ? mfma_d<KV, DT_F16, true>(a, s) : mfma_d<KV, DT_F16, false>(a, s);
}

hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t s) {
  switch (a.kv_dtype) {
    case DT_BF16: return mfma_d<DT_BF16, DT_BF16, false>(a, s);
    case DT_F16: return mfma_d<DT_F16, DT_F16, false>(a, s);
    case DT_FP8: return mfma_8<DT_FP8>(a, s);
    default: return mfma_8<DT_BF8>(a, s);
  }
}

// ---- resident workgroups per CU of the partial kernel a launch would use ----

template <typename K>
static int occupancy_of(K kernel) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, 256, 0) != hipSuccess) n = 1;
  return n > 0 ? n : 1;
}

template <int KV, int QD, int D, bool VS>
static int valu_occ(int rows) {
  static int cache[2] = {0, 0};
  const int k = rows <= 4 ? 0 : 1;
  if (!cache[k])
    cache[k] = k == 0 ? occupancy_of(decode_valu<KV, QD, D, 4, VS>)
                      : occupancy_of(decode_valu<KV, QD, D, 8, VS>);
  return cache[k];
}

template <int KV, int QD, int D, bool VS>
static int mfma_occ(int rows) {
  static int cache[3] = {0, 0, 0};
  const int nb = (rows + 15) / 16;
  const int k = nb <= 1 ? 0 : nb == 2 ? 1 : 2;
  if (!cache[k])
    cache[k] = k == 0 ? occupancy_of(decode_mfma<KV, QD, D, 1, VS>)
             : k == 1 ? occupancy_of(decode_mfma<KV, QD, D, 2, VS>)
                      : occupancy_of(decode_mfma<KV, QD, D, 4, VS>);
  return cache[k];
}

template <int KV, int QD, bool VS>
static int occ_d(bool mfma, int D, int rows) {
  if constexpr (KV != DT_F32) {
    if (mfma) return D == 64 ? mfma_occ<KV, QD, 64, VS>(rows) : mfma_occ<KV, QD, 128, VS>(rows);
    if (D == 256) return valu_occ<KV, QD, 256, VS>(rows);
  }
  return D == 64 ? valu_occ<KV, QD, 64, VS>(rows) : valu_occ<KV, QD, 128, VS>(rows);
}

template <int KV>
static int occ_8(bool mfma, int qd, int D, int rows, bool vs) {
  if (qd == DT_BF16) return vs ? occ_d<KV, DT_BF16, true>(mfma, D, rows) : occ_d<KV, DT_BF16, false>(mfma, D, rows);
  return vs ? occ_d<KV, DT_F16, true>(mfma, D, rows) : occ_d<KV, DT_F16, false>(mfma, D, rows);
}

int decode_blocks_per_cu(bool mfma, int kv, int qd, int D, int rows, bool vs) {
  switch (kv) {
    case DT_F32:
      if (qd == DT_F32) return occ_d<DT_F32, DT_F32, false>(false, D, rows);
      if (qd == DT_BF16) return occ_d<DT_F32, DT_BF16, false>(false, D, rows);
      return occ_d<DT_F32, DT_F16, false>(false, D, rows);
    case DT_BF16: return occ_d<DT_BF16, DT_BF16, false>(mfma, D, rows);
    case DT_F16: return occ_d<DT_F16, DT_F16, false>(mfma, D, rows);
    case DT_FP8: return occ_8<DT_FP8>(mfma, qd, D, rows, vs);
    default: return occ_8<DT_BF8>(mfma, qd, D, rows, vs);
  }
}

hipError_t launch_decode_merge(const DecodeArgs &a, hipStream_t s) {
  dim3 grid((a.rows + kWaves - 1) / kWaves, a.Hkv, a.B);
  if (a.D == 64) hipLaunchKernelGGL((decode_merge<64>), grid, dim3(256), 0, s, a);
  else if (a.D == 128) hipLaunchKernelGGL((decode_merge<128>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((decode_merge<256>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---- device-resident decode workspace -------------------------------------------
// attn_paged_decode_noalloc keeps its partition partials in this file-scope
// array instead of a caller workspace, for callers that cannot allocate
// device memory.  Every device the library runs on holds its own copy until
// the process ends, and every call on a device shares it: calls that overlap
// on one device race.  The kernels never read what they did not write in the
// same call (empty partitions are not merged), so nothing needs clearing.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch_address(void **ptr) {
  void *p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_debug_gather(const void *k, const void *v, int64_t k_sp, int64_t k_sh,
                               int64_t v_sp, int64_t v_sh, int kv_dtype, int Hkv, int D,
                               float k_scale, float v_scale, const float *k_vs,
                               const float *v_vs, int64_t vs_sp, int64_t vs_sh,
                               const uint64_t *k_frag, const uint64_t *v_frag, int frag_shift,
                               const int32_t *pt_row, int seq_len, float *k_out, float *v_out,
                               hipStream_t s) {
  const int64_t total = (int64_t)Hkv * seq_len * D;
  if (total == 0) return hipSuccess;
  const int blocks = (int)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
#define PA_GATHER(DT, VS)                                                                     \
  hipLaunchKernelGGL((debug_gather<DT, VS>), dim3(blocks), dim3(256), 0, s, k, v, k_sp, k_sh, \
                     v_sp, v_sh, Hkv, D, k_scale, v_scale, k_vs, v_vs, vs_sp, vs_sh, k_frag, \
                     v_frag, frag_shift, pt_row, seq_len, k_out, v_out)
  const bool vs = k_vs != nullptr;
  switch (kv_dtype) {
    case DT_F32: PA_GATHER(DT_F32, false); break;
    case DT_F16: PA_GATHER(DT_F16, false); break;
    case DT_BF16: PA_GATHER(DT_BF16, false); break;
    case DT_FP8: if (vs) PA_GATHER(DT_FP8, true); else PA_GATHER(DT_FP8, false); break;
    default: if (vs) PA_GATHER(DT_BF8, true); else PA_GATHER(DT_BF8, false); break;
  }
#undef PA_GATHER
  return hipGetLastError();
}

}  // namespace pa
