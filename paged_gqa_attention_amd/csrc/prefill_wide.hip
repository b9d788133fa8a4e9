// Causal prefill attention (sinks, optional block mask) at head_dim 256 over
// a paged K/V cache, for gfx950: the K/V layout of models with a few wide KV
// heads (Geramy/LSE README, "K/V storage": four KV heads of 256 per layer).
//
// The head_dim 64/128 kernel keeps 32 query rows per wave; at 256 its Q
// fragments and output accumulators would need about 500 registers.  Here a
// wave owns 16 rows of one query head and uses the 16x16x32 MFMA:
//     S^T = K Q^T        (Q^T fragments: 32 VGPRs)
//     online softmax     (FP32, 8 scores per lane and tile, lazy rescaling)
//     O^T += V^T P^T     (O^T accumulators: 64 VGPRs)
// A workgroup of 8 waves owns 128 rows; 32-key K/V tiles (two pages) are
// gathered through the page table into LDS, double buffered.  K rows are
// stored so that after the two 16-key S^T blocks of a tile each lane holds
// the scores of 8 consecutive keys - exactly the 8 keys it supplies as the
// P^T operand of the P.V product - and V pages are token-minor, so neither
// P nor V is transposed.
//
// Skipped tiles, sinks, ragged rows, the block mask, 8-bit decoding with
// per-vector scales and fragment addressing behave as in the 64/128 kernel
// (Geramy/LSE releases, v0.4.14: masked key windows skipped; TokenSpeed-
// Kernel-AMD page, "Attention": sinks in the denominator; LSE README,
// FlashPrefill V2 paragraph: attention on kept blocks only).
//
// The same kernel, in its decode mode (DEC), is the multi-row verify partial
// at head_dim 256: a workgroup of up to 4 waves owns the G.R rows of one KV
// head (16 per wave) and one KV partition, so each K/V tile is read from HBM
// once for all rows (Geramy/LSE releases, v0.4.21: K/V reads shared across
// query heads and verify rows; v0.4.19/v0.4.20: partitions merged by a
// log-sum-exp merge, which the decode merge kernel does); each wave writes its
// rows' unnormalised partial output, max and sum.
#include <type_traits>

#include "attn_internal.h"
#include "common.h"

namespace pa {

namespace {

constexpr int kXcds = 8;
constexpr int kD = 256;
constexpr int kTileK = 32;     // keys per tile (two pages)
constexpr int kRowsW = 16;     // query rows per wave
template <bool DEC> constexpr int waves() { return DEC ? 4 : 8; }
constexpr int kTileQ = kRowsW * 8;       // prefill rows per workgroup
constexpr float kNegInf = -__builtin_inff();
constexpr float kLazy = 8.0f;  // rescale only when the max grows by more than 2^8

template <bool F16>
__device__ __forceinline__ f32x4 mfma16(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <bool F16>
__device__ __forceinline__ uint32_t pack16w(float a, float b) {
  return F16 ? pack_f16x2(a, b) : pack_bf16x2(a, b);
}

// LDS row of key t (0..31) of a tile: block bb = bit 2 of t, row i inside the
// block = 4 * (t >> 3) + (t & 3); block bb row i then holds key
// 8 * (i >> 2) + 4 * bb + (i & 3), so lane group g of the S^T output holds
// keys 8g .. 8g+3 (block 0) and 8g+4 .. 8g+7 (block 1).
__device__ __forceinline__ int wide_row(int t) {
  return 16 * ((t >> 2) & 1) + 4 * (t >> 3) + (t & 3);
}

}  // namespace

// Arguments of either mode: prefill (DEC false) or the decode partial.
template <bool DEC> struct WideArgs;
template <> struct WideArgs<false> { typedef PrefillArgs T; };
template <> struct WideArgs<true> { typedef DecodeArgs T; };

template <int KVDT, int QDT, bool MASK, bool VS, bool DEC>
__global__ __launch_bounds__(waves<DEC>() * 64) void attn_wide(typename WideArgs<DEC>::T a) {
  constexpr int kWaves = waves<DEC>();
  constexpr int kThreads = kWaves * 64;
  static_assert(!(DEC && MASK), "decode takes no block mask");
  constexpr int ELT = DtInfo<KVDT>::bytes;
  constexpr bool F16 = (KVDT == DT_F16) || (is8bit(KVDT) && QDT == DT_F16);
  // The 32 lanes an LDS read serves together (16 rows x 2 chunks of an MFMA
  // operand) must hit 32 distinct 16-byte chunks of the 512-byte bank window:
  // K rows are padded to 544 bytes (32 mod 512); V^T rows are unpadded and
  // chunk j of row d sits at j ^ (2 ((d / 8) mod 2)), which keeps pairs
  // (2i, 2i + 1) adjacent.
  constexpr int KSTR = kD + 16;           // K LDS row stride (16-bit elements)
  constexpr int KBUF = kTileK * KSTR;
  constexpr int VBUF = kD * kTileK;
  constexpr int CPK = kD * ELT / 16;      // 16-byte chunks per stored K row
  constexpr int KCH = kTileK * CPK;       // chunks per K tile (= per V tile)
  constexpr int KPT = KCH / kThreads;     // chunks per thread (exact)
  constexpr int EPC = 16 / ELT;           // stored elements per chunk
  constexpr int LIST = 1024;              // tiles per mask window
  static_assert(KCH % kThreads == 0, "whole chunks per thread");
  static_assert(64 % CPK == 0 || CPK % 64 == 0, "a wave's K chunks lie in one page");

  // prefill stages two tiles per barrier (two pairs of buffers); decode keeps
  // one tile per barrier, so that two of its workgroups fit per CU
  constexpr int NBUF = DEC ? 2 : 4;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[NBUF][KBUF];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[NBUF][VBUF];
  __shared__ int tile_list[MASK ? LIST : 1];
  __shared__ int list_count[MASK ? kWaves : 1];
  __shared__ __attribute__((aligned(16))) float vs_lds[2][VS ? kTileK : 4];   // per buffer parity

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 15, g = lane >> 4;

  // ---- task and the rows of this wave ----
  // prefill: (sequence, KV head) groups dealt to the XCDs, heaviest tile first;
  //   the wave owns rows q0 .. q0+15 of query head h, row at position off + row.
  // decode: one KV partition [k_lo, k_hi) of one (sequence, KV head); the wave
  //   owns rows 16 wave .. +15 of the group's G.R rows (r -> head r / R, verify
  //   row r % R at position L - n_b + r % R).
  int b, kvh, h, L, k_lo, k_hi, pos_row, wave_first_pos, wave_key_end, nt;
  bool wave_has_rows, row_ok;
  int64_t q_off;         // element offset of this lane's query row
  int qt = 0, off = 0, nq = 0, tile_last = 0, part = 0;
  if constexpr (!DEC) {
    const int x = blockIdx.x;
    const int xcd = x % kXcds, slot = x / kXcds;
    const int task_local = slot / a.G, hp = slot % a.G;
    const int gi = (task_local / a.q_tiles) * kXcds + xcd;
    qt = a.q_tiles - 1 - task_local % a.q_tiles;
    if (gi >= a.B * a.Hkv) return;
    b = gi / a.Hkv;
    kvh = gi % a.Hkv;
    h = kvh * a.G + hp;
    L = min(a.lens[b], a.capacity);
    nq = seq_rows(a.rows_b, b, a.n_q);
    if (qt * kTileQ >= nq) return;
    off = L - nq;
    const int q0 = qt * kTileQ + wave * kRowsW;
    tile_last = min(qt * kTileQ + kTileQ, nq) - 1;
    const int wave_last = min(q0 + kRowsW, nq) - 1;
    wave_has_rows = q0 < nq;
    k_lo = 0;
    k_hi = min(L, off + tile_last + 1);
    wave_key_end = wave_has_rows ? min(L, off + wave_last + 1) : 0;
    wave_first_pos = off + q0;
    const int row = q0 + nl;
    row_ok = row < nq;
    pos_row = row_ok ? off + row : -1;
    q_off = (int64_t)b * a.q_sb + (int64_t)(row_ok ? row : 0) * a.q_sr + (int64_t)h * a.q_sh;
  } else {
    kvh = blockIdx.x;
    part = blockIdx.y;
    b = blockIdx.z;
    L = min(a.lens[b], a.capacity);
    if (part * decode_tokens_lo(a, L) >= L) return;   // empty partition: never merged
    const int T = decode_tokens(a);
    k_lo = part * T;
    if (k_lo >= L) return;                     // empty partition: never merged
    k_hi = min(L, k_lo + T);
    const int nrows = seq_rows(a.rows_b, b, a.R);
    const int r = kRowsW * wave + nl;
    row_ok = r < a.rows;
    const int i = row_ok ? r % a.R : 0;
    h = kvh * a.G + (row_ok ? r / a.R : 0);
    pos_row = (row_ok && i < nrows) ? L - nrows + i : -1;
    wave_has_rows = kRowsW * wave < a.rows;
    // the wave's smallest position (rows are head-major, so any of its first R)
    wave_first_pos = L - nrows;
    wave_key_end = k_hi;
    q_off = (int64_t)b * a.q_sb + (int64_t)i * a.q_sr + (int64_t)h * a.q_sh;
  }
  const int key_end = k_hi;
  nt = key_end > k_lo ? (key_end - k_lo + kTileK - 1) / kTileK : 0;
  const int npages = (L + kPage - 1) / kPage;

  // ---- Q^T fragments: B[k = d][n = row]; lane (row nl, d 32c + 8g .. +8) ----
  u32x4 qf[kD / 32];
  {
    const bool ok = row_ok;
    const char *qrow = reinterpret_cast<const char *>(a.q) + q_off * 2;
#pragma unroll
    for (int c = 0; c < kD / 32; ++c) {
      const u32x4 v = ld16(qrow + (32 * c + 8 * g) * 2);
      qf[c] = ok ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  f32x4 oacc[kD / 16];
#pragma unroll
  for (int db = 0; db < kD / 16; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  const int32_t *pt = a.page_table + (int64_t)b * a.pt_stride;
  const int64_t k_head = (int64_t)kvh * a.k_sh * ELT, v_head = (int64_t)kvh * a.v_sh * ELT;
  const char *kbase = reinterpret_cast<const char *>(a.k) + k_head;
  const char *vbase = reinterpret_cast<const char *>(a.v) + v_head;
  const int64_t k_page_bytes = a.k_sp * ELT, v_page_bytes = a.v_sp * ELT;
  const uint8_t *mrow = nullptr;
  if constexpr (MASK) {
    const int mh = a.mask_heads != 1 ? kvh : 0;
    mrow = a.mask + ((int64_t)b * a.mask_heads + mh) * (int64_t)a.mask_nqb * a.mask_nkb;
  }

  // ---- staging: each wave's 64 consecutive chunks of a K or V tile lie in
  // one page; page bases are wave-uniform, per-thread offsets fixed ----
  int k_pg[KPT], v_pg[KPT];
  uint32_t k_goff[KPT], v_goff[KPT], k_loff[KPT], v_loff[KPT];
  int v_tok0[KPT], k_slot[KPT];
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    const int ch = tid + c * kThreads;
    const int key = ch / CPK, part = ch % CPK;
    k_slot[c] = key & 15;
    k_pg[c] = __builtin_amdgcn_readfirstlane(key >> 4);
    k_goff[c] = (uint32_t)(((key & 15) * kD + part * EPC) * ELT);
    k_loff[c] = (uint32_t)(wide_row(key) * KSTR + part * EPC);
    const int vpg = ch / (kD * ELT), cc = ch % (kD * ELT);
    const int d = cc / ELT, tg = cc % ELT;          // value row, token group
    v_pg[c] = __builtin_amdgcn_readfirstlane(vpg);
    v_goff[c] = (uint32_t)(cc * 16);
    const int vj = (16 * vpg + tg * EPC) / 8;
    v_loff[c] = (uint32_t)(d * kTileK + ((vj ^ (((d >> 3) & 1) << 1)) << 3));
    v_tok0[c] = 16 * vpg + tg * EPC;
  }

  u32x4 kreg[KPT], vreg[KPT];
  float ksr[KPT];
  float vsr = 0.f;     // V scale of key `tid` of the tile (threads < 32)
  const float *ks_head = VS ? a.k_vs + (int64_t)kvh * a.vs_sh : nullptr;
  const float *vs_head = VS ? a.v_vs + (int64_t)kvh * a.vs_sh : nullptr;
  // tile t covers keys k_lo + 32 t .. +31 (k_lo is a multiple of 32)
  const int pg_lo = k_lo / kPage;
  auto gload = [&](int t) {
    t = __builtin_amdgcn_readfirstlane(t);
    const int pid0 = pt[min(pg_lo + 2 * t, npages - 1)];
    const int pid1 = pt[min(pg_lo + 2 * t + 1, npages - 1)];
#pragma unroll
    for (int c = 0; c < KPT; ++c) {
      const int pk = __builtin_amdgcn_readfirstlane(k_pg[c] == 0 ? pid0 : pid1);
      const int pv = __builtin_amdgcn_readfirstlane(v_pg[c] == 0 ? pid0 : pid1);
      const char *kpage = page_addr(kbase, a.k_frag, a.frag_shift, pk, k_page_bytes, k_head);
      const char *vpage = page_addr(vbase, a.v_frag, a.frag_shift, pv, v_page_bytes, v_head);
      // decode streams each tile once (non-temporal); prefill tiles are
      // re-read by the other heads' workgroups through L2
      kreg[c] = DEC ? ld16_nt(kpage + k_goff[c]) : ld16(kpage + k_goff[c]);
      vreg[c] = DEC ? ld16_nt(vpage + v_goff[c]) : ld16(vpage + v_goff[c]);
      if constexpr (VS) ksr[c] = ks_head[(int64_t)pk * a.vs_sp + k_slot[c]];
    }
    if constexpr (VS) {
      if (tid < kTileK) vsr = vs_head[(int64_t)(tid < 16 ? pid0 : pid1) * a.vs_sp + (tid & 15)];
    }
  };
  auto lstore = [&](int t, int buf) {
    const int kbase_tok = k_lo + t * kTileK;
    const bool tail = kbase_tok + kTileK > L;   // V slots at or past the end: zero them
    if constexpr (VS) {
      if (tid < kTileK) vs_lds[buf & 1][tid] = vsr;
      __syncthreads();
    }
#pragma unroll
    for (int c = 0; c < KPT; ++c) {
      uint16_t *kdst = &k_lds[buf][k_loff[c]];
      uint16_t *vdst = &v_lds[buf][v_loff[c]];
      constexpr int NQ = EPC / 8;   // 16-byte LDS words per V chunk
      u32x4 vv[NQ];
      if constexpr (is8bit(KVDT) && VS) {
        u32x4 kw[2];
        const float ks = ksr[c];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const f32x2 x0 = e8x2_to_f32<KVDT, false>(kreg[c][w]);
          const f32x2 x1 = e8x2_to_f32<KVDT, true>(kreg[c][w]);
          kw[w >> 1][2 * (w & 1)] = pack16w<F16>(x0[0] * ks, x0[1] * ks);
          kw[w >> 1][2 * (w & 1) + 1] = pack16w<F16>(x1[0] * ks, x1[1] * ks);
        }
        *reinterpret_cast<u32x4 *>(kdst) = kw[0];
        *reinterpret_cast<u32x4 *>(kdst + 8) = kw[1];
#pragma unroll
        for (int w = 0; w < 4; ++w) {   // word w: tokens 4w .. 4w+3 of the page row
          const f32x2 x0 = e8x2_to_f32<KVDT, false>(vreg[c][w]);
          const f32x2 x1 = e8x2_to_f32<KVDT, true>(vreg[c][w]);
          const f32x4 sv = *reinterpret_cast<const f32x4 *>(&vs_lds[buf & 1][v_tok0[c] + 4 * w]);
          vv[w >> 1][2 * (w & 1)] = pack16w<F16>(x0[0] * sv[0], x0[1] * sv[1]);
          vv[w >> 1][2 * (w & 1) + 1] = pack16w<F16>(x1[0] * sv[2], x1[1] * sv[3]);
        }
      } else if constexpr (is8bit(KVDT)) {
        u32x4 lo, hi;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          lo[2 * w] = e8x2_to_16<KVDT, F16, false>(kreg[c][w]);
          lo[2 * w + 1] = e8x2_to_16<KVDT, F16, true>(kreg[c][w]);
          hi[2 * w] = e8x2_to_16<KVDT, F16, false>(kreg[c][w + 2]);
          hi[2 * w + 1] = e8x2_to_16<KVDT, F16, true>(kreg[c][w + 2]);
        }
        *reinterpret_cast<u32x4 *>(kdst) = lo;
        *reinterpret_cast<u32x4 *>(kdst + 8) = hi;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          vv[w >> 1][2 * (w & 1)] = e8x2_to_16<KVDT, F16, false>(vreg[c][w]);
          vv[w >> 1][2 * (w & 1) + 1] = e8x2_to_16<KVDT, F16, true>(vreg[c][w]);
        }
      } else {
        *reinterpret_cast<u32x4 *>(kdst) = kreg[c];
        vv[0] = vreg[c];
      }
      if (tail) {
        const int tok0 = kbase_tok + v_tok0[c];
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int tk = tok0 + 8 * q + 2 * e;
            uint32_t wv = vv[q][e];
            if (tk >= L) wv &= 0xffff0000u;
            if (tk + 1 >= L) wv &= 0x0000ffffu;
            vv[q][e] = wv;
          }
      }
#pragma unroll
      for (int q = 0; q < NQ; ++q) *reinterpret_cast<u32x4 *>(vdst + 8 * q) = vv[q];
    }
  };

  // ---- per-tile work of one wave ----
  const float sc = a.score_scale;
  auto compute = [&](int t, int buf) {
    const int kt0 = k_lo + t * kTileK;
    if (!wave_has_rows || kt0 >= wave_key_end) return;
    bool keep = true;
    if constexpr (MASK) {
      keep = false;
      if (pos_row >= 0) {
        const int qb = pos_row / a.mask_block, kb = kt0 / a.mask_block;
        keep = qb < a.mask_nqb && kb < a.mask_nkb && mrow[(int64_t)qb * a.mask_nkb + kb] != 0;
      }
      if (!__builtin_amdgcn_ballot_w64(keep)) return;
    }
    const uint16_t *kl = k_lds[buf];
    const uint16_t *vl = v_lds[buf];

    // S^T blocks: lane (row nl) holds keys 8g + 4bb + k, k < 4
    f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int c = 0; c < kD / 32; ++c)
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const u32x4 ka = *reinterpret_cast<const u32x4 *>(kl + (16 * bb + nl) * KSTR + 32 * c + 8 * g);
        s[bb] = mfma16<F16>(ka, qf[c], s[bb]);
      }
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = s[e >> 2][e & 3];

    const bool diag = (kt0 + kTileK - 1 > wave_first_pos) || (kt0 + kTileK > key_end);
    bool need_mask = diag;
    if constexpr (MASK) need_mask = need_mask || __builtin_amdgcn_ballot_w64(!keep) != 0;
    if (need_mask) {
      const int lim = keep ? min(pos_row, key_end - 1) : -1;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (kt0 + 8 * g + e <= lim) ? x[e] : kNegInf;
    }

    // online softmax (lazy rescaling) of row nl; its 32 keys are spread over
    // the four lane groups g (lanes nl, nl + 16, nl + 32, nl + 48)
    float mx = max3(max3(x[0], x[1], x[2]), max3(x[3], x[4], x[5]), __builtin_fmaxf(x[6], x[7]));
    mx = max_xor16(mx);
    mx = max_xor32(mx);
    const float mxs = mx * sc;
    const bool grow = mxs > m_run + kLazy;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? mxs : m_run;
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.0f;
#pragma unroll
      for (int db = 0; db < kD / 16; ++db) oacc[db] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    u32x4 pf;   // P^T fragment: keys 8g .. 8g+7 of row nl
    float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = fast_exp2(__builtin_fmaf(x[2 * e], sc, -m_use));
      const float p1 = fast_exp2(__builtin_fmaf(x[2 * e + 1], sc, -m_use));
      const uint32_t w = pack16w<F16>(p0, p1);
      pf[e] = w;
      if (e & 1) ls1 = F16 ? dot2_f16(w, 0x3C003C00u, ls1) : dot2_bf16(w, 0x3F803F80u, ls1);
      else ls0 = F16 ? dot2_f16(w, 0x3C003C00u, ls0) : dot2_bf16(w, 0x3F803F80u, ls0);
    }
    l_run += ls0 + ls1;

    // O^T[db] += V^T[16 value rows, 32 keys] P^T[32 keys, 16 rows]
#pragma unroll
    for (int db = 0; db < kD / 16; ++db) {
      const u32x4 va = *reinterpret_cast<const u32x4 *>(vl + (16 * db + nl) * kTileK + ((g ^ (((nl >> 3) & 1) << 1)) << 3));
      oacc[db] = mfma16<F16>(va, pf, oacc[db]);
    }
  };

  // ---- tile loop: prefill two tiles per barrier (tiles i, i + 1 read from one
  // buffer pair while i + 2, i + 3 are staged into the other, whose last
  // readers passed the previous barrier); decode one tile per barrier ----
  auto run_pairs = [&](auto tl, int cnt) __attribute__((always_inline)) {
    gload(tl(0));
    lstore(tl(0), 0);
    if (cnt > 1) {
      gload(tl(1));
      lstore(tl(1), 1);
    }
    __syncthreads();
    for (int i = 0; i < cnt; i += 2) {
      const int pb = i & 2;
      if (i + 2 < cnt) gload(tl(i + 2));
      compute(tl(i), pb);
      if (i + 2 < cnt) lstore(tl(i + 2), pb ^ 2);
      if (i + 3 < cnt) gload(tl(i + 3));
      if (i + 1 < cnt) compute(tl(i + 1), pb + 1);
      if (i + 3 < cnt) lstore(tl(i + 3), (pb ^ 2) + 1);
      __syncthreads();
    }
  };
  if (nt > 0) {
    if constexpr (!MASK && !DEC) {
      run_pairs([](int i) { return i; }, nt);
    } else if constexpr (!MASK) {
      gload(0);
      lstore(0, 0);
      __syncthreads();
      for (int t = 0; t < nt; ++t) {
        const int buf = t & 1;
        if (t + 1 < nt) gload(t + 1);
        compute(t, buf);
        if (t + 1 < nt) lstore(t + 1, buf ^ 1);
        __syncthreads();
      }
    } else if constexpr (MASK) {
      const int first_row = qt * kTileQ;
      const int qb_lo = max(0, off + first_row) / a.mask_block;
      const int qb_hi = max(0, off + tile_last) / a.mask_block;
      for (int w0 = 0; w0 < nt; w0 += LIST) {
        const int wn = min(LIST, nt - w0);
        int base = 0;
        for (int c0 = 0; c0 < wn; c0 += kThreads) {
          const int t = w0 + c0 + tid;
          bool kept = false;
          if (c0 + tid < wn) {
            const int kb = (t * kTileK) / a.mask_block;
            for (int qb = qb_lo; qb <= qb_hi && !kept; ++qb)
              kept = qb < a.mask_nqb && kb < a.mask_nkb && kb <= qb &&
                     mrow[(int64_t)qb * a.mask_nkb + kb] != 0;
          }
          const uint64_t bal = __builtin_amdgcn_ballot_w64(kept);
          const int below = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
          if (lane == 0) list_count[wave] = __builtin_popcountll(bal);
          __syncthreads();
          int wbase = base;
          for (int w = 0; w < wave; ++w) wbase += list_count[w];
          if (kept) tile_list[wbase + below] = t;
          int tot = 0;
          for (int w = 0; w < kWaves; ++w) tot += list_count[w];
          __syncthreads();
          base += tot;
        }
        const int cnt = base;
        if (cnt == 0) continue;
        run_pairs([&](int i) { return __builtin_amdgcn_readfirstlane(tile_list[i]); }, cnt);
      }
    }
  }

  if (!wave_has_rows) return;
  const float l = sum_xor32(sum_xor16(l_run));
  if constexpr (DEC) {
    // ---- decode: this partition's unnormalised output, max and sum ----
    if (!row_ok) return;
    const int r = kRowsW * wave + nl;
    const int64_t slot_i = (((int64_t)b * a.Hkv + kvh) * a.rows + r) * a.P + part;
    float *wo = a.ws_o + slot_i * kD;
#pragma unroll
    for (int db = 0; db < kD / 16; ++db)
      *reinterpret_cast<f32x4 *>(wo + 16 * db + 4 * g) = oacc[db];
    if (g == 0) {
      a.ws_ml[slot_i * 2 + 0] = m_run;
      a.ws_ml[slot_i * 2 + 1] = l;
    }
    return;
  } else {
  // ---- epilogue: sink, normalisation, output ----
  const int row = qt * kTileQ + wave * kRowsW + nl;
  const float sink = a.sinks ? a.sinks[h] * kLog2e : kNegInf;
  const float M = __builtin_fmaxf(m_run, sink);
  float scale_o = 0.f, lse = kNegInf;
  if (M != kNegInf) {
    const float em = fast_exp2(m_run - M);
    const float Z = l * em + fast_exp2(sink - M);
    scale_o = em * a.v_scale / Z;
    lse = (M + __builtin_log2f(Z)) * kLn2;
  }
  if (row < nq) {
    char *obase = reinterpret_cast<char *>(a.o);
    const int64_t orow = (int64_t)b * a.o_sb + (int64_t)row * a.o_sr + (int64_t)h * a.o_sh;
#pragma unroll
    for (int db = 0; db < kD / 16; ++db) {
      const int d0 = 16 * db + 4 * g;
      const float v0 = oacc[db][0] * scale_o, v1 = oacc[db][1] * scale_o;
      const float v2 = oacc[db][2] * scale_o, v3 = oacc[db][3] * scale_o;
      if (a.o_dtype == DT_BF16) {
        const u32x2 w = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
        *reinterpret_cast<u32x2 *>(obase + (orow + d0) * 2) = w;
      } else if (a.o_dtype == DT_F16) {
        const u32x2 w = {pack_f16x2(v0, v1), pack_f16x2(v2, v3)};
        *reinterpret_cast<u32x2 *>(obase + (orow + d0) * 2) = w;
      } else {
        *reinterpret_cast<f32x4 *>(obase + (orow + d0) * 4) = f32x4{v0, v1, v2, v3};
      }
    }
    if (a.lse && g == 0) a.lse[((int64_t)b * a.Hq + h) * a.n_q + row] = lse;
  }
  }
}

namespace {

template <int KV, int QD, bool VS>
hipError_t wide_m(const PrefillArgs &a, hipStream_t s) {
  constexpr int NT = waves<false>() * 64;
  if (a.mask)
    hipLaunchKernelGGL((attn_wide<KV, QD, true, VS, false>), dim3(a.num_wg), dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL((attn_wide<KV, QD, false, VS, false>), dim3(a.num_wg), dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <int KV, int QD, bool VS>
hipError_t wide_dec(const DecodeArgs &a, hipStream_t s) {
  constexpr int NT = waves<true>() * 64;
  hipLaunchKernelGGL((attn_wide<KV, QD, false, VS, true>), dim3(a.Hkv, a.P, a.B), dim3(NT), 0, s, a);
  return hipGetLastError();
}

// dtype dispatch shared by both modes: f(KV, QD, VS) as integral constants
template <int KV, typename F>
hipError_t wide_dispatch8(bool vs, int qd, F &&f) {
  using K = std::integral_constant<int, KV>;
  using QB = std::integral_constant<int, DT_BF16>;
  using QF = std::integral_constant<int, DT_F16>;
  if (qd == DT_BF16) return vs ? f(K{}, QB{}, std::true_type{}) : f(K{}, QB{}, std::false_type{});
  return vs ? f(K{}, QF{}, std::true_type{}) : f(K{}, QF{}, std::false_type{});
}

template <typename Args, typename F>
hipError_t wide_dispatch(const Args &a, F &&f) {
  using B16 = std::integral_constant<int, DT_BF16>;
  using H16 = std::integral_constant<int, DT_F16>;
  const bool vs = a.k_vs != nullptr;
  switch (a.kv_dtype) {
    case DT_BF16: return f(B16{}, B16{}, std::false_type{});
    case DT_F16: return f(H16{}, H16{}, std::false_type{});
    case DT_FP8: return wide_dispatch8<DT_FP8>(vs, a.q_dtype, f);
    default: return wide_dispatch8<DT_BF8>(vs, a.q_dtype, f);
  }
}

}  // namespace

hipError_t launch_prefill_wide(const PrefillArgs &a, hipStream_t s) {
  return wide_dispatch(a, [&](auto kv, auto qd, auto vs) {
    return wide_m<decltype(kv)::value, decltype(qd)::value, decltype(vs)::value>(a, s);
  });
}

hipError_t launch_decode_wide(const DecodeArgs &a, hipStream_t s) {
  return wide_dispatch(a, [&](auto kv, auto qd, auto vs) {
    return wide_dec<decltype(kv)::value, decltype(qd)::value, decltype(vs)::value>(a, s);
  });
}

int decode_wide_blocks_per_cu(int kv, int qd, bool vs) {
  int n = 0;
  DecodeArgs dummy{};
  dummy.kv_dtype = kv;
  dummy.q_dtype = qd;
  dummy.k_vs = vs ? reinterpret_cast<const float *>(16) : nullptr;
  wide_dispatch(dummy, [&](auto kvc, auto qdc, auto vsc) {
    constexpr int KV = decltype(kvc)::value, QD = decltype(qdc)::value;
    constexpr bool VS = decltype(vsc)::value;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_wide<KV, QD, false, VS, true>,
                                                     waves<true>() * 64, 0) != hipSuccess)
      n = 1;
    return hipSuccess;
  });
  return n > 0 ? n : 1;
}

bool decode_wide_supported(int kv, int qd, int D, int rows) {
  if (D != 256 || rows > 4 * kRowsW) return false;
  if (kv == DT_BF16) return qd == DT_BF16;
  if (kv == DT_F16) return qd == DT_F16;
  if (is8bit(kv)) return qd == DT_BF16 || qd == DT_F16;
  return false;
}

}  // namespace pa
