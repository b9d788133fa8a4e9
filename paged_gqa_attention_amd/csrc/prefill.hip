// Causal prefill attention (with optional per-head sinks and an optional
// block mask) over a paged K/V cache, for gfx950.
//
// A workgroup owns a 128-row query tile of HPW (1 or 2) query heads of one
// KV group; each wave owns 32 rows of one head.  64-key K/V tiles are
// gathered through the page table into LDS (two tiles staged per barrier,
// into one pair of buffers while the other pair is read) and shared by all
// waves.  Per wave and tile:
//     S^T = K Q^T        (32x32x16 MFMA, FP32 accumulators)
//     online softmax     (FP32, one row per lane column; the reference
//                         maximum is refreshed only when a tile's
//                         exponentials leave their bound)
//     O^T += V^T P^T     (P rounded to the MFMA operand type)
// The K rows of each 32-key block are stored in LDS in the order that makes
// every lane's 16 scores of a row exactly the 16 keys it then supplies to
// the P.V products, and V pages are token-minor, so no transposes are needed.
// 16-bit K/V at head_dim 64 and 128 (two heads per workgroup) skip the
// staging registers: each wave copies its share of a tile from global memory
// straight into LDS (K rows with XOR-swizzled 16-byte chunks, V pages as
// stored), one pair of tiles ahead of the pair being computed.
//
// Tiles wholly above a wave's diagonal are skipped (Geramy/LSE releases,
// v0.4.14: fully masked key windows skipped, the rest keep their arithmetic);
// with a block mask only tiles some row keeps are visited (FlashPrefill V2
// paragraph of the Geramy/LSE README).  Sinks are added to the softmax
// denominator at the end (TokenSpeed-Kernel-AMD page, "Attention").
//
// 8-bit K/V (e4m3fn, e5m2) is decoded to the 16-bit operand type while it is
// staged; with per-vector scales (template flag VS) each value is multiplied
// by its vector's FP32 scale on the way (Geramy/LSE README, architecture
// paragraph: FP8/BF8 operand loads staged through shared memory with decoding
// and per-vector scales), so the tile loop is the same for every format.
//
// Workgroup order: (sequence, KV head) groups are dealt to the 8 XCDs; an
// XCD runs a group's query tiles back to back, heaviest first, with the G/HPW
// workgroups of one query tile adjacent, so resident workgroups share K/V
// tiles through that XCD's L2.
#include "attn_internal.h"
#include "common.h"

namespace pa {

namespace {

constexpr int kXcds = 8;
constexpr int kTileK = 64;     // keys per tile
constexpr int kTileQ = 128;    // query rows per workgroup
constexpr float kNegInf = -__builtin_inff();
constexpr float kLazy = 8.0f;  // per-tile rule: rescale when the max grows by more than 2^8

__device__ __forceinline__ f32x16 mfma32(const u32x4 &a, const u32x4 &b, const f32x16 &c,
                                         bool f16) {
  if (f16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// LDS row of key k within a 32-key block: swap bits 2 and 3 (an involution)
__device__ __forceinline__ int kperm(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <int KVDT, int QDT>
struct Cfg {
  static constexpr bool f16 = (KVDT == DT_F16) || (is8bit(KVDT) && QDT == DT_F16);
};

template <bool F16>
__device__ __forceinline__ uint32_t pack16(float a, float b) {
  return F16 ? pack_f16x2(a, b) : pack_bf16x2(a, b);
}

// max(a, b) as a median with +inf: one instruction, where fmaxf first
// quiets both operands (two more)
__device__ __forceinline__ float max2(float a, float b) {
  return __builtin_amdgcn_fmed3f(a, b, __builtin_inff());
}

}  // namespace

template <int KVDT, int QDT, int D, int HPW, bool MASK, bool VS>
__global__ __launch_bounds__(HPW * 256) void prefill_mfma(PrefillArgs a) {
  constexpr int ELT = DtInfo<KVDT>::bytes;
  constexpr bool F16 = Cfg<KVDT, QDT>::f16;
  constexpr int NW = HPW * 4;           // waves: 4 per query head, 32 rows each
  constexpr int NT = NW * 64;           // threads
  constexpr int KS = D / 16;            // 16-wide d steps of QK^T
  constexpr int DB = D / 32;            // 32-row value blocks of PV
  constexpr int KSTR = D + 8;           // K LDS row stride (16-bit elements)
  constexpr int VSTR = kTileK + 8;      // V^T LDS row stride
  constexpr int KBUF = kTileK * KSTR;
  constexpr int VBUF = D * VSTR;
  constexpr int CPK = D * ELT / 16;     // 16-byte chunks per stored K row
  constexpr int KCH = kTileK * CPK;     // chunks per K tile (= per V tile)
  constexpr int KPT = (KCH + NT - 1) / NT;
  constexpr int EPC = 16 / ELT;         // stored elements per chunk
  constexpr int LIST = 1024;            // tiles per mask window
  // 16-bit K/V at d 64 / 128 with eight waves: tiles are copied from global
  // memory straight into LDS (no staging registers), one pair of tiles ahead
  constexpr bool DL = !is8bit(KVDT) && !VS && (D == 64 || D == 128) && NW == 8;
  constexpr int DL_RPI = 1024 / (D * 2);       // K rows per wave-wide copy (1 KiB)
  constexpr int DL_IK = 8 / DL_RPI;            // K copies per wave and tile (8 rows)
  constexpr int DL_IV = (16 * D * 2 / 2) / 1024;   // V copies per wave (half a page)

  // LDS buffers: the loop stages two tiles per barrier (two pairs of buffers)
  constexpr int NBUF = 4;
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[NBUF][KBUF];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[NBUF][VBUF];
  __shared__ int tile_list[MASK ? LIST : 1];
  // V scales of a tile, one slot per buffer parity (two tiles are staged
  // between barriers)
  __shared__ __attribute__((aligned(16))) float vs_lds[2][VS ? kTileK : 4];
  __shared__ int list_count[MASK ? NW : 1];

  // ---- task of this workgroup ----
  // Workgroups are dispatched round-robin over the XCDs (block x -> XCD x % 8).
  // Each XCD receives whole (sequence, KV head) groups and runs a group's
  // query tiles back to back, heaviest first, so the query tiles that are
  // resident together stream the same K/V tiles through that XCD's L2.
  const int wpt = a.G / HPW;  // workgroups per (query tile, group) task
  const int x = blockIdx.x;
  const int xcd = x % kXcds, slot = x / kXcds;
  const int task_local = slot / wpt, hp = slot % wpt;
  const int gi = (task_local / a.q_tiles) * kXcds + xcd;
  const int qt = a.q_tiles - 1 - task_local % a.q_tiles;
  if (gi >= a.B * a.Hkv) return;
  const int b = gi / a.Hkv, kvh = gi % a.Hkv;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = kvh * a.G + hp * HPW + (wave >> 2);
  const int q0 = qt * kTileQ + (wave & 3) * 32;  // first row of this wave
  const int L = min(a.lens[b], a.capacity);
  const int nq = seq_rows(a.rows_b, b, a.n_q);    // rows of this sequence
  if (qt * kTileQ >= nq) return;                  // the whole workgroup has no rows
  const int off = L - nq;                         // position of row i is off + i
  const int nl = lane & 31, hh = lane >> 5;
  const int npages = (L + kPage - 1) / kPage;

  const int tile_last = min(qt * kTileQ + kTileQ, nq) - 1;
  const int wave_last = min(q0 + 32, nq) - 1;
  const bool wave_has_rows = q0 < nq;
  const int key_end = min(L, off + tile_last + 1);  // keys any row of the tile can see
  const int nt = key_end > 0 ? (key_end + kTileK - 1) / kTileK : 0;
  const int wave_key_end = wave_has_rows ? min(L, off + wave_last + 1) : 0;
  const int wave_first_pos = off + q0;
  const int row = q0 + nl;
  const int pos_row = row < nq ? off + row : -1;

  // ---- Q^T fragments: B[k = d][n = row]; lane (row nl, k half hh) ----
  u32x4 qf[KS];
  {
    const bool ok = row < nq;
    const char *qrow = reinterpret_cast<const char *>(a.q) +
                       ((int64_t)b * a.q_sb + (int64_t)(ok ? row : 0) * a.q_sr +
                        (int64_t)h * a.q_sh) * 2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 v = ld16(qrow + (16 * ks + 8 * hh) * 2);
      qf[ks] = ok ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = kNegInf, l_run = 0.f;
  float neg_m = 0.f;   // exponent offset: -m_run (0 while the row has no maximum)
  float grow_at = kNegInf;   // per-tile rule: raw score above which the reference moves
  bool unset = wave_has_rows;   // some row of the wave has no maximum yet (wave-uniform)
  // bound on a lane's sum of one tile's exponentials (32 of them) before the
  // reference maximum is refreshed: every P stays below 2^16 (2^14 as FP16)
  constexpr float kTrig = F16 ? 16384.0f : 65536.0f;

  const int32_t *pt = a.page_table + (int64_t)b * a.pt_stride;
  const char *kbase = reinterpret_cast<const char *>(a.k) + (int64_t)kvh * a.k_sh * ELT;
  const char *vbase = reinterpret_cast<const char *>(a.v) + (int64_t)kvh * a.v_sh * ELT;
  const int mh = (MASK && a.mask_heads != 1) ? kvh : 0;
  const uint8_t *mrow = MASK ? a.mask + ((int64_t)b * a.mask_heads + mh) *
                                          (int64_t)a.mask_nqb * a.mask_nkb
                             : nullptr;
  // block mask: the rows of the tile span query blocks qb_lo .. qb_lo + 2 at
  // most (128 rows, blocks of at least 64); each listed K/V tile carries one
  // bit per such block (kept for that block), and a row reads the bit of its
  // own block
  const int qb_lo = MASK ? max(0, off + qt * kTileQ) / a.mask_block : 0;
  const int qb_hi = MASK ? max(0, off + tile_last) / a.mask_block : 0;
  const int rel_qb = (MASK && pos_row >= 0) ? pos_row / a.mask_block - qb_lo : 0;

  // ---- staging: global -> registers -> LDS.  The 4 page ids of a tile are
  // workgroup-uniform scalar loads.  Each wave's 64 consecutive 16-byte chunks
  // of a K or V tile lie in one page, so a load is a wave-uniform page base
  // (scalar 64-bit arithmetic) plus a per-lane offset inside the page that,
  // like the chunk's LDS position, is the same for every tile and computed
  // once here.
  static_assert(64 % CPK == 0 && 16 % (64 / CPK) == 0, "a wave's K chunks span one page");
  static_assert((D * ELT) % 64 == 0, "a wave's V chunks span one page");
  const int64_t k_page_bytes = a.k_sp * ELT, v_page_bytes = a.v_sp * ELT;
  int k_pg[KPT], v_pg[KPT];                 // page of the tile (wave-uniform)
  uint32_t k_goff[KPT], v_goff[KPT];        // byte offset inside the page tile
  uint32_t k_loff[KPT], v_loff[KPT];        // element offset inside an LDS buffer
  int v_tok0[KPT];                          // first token of the V chunk in its tile
  int k_slot[KPT];                          // slot of the K chunk's token in its page
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    const int ch = tid + c * NT;
    const int key = ch / CPK, part = ch % CPK;
    k_slot[c] = key & 15;
    k_pg[c] = __builtin_amdgcn_readfirstlane(key >> 4);
    k_goff[c] = (uint32_t)(((key & 15) * D + part * EPC) * ELT);
    k_loff[c] = (uint32_t)(((key & ~31) | kperm(key & 31)) * KSTR + part * EPC);
    const int vpg = ch / (D * ELT), cc = ch % (D * ELT);
    const int d = cc / ELT, tg = cc % ELT;          // value row, token group
    v_pg[c] = __builtin_amdgcn_readfirstlane(vpg);
    v_goff[c] = (uint32_t)(cc * 16);
    v_loff[c] = (uint32_t)(d * VSTR + 16 * vpg + tg * EPC);
    v_tok0[c] = 16 * vpg + tg * EPC;
  }

  static_assert(!VS || EPC == 16, "per-vector scales: a V chunk is one page row");
  static_assert(!VS || NT >= kTileK, "per-vector scales: one thread per key of a tile");
  u32x4 kreg[KPT], vreg[KPT];
  float ksr[KPT];           // per-vector scale of the K chunk's token
  float vsr = 0.f;          // V scale of key `tid` of the tile (threads < 64)
  const float *ks_head = VS ? a.k_vs + (int64_t)kvh * a.vs_sh : nullptr;
  const float *vs_head = VS ? a.v_vs + (int64_t)kvh * a.vs_sh : nullptr;
  auto gload = [&](int t) {
    t = __builtin_amdgcn_readfirstlane(t);
    int pid[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) pid[k] = pt[min(4 * t + k, npages - 1)];
#pragma unroll
    for (int c = 0; c < KPT; ++c) {
      const int ch = tid + c * NT;
      if (KCH % NT == 0 || ch < KCH) {
        const int kp = k_pg[c], vp = v_pg[c];
        const int pk = kp == 0 ? pid[0] : kp == 1 ? pid[1] : kp == 2 ? pid[2] : pid[3];
        const int pv = vp == 0 ? pid[0] : vp == 1 ? pid[1] : vp == 2 ? pid[2] : pid[3];
        const char *kpage = page_addr(kbase, a.k_frag, a.frag_shift,
                                      __builtin_amdgcn_readfirstlane(pk), k_page_bytes,
                                      (int64_t)kvh * a.k_sh * ELT);
        const char *vpage = page_addr(vbase, a.v_frag, a.frag_shift,
                                      __builtin_amdgcn_readfirstlane(pv), v_page_bytes,
                                      (int64_t)kvh * a.v_sh * ELT);
        kreg[c] = ld16(kpage + k_goff[c]);
        vreg[c] = ld16(vpage + v_goff[c]);
        if constexpr (VS)
          ksr[c] = ks_head[(int64_t)__builtin_amdgcn_readfirstlane(pk) * a.vs_sp + k_slot[c]];
      }
    }
    if constexpr (VS) {
      // the tile's 64 V scales, one per thread of the first wave (uniform page)
      const int k = tid >> 4;
      const int ps = k == 0 ? pid[0] : k == 1 ? pid[1] : k == 2 ? pid[2] : pid[3];
      if (tid < kTileK) vsr = vs_head[(int64_t)ps * a.vs_sp + (tid & 15)];
    }
  };
  auto lstore = [&](int t, int buf) {
    const int kbase_tok = t * kTileK;
    // V slots at or past the end may hold anything: zero them (last tile only)
    const bool tail = kbase_tok + kTileK > L;
    if constexpr (VS) {
      // V scales -> LDS.  The previous readers of this slot are past a
      // barrier; this barrier makes the new scales visible to every wave.
      if (tid < kTileK) vs_lds[buf & 1][tid] = vsr;
      __syncthreads();
    }
#pragma unroll
    for (int c = 0; c < KPT; ++c) {
      const int ch = tid + c * NT;
      if (KCH % NT == 0 || ch < KCH) {
        uint16_t *kdst = &k_lds[buf][k_loff[c]];
        uint16_t *vdst = &v_lds[buf][v_loff[c]];
        constexpr int NQ = EPC / 8;   // 16-byte LDS words per V chunk
        u32x4 vv[NQ];
        if constexpr (is8bit(KVDT) && VS) {
          // codes -> FP32, times the vector's scale, rounded once to the operand type
          u32x4 kw[2];
          const float ks = ksr[c];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const f32x2 x0 = e8x2_to_f32<KVDT, false>(kreg[c][w]);
            const f32x2 x1 = e8x2_to_f32<KVDT, true>(kreg[c][w]);
            kw[w >> 1][2 * (w & 1)] = pack16<F16>(x0[0] * ks, x0[1] * ks);
            kw[w >> 1][2 * (w & 1) + 1] = pack16<F16>(x1[0] * ks, x1[1] * ks);
          }
          *reinterpret_cast<u32x4 *>(kdst) = kw[0];
          *reinterpret_cast<u32x4 *>(kdst + 8) = kw[1];
#pragma unroll
          for (int w = 0; w < 4; ++w) {   // word w: tokens 4w .. 4w+3 of the page row
            const f32x2 x0 = e8x2_to_f32<KVDT, false>(vreg[c][w]);
            const f32x2 x1 = e8x2_to_f32<KVDT, true>(vreg[c][w]);
            const f32x4 sv = *reinterpret_cast<const f32x4 *>(&vs_lds[buf & 1][v_tok0[c] + 4 * w]);
            vv[w >> 1][2 * (w & 1)] = pack16<F16>(x0[0] * sv[0], x0[1] * sv[1]);
            vv[w >> 1][2 * (w & 1) + 1] = pack16<F16>(x1[0] * sv[2], x1[1] * sv[3]);
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
    }
  };

  // direct copies (DL): K rows of D elements, 16-byte chunk c of LDS row R at
  // slot c ^ (R & 7); wave w copies LDS rows 8w .. 8w + 7 (keys of page w / 2)
  // and half w % 2 of V page w / 2, stored as in memory (d-major, 16 tokens
  // per row).  One copy instruction writes 1 KiB of LDS, lane by lane.
  uint32_t dl_koff[DL ? DL_IK : 1], dl_voff[DL ? DL_IV : 1];
  if constexpr (DL) {
#pragma unroll
    for (int j = 0; j < DL_IK; ++j) {
      const int R = 8 * wave + j * DL_RPI + lane / (D / 8), slot = lane % (D / 8);
      const int c = slot ^ (R & 7);
      const int key = (R & ~31) | kperm(R & 31);
      dl_koff[j] = (uint32_t)((key & 15) * D * 2 + c * 16);
    }
#pragma unroll
    for (int j = 0; j < DL_IV; ++j) dl_voff[j] = (uint32_t)((wave & 1) * 16 * D + j * 1024 + lane * 16);
  }
  auto gload_dl = [&](int t, int buf) {
    if constexpr (DL) {
      t = __builtin_amdgcn_readfirstlane(t);
      const int pg = wave >> 1;
      typedef const __attribute__((address_space(4))) int32_t ci32;   // scalar load: the table is read-only here
      const int pid = ((ci32 *)pt)[min(4 * t + pg, npages - 1)];
      const char *kpage = page_addr(kbase, a.k_frag, a.frag_shift, pid, k_page_bytes,
                                    (int64_t)kvh * a.k_sh * ELT);
      const char *vpage = page_addr(vbase, a.v_frag, a.frag_shift, pid, v_page_bytes,
                                    (int64_t)kvh * a.v_sh * ELT);
      // issued as instructions the compiler does not track: it would otherwise
      // wait for these copies before every LDS read of the other buffers; the
      // loop waits for them itself before the barrier that publishes them
#pragma unroll
      for (int j = 0; j < DL_IK; ++j) {
        const uint32_t dst = __builtin_amdgcn_readfirstlane(
            (uint32_t)(uintptr_t)&k_lds[buf][(8 * wave + j * DL_RPI) * D]);
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(kpage + dl_koff[j]), "s"(dst) : "memory", "m0");
      }
#pragma unroll
      for (int j = 0; j < DL_IV; ++j) {
        const uint32_t dst = __builtin_amdgcn_readfirstlane(
            (uint32_t)(uintptr_t)&v_lds[buf][pg * 16 * D + (wave & 1) * 8 * D + j * 512]);
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(vpage + dl_voff[j]), "s"(dst) : "memory", "m0");
      }
    }
  };
  // after this wave's copies landed: V slots at or past the end are zeroed
  auto fix_tail = [&](int t, int buf) {
    if constexpr (DL) {
      const int kb0 = t * kTileK;
      if (kb0 + kTileK <= L) return;
      const int pg = wave >> 1;
      const int tok0 = kb0 + 16 * pg + 8 * (lane & 1);
#pragma unroll
      for (int j = 0; j < DL_IV; ++j) {
        uint16_t *vp = &v_lds[buf][pg * 16 * D + (wave & 1) * 8 * D + j * 512 + lane * 8];
        u32x4 v = *reinterpret_cast<u32x4 *>(vp);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t w = v[e];
          if (tok0 + 2 * e >= L) w &= 0xffff0000u;
          if (tok0 + 2 * e + 1 >= L) w &= 0x0000ffffu;
          v[e] = w;
        }
        *reinterpret_cast<u32x4 *>(vp) = v;
      }
    }
  };
  auto vm_wait = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };   // vmcnt(0)

  // ---- per-tile work of one wave ----
  const float sc = a.score_scale;
  auto compute = [&](int t, int buf, int bits) {
    const int kt0 = t * kTileK;
    if (!wave_has_rows || kt0 >= wave_key_end) return;
    bool keep = true;
    if constexpr (MASK) {
      keep = pos_row >= 0 && ((bits >> rel_qb) & 1);
      if (!__builtin_amdgcn_ballot_w64(keep)) return;
    }
    const uint16_t *kl = k_lds[buf];
    const uint16_t *vl = v_lds[buf];

    // S^T[mb]: keys 32mb + kperm(m) of the tile, rows nl
    f32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[mb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int R = 32 * mb + nl, c = 2 * ks + hh;
        const u32x4 ka = DL ? *reinterpret_cast<const u32x4 *>(kl + R * D + ((c ^ (R & 7)) * 8))
                            : *reinterpret_cast<const u32x4 *>(kl + R * KSTR + 16 * ks + 8 * hh);
        s[mb] = mfma32(ka, qf[ks], s[mb], F16);
      }
    }

    // masking only where a tile reaches past some row's position (or a row drops the tile)
    const bool diag = (kt0 + kTileK - 1 > wave_first_pos) || (kt0 + kTileK > L);
    bool need_mask = diag;
    if constexpr (MASK) need_mask = need_mask || __builtin_amdgcn_ballot_w64(!keep) != 0;
    if (need_mask) {
      // key kt0 + 8hh + c of this lane is visible when c <= rel: one compare
      // with a small constant per score
      const int rel = (keep ? min(pos_row, L - 1) : -1) - (kt0 + 8 * hh);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = 32 * mb + 16 * (i >> 3) + 4 * ((i >> 2) & 1) + (i & 3);
          s[mb][i] = c <= rel ? s[mb][i] : kNegInf;
        }
    }

    // online softmax for row nl (the two lane halves hold keys 16g' + 8hh + ...
    // of each 32-key block).  Dense tiles copied straight into LDS: the
    // exponentials use the current reference maximum; it is refreshed only
    // when this lane's sum of the tile's exponentials leaves its bound (kTrig)
    // or a row of the wave has no maximum yet: then the row maxima are taken,
    // the accumulators rescaled and the tile's exponentials recomputed.  Any
    // reference works for the result (the sum and the output carry the same
    // factor); the bound keeps P and the FP32 accumulators in range.
    u32x4 pf[2][2];   // [mb][kk]: P^T fragment, keys 32mb + 16kk + 8hh .. +8
    auto expo = [&]() {
      float la = 0.f, lb = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = fast_exp2(__builtin_fmaf(s[mb][8 * kk + 2 * e], sc, neg_m));
            const float p1 = fast_exp2(__builtin_fmaf(s[mb][8 * kk + 2 * e + 1], sc, neg_m));
            const uint32_t w = F16 ? pack_f16x2(p0, p1) : pack_bf16x2(p0, p1);
            pf[mb][kk][e] = w;
            if (e & 1) lb = F16 ? dot2_f16(w, 0x3C003C00u, lb) : dot2_bf16(w, 0x3F803F80u, lb);
            else la = F16 ? dot2_f16(w, 0x3C003C00u, la) : dot2_bf16(w, 0x3F803F80u, la);
          }
      return la + lb;
    };
    if constexpr ((MASK && D == 64) || !DL) {
      // the head_dim 64 block-mask variant and those with register staging
      // keep the maximum of every tile (fewer live registers across the
      // exponentials): the accumulators are rescaled when the scaled maximum
      // exceeds the reference by more than 2^kLazy
      float t1[10];
#pragma unroll
      for (int k = 0; k < 10; ++k) {
        const int a0 = 3 * k, a1 = 3 * k + 1, a2 = 3 * k + 2;
        t1[k] = max3(s[a0 >> 4][a0 & 15], s[a1 >> 4][a1 & 15], s[a2 >> 4][a2 & 15]);
      }
      float mx = max2(max3(max3(t1[0], t1[1], t1[2]), max3(t1[3], t1[4], t1[5]),
                           max3(t1[6], t1[7], t1[8])),
                      max3(t1[9], s[1][14], s[1][15]));
      {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
      }
      const bool grow = mx > grow_at;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? mx * sc : m_run;
        const float alpha = grow ? fast_exp2(m_run - m_new) : 1.0f;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
        l_run *= alpha;
        m_run = m_new;
        neg_m = (m_run == kNegInf) ? 0.f : -m_run;
        grow_at = (m_run + kLazy) / sc;
      }
      l_run += expo();
    } else {
    float ts = expo();
    if (unset || __builtin_amdgcn_ballot_w64(ts > kTrig)) {
      float t1[10];
#pragma unroll
      for (int k = 0; k < 10; ++k) {
        const int a0 = 3 * k, a1 = 3 * k + 1, a2 = 3 * k + 2;
        t1[k] = max3(s[a0 >> 4][a0 & 15], s[a1 >> 4][a1 & 15], s[a2 >> 4][a2 & 15]);
      }
      float mx = max2(max3(max3(t1[0], t1[1], t1[2]), max3(t1[3], t1[4], t1[5]),
                           max3(t1[6], t1[7], t1[8])),
                      max3(t1[9], s[1][14], s[1][15]));
      {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
      }
      const float m_new = __builtin_fmaxf(m_run, mx * sc);
      const float alpha = m_new == m_run ? 1.0f : fast_exp2(m_run - m_new);
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      l_run *= alpha;
      const bool moved = __builtin_amdgcn_ballot_w64(m_new != m_run) != 0;
      m_run = m_new;
      neg_m = m_run == kNegInf ? 0.f : -m_run;
      if (moved) ts = expo();
      unset = __builtin_amdgcn_ballot_w64(pos_row >= 0 && m_run == kNegInf) != 0;
    }
    l_run += ts;
    }

    // O^T[db] += V^T[32 rows, 16 keys] P^T[16 keys, 32 rows]
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x4 va = DL ? *reinterpret_cast<const u32x4 *>(vl + (2 * mb + kk) * 16 * D + (32 * db + nl) * 16 + 8 * hh)
                              : *reinterpret_cast<const u32x4 *>(vl + (32 * db + nl) * VSTR + 32 * mb + 16 * kk + 8 * hh);
          oacc[db] = mfma32(va, pf[mb][kk], oacc[db], F16);
        }
  };

  // ---- tile loop (LDS buffers as above; one barrier per two tiles) ----
  if (nt > 0) {
    if constexpr (DL && !MASK) {
      // the next pair of tiles is copied into the other pair of buffers while
      // this pair is computed; their copies have two tiles' time to land
      gload_dl(0, 0);
      if (nt > 1) gload_dl(1, 1);
      vm_wait();
      fix_tail(0, 0);
      if (nt > 1) fix_tail(1, 1);
      __syncthreads();
      for (int t = 0; t < nt; t += 2) {
        const int pb = t & 2;
        if (t + 2 < nt) gload_dl(t + 2, pb ^ 2);
        if (t + 3 < nt) gload_dl(t + 3, (pb ^ 2) + 1);
        compute(t, pb, 0);
        if (t + 1 < nt) compute(t + 1, pb + 1, 0);
        vm_wait();
        if (t + 2 < nt) fix_tail(t + 2, pb ^ 2);
        if (t + 3 < nt) fix_tail(t + 3, (pb ^ 2) + 1);
        __syncthreads();
      }
    } else if constexpr (!MASK) {
      // two tiles per barrier: tiles t, t + 1 in buffer pair (t & 2), while
      // t + 2, t + 3 are staged into the other pair, whose last readers
      // passed the previous barrier (about 2% over one tile per barrier)
      gload(0);
      lstore(0, 0);
      if (nt > 1) {
        gload(1);
        lstore(1, 1);
      }
      __syncthreads();
      for (int t = 0; t < nt; t += 2) {
        const int pb = t & 2;
        if (t + 2 < nt) gload(t + 2);
        compute(t, pb, 0);
        if (t + 2 < nt) lstore(t + 2, pb ^ 2);
        if (t + 3 < nt) gload(t + 3);
        if (t + 1 < nt) compute(t + 1, pb + 1, 0);
        if (t + 3 < nt) lstore(t + 3, (pb ^ 2) + 1);
        __syncthreads();
      }
    } else {
      for (int w0 = 0; w0 < nt; w0 += LIST) {
        const int wn = min(LIST, nt - w0);
        // compact list of tiles in [w0, w0 + wn) that some row of the tile
        // keeps, each entry t | (bits << 24), bit j: kept for block qb_lo + j
        int base = 0;
        for (int c0 = 0; c0 < wn; c0 += NT) {
          const int t = w0 + c0 + tid;
          int bits = 0;
          if (c0 + tid < wn) {
            const int kb = (t * kTileK) / a.mask_block;
            for (int qb = qb_lo; qb <= qb_hi; ++qb)
              if (qb < a.mask_nqb && kb < a.mask_nkb && kb <= qb &&
                  mrow[(int64_t)qb * a.mask_nkb + kb] != 0)
                bits |= 1 << (qb - qb_lo);
          }
          const bool kept = bits != 0;
          const uint64_t bal = __builtin_amdgcn_ballot_w64(kept);
          const int below = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
          if (lane == 0) list_count[wave] = __builtin_popcountll(bal);
          __syncthreads();
          int wbase = base;
          for (int w = 0; w < wave; ++w) wbase += list_count[w];
          if (kept) tile_list[wbase + below] = t | (bits << 24);
          int tot = 0;
          for (int w = 0; w < NW; ++w) tot += list_count[w];
          __syncthreads();
          base += tot;
        }
        const int cnt = base;
        if (cnt == 0) continue;
        // the listed tiles, two per barrier as in the unmasked loop
        auto tl = [&](int i) { return __builtin_amdgcn_readfirstlane(tile_list[i]) & 0xffffff; };
        auto tb = [&](int i) { return __builtin_amdgcn_readfirstlane(tile_list[i]) >> 24; };
        if constexpr (DL) {
          gload_dl(tl(0), 0);
          if (cnt > 1) gload_dl(tl(1), 1);
          vm_wait();
          fix_tail(tl(0), 0);
          if (cnt > 1) fix_tail(tl(1), 1);
          __syncthreads();
          for (int idx = 0; idx < cnt; idx += 2) {
            const int pb = idx & 2;
            if (idx + 2 < cnt) gload_dl(tl(idx + 2), pb ^ 2);
            if (idx + 3 < cnt) gload_dl(tl(idx + 3), (pb ^ 2) + 1);
            compute(tl(idx), pb, tb(idx));
            if (idx + 1 < cnt) compute(tl(idx + 1), pb + 1, tb(idx + 1));
            vm_wait();
            if (idx + 2 < cnt) fix_tail(tl(idx + 2), pb ^ 2);
            if (idx + 3 < cnt) fix_tail(tl(idx + 3), (pb ^ 2) + 1);
            __syncthreads();
          }
          continue;
        }
        gload(tl(0));
        lstore(tl(0), 0);
        if (cnt > 1) {
          gload(tl(1));
          lstore(tl(1), 1);
        }
        __syncthreads();
        for (int idx = 0; idx < cnt; idx += 2) {
          const int pb = idx & 2;
          if (idx + 2 < cnt) gload(tl(idx + 2));
          compute(tl(idx), pb, tb(idx));
          if (idx + 2 < cnt) lstore(tl(idx + 2), pb ^ 2);
          if (idx + 3 < cnt) gload(tl(idx + 3));
          if (idx + 1 < cnt) compute(tl(idx + 1), pb + 1, tb(idx + 1));
          if (idx + 3 < cnt) lstore(tl(idx + 3), (pb ^ 2) + 1);
          __syncthreads();
        }
      }
    }
  }

  // ---- epilogue: sink, normalisation, output ----
  if (!wave_has_rows) return;
  const float sink = a.sinks ? a.sinks[h] * kLog2e : kNegInf;
  const float l = sum_xor32(l_run);
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
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * hh;
        const float v0 = oacc[db][4 * g + 0] * scale_o;
        const float v1 = oacc[db][4 * g + 1] * scale_o;
        const float v2 = oacc[db][4 * g + 2] * scale_o;
        const float v3 = oacc[db][4 * g + 3] * scale_o;
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
    if (a.lse && hh == 0) a.lse[((int64_t)b * a.Hq + h) * a.n_q + row] = lse;
  }
}

bool prefill_supported(int kv, int qd, int D) {
  if (D != 64 && D != 128 && D != 256) return false;
  if (kv == DT_BF16) return qd == DT_BF16;
  if (kv == DT_F16) return qd == DT_F16;
  if (is8bit(kv)) return qd == DT_BF16 || qd == DT_F16;
  return false;
}

template <int KV, int QD, int D, int HPW, bool VS>
static hipError_t prefill_m(const PrefillArgs &a, hipStream_t s) {
  if (a.mask)
    hipLaunchKernelGGL((prefill_mfma<KV, QD, D, HPW, true, VS>), dim3(a.num_wg), dim3(HPW * 256), 0, s, a);
  else
    hipLaunchKernelGGL((prefill_mfma<KV, QD, D, HPW, false, VS>), dim3(a.num_wg), dim3(HPW * 256), 0, s, a);
  return hipGetLastError();
}

template <int KV, int QD, int D, bool VS>
static hipError_t prefill_h(const PrefillArgs &a, hipStream_t s) {
  return a.heads_per_wg == 2 ? prefill_m<KV, QD, D, 2, VS>(a, s) : prefill_m<KV, QD, D, 1, VS>(a, s);
}

template <int KV, int QD, bool VS>
static hipError_t prefill_d(const PrefillArgs &a, hipStream_t s) {
  return a.D == 64 ? prefill_h<KV, QD, 64, VS>(a, s) : prefill_h<KV, QD, 128, VS>(a, s);
}

template <int KV>
static hipError_t prefill_8(const PrefillArgs &a, hipStream_t s) {
  const bool vs = a.k_vs != nullptr;
  if (a.q_dtype == DT_BF16) return vs ? prefill_d<KV, DT_BF16, true>(a, s) : prefill_d<KV, DT_BF16, false>(a, s);
  return vs ? prefill_d<KV, DT_F16, true>(a, s) : prefill_d<KV, DT_F16, false>(a, s);
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s) {
  if (a.D == 256) return launch_prefill_wide(a, s);
  switch (a.kv_dtype) {
    case DT_BF16: return prefill_d<DT_BF16, DT_BF16, false>(a, s);
    case DT_F16: return prefill_d<DT_F16, DT_F16, false>(a, s);
    case DT_FP8: return prefill_8<DT_FP8>(a, s);
    default: return prefill_8<DT_BF8>(a, s);
  }
}

}  // namespace pa
