// Kernel argument blocks and launcher declarations (host <-> kernel files).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// rows of sequence b: all R, or the per-sequence count clamped to [0, R]
__device__ __forceinline__ int seq_rows(const int32_t *rows_b, int b, int R) {
  return rows_b ? min(max(rows_b[b], 0), R) : R;
}

// Everything a decode launch needs; all pointers are device pointers.
struct DecodeArgs {
  const void *q;
  int64_t q_sb, q_sr, q_sh;
  const void *k, *v;
  int64_t k_sp, k_sh, v_sp, v_sh;
  const int32_t *page_table;
  int32_t pt_stride;
  int32_t capacity;       // pt_stride * 16
  const int32_t *lens;
  int32_t B, R, Hq, Hkv, G, D;
  int32_t rows;           // G * R rows share each K/V read
  int32_t kv_dtype, q_dtype, o_dtype;
  float score_scale;      // softmax_scale * k_scale * log2(e): scores in log2 units
  float v_scale;
  const float *sinks;     // nullable [Hq]
  void *o;
  int64_t o_sb, o_sr, o_sh;
  float *lse;             // nullable [B][Hq][R]
  int32_t P;              // partitions per sequence
  int32_t T;              // tokens per partition (multiple of 128)
  int32_t row_blocks;     // VALU path: ceil(rows / rows_per_block)
  float *ws_o;            // [B][Hkv][rows][P][D]   unnormalised partial outputs
  float *ws_ml;           // [B][Hkv][rows][P][2]   partial max (log2 units) and sum
  const int32_t *rows_b;  // nullable [B]: rows of each sequence (<= R); the rest are skipped
  const float *k_vs, *v_vs;   // per-vector scales [page][head][16] (8-bit K/V), or null
  int64_t vs_sp, vs_sh;       // their page / head strides (floats)
  const uint64_t *k_frag, *v_frag;   // fragment tables (device addresses), or null
  int32_t frag_shift;                // log2(pages per fragment)
  // partition size from the batch's longest sequence (t_dyn = 1): the plan's
  // rule with that length in place of the capacity (see decode_tokens)
  int32_t t_dyn, t_target, t_min, t_cap;
  // Balanced partitions (sk = 1: at most 64 sequences, one row block; see
  // sk_plan): per KV head, sequence b of u_b units (pages for the VALU
  // kernel, page pairs for the MFMA kernel) is cut into q_b = ceil(u_b / lam)
  // equal partitions, so every partition of every sequence is at most lam
  // units.  Partition p of sequence b is the head's partial slot
  // qe_b + p, qe_b = sum_{b'<b} q_b'.  The one-dimensional grid has
  // Hkv * sk_wgs workgroups; workgroup q takes slot q / Hkv of KV head
  // q % Hkv (consecutive workgroups, dealt round-robin to the XCDs, take
  // different heads of the same pages, as in the partition grid, and the
  // empty slots come last).  Partial row r of head h's slot j is at index
  // (h * sk_wgs + j) * sk_rbw + r of ws_o (times D) and ws_ml (times 2);
  // partition 0 of each sequence also leaves (qe_b, q_b) in sk_tab[h][b] for
  // the merge.
  int32_t sk, sk_wgs, sk_cmin, sk_unit;
  int32_t sk_round;       // slots of one round of resident workgroups (per KV head)
  int32_t *sk_tab;        // [Hkv][B][2]
  int32_t sk_rbw;         // rows per block (row block size, or all rows)
  // dynamic LDS bytes of a balanced-split launch: sized so that no more than
  // the planned workgroups per CU are resident (the grid carries empty slots,
  // and a CU running two ranges at once would finish last)
  int32_t sk_lds;
};

// Tokens per partition of this call.  The plan sees only the page table's
// capacity; its rule -- T = max(t_min, ceil(len / t_target) rounded up to 128),
// at most t_cap -- is applied here to the longest sequence of the batch, and T
// is kept large enough that no sequence needs more than the P partitions the
// grid has.  With the longest sequence at the capacity this is the plan's T.
// Every lane of the calling wave must be active.
__device__ __forceinline__ int decode_tokens(const DecodeArgs &a) {
  if (!a.t_dyn) return a.T;
  // the longest sequence: up to 64 lengths with scalar loads (wave-uniform, 16
  // at a time), more with vector loads of 64 and a reduction across the wave
  int m = 0;
  if (a.B <= 64) {
    typedef const __attribute__((address_space(4))) int32_t ci32;
    const ci32 *lens = (const ci32 *)a.lens;
    int b = 0;
    for (; b + 16 <= a.B; b += 16) {
#pragma unroll
      for (int k = 0; k < 16; ++k) m = max(m, lens[b + k]);
    }
    for (; b < a.B; ++b) m = max(m, lens[b]);
  } else {
    typedef const __attribute__((address_space(1))) int32_t gi32;
    const gi32 *lens = (const gi32 *)a.lens;
    for (int b = (int)(threadIdx.x & 63); b < a.B; b += 64) m = max(m, lens[b]);
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) m = max(m, __shfl_xor(m, k));
    m = __builtin_amdgcn_readfirstlane(m);
  }
  m = min(m, a.capacity);
  const int t = max(a.t_min, ((m + a.t_target - 1) / a.t_target + 127) & ~127);
  return max(min(t, a.t_cap), ((m + a.P - 1) / a.P + 127) & ~127);
}

// A lower bound of decode_tokens from one sequence's own length (the longest
// one is at least as long): partition p of a sequence of length L is empty if
// p * decode_tokens_lo(a, L) >= L, which a workgroup can tell before the
// reduction over the batch.
__device__ __forceinline__ int decode_tokens_lo(const DecodeArgs &a, int L) {
  if (!a.t_dyn) return a.T;
  const int l = max(L, 0);
  return min(a.t_cap, max(a.t_min, ((l + a.t_target - 1) / a.t_target + 127) & ~127));
}

// Balanced partitions over at most 64 sequences, one per lane: lane b holds
// sequence b's units u (pages or page pairs; 0 past the batch), its partition
// count q = ceil(u / lam) and the exclusive prefix qe of the counts, where lam
// is the smallest partition size >= sk_cmin with sum q <= N.  N is sk_round
// (one round of resident workgroups) when the non-empty sequences are equally
// long, else sk_wgs (all the planned rounds: unequal sequences cut into
// partitions for one round leave some workgroups a partition well above the
// mean).
struct SkPlan {
  int u, q, qe;
  int total;   // sum q: the non-empty slots of each KV head
};

// Reductions over the 64 lanes with DPP within rows of 16 (quad_perm
// [1,0,3,2], [2,3,0,1], row_ror 4, 8) and permlane swaps across rows; every
// lane receives the result.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <bool MAX>
__device__ __forceinline__ int wave_ext(int v) {
  auto op = [](int x, int y) { return MAX ? max(x, y) : min(x, y); };
  v = op(v, dpp_i<0xB1>(v));
  v = op(v, dpp_i<0x4E>(v));
  v = op(v, dpp_i<0x124>(v));
  v = op(v, dpp_i<0x128>(v));
  auto r = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  v = op((int)r[0], (int)r[1]);
  r = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  return op((int)r[0], (int)r[1]);
}
// sum of values below 2^26 per lane: rows of 16 in 32 bits, the rows in 64
__device__ __forceinline__ int64_t wave_sum64(int v) {
  v += dpp_i<0xB1>(v);
  v += dpp_i<0x4E>(v);
  v += dpp_i<0x124>(v);
  v += dpp_i<0x128>(v);
  return (int64_t)__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

// smallest lam in [cmin, umax] with sum ceil(u / lam) <= N (lam = umax gives
// one partition per non-empty sequence, nonempty <= N)
__device__ __forceinline__ int sk_lam(int u, int64_t W, int umax, int nonempty, int N, int cmin) {
  const int64_t w_lo = (W + N - 1) / N;                       // sum q >= W / lam
  int lo = max(cmin, (int)(w_lo < umax ? w_lo : umax));
  int hi = umax;
  if (N > nonempty) {                                         // sum q <= W / lam + nonempty
    const int64_t w_hi = (W + (N - nonempty) - 1) / (N - nonempty);
    if (w_hi < hi) hi = (int)w_hi;
  }
  hi = max(lo, hi);
  while (lo < hi) {
    const int mid = lo + (hi - lo) / 2;
    if (wave_sum64(u > 0 ? (u + mid - 1) / mid : 0) <= N) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// Every lane of the wave must be active; B <= 64.  Returns false if slot
// `slot` is empty, as soon as it can tell.
__device__ __forceinline__ bool sk_plan(const DecodeArgs &a, int slot, SkPlan &s) {
  const int lane = threadIdx.x & 63;
  const int L = lane < a.B ? min(max(a.lens[lane], 0), a.capacity) : 0;
  s.u = (L + a.sk_unit - 1) / a.sk_unit;
  const uint64_t live = __builtin_amdgcn_ballot_w64(s.u > 0);
  const int nonempty = __builtin_popcountll(live);
  if (nonempty == 0) return false;
  const int umax = wave_ext<true>(s.u);
  const int umin = wave_ext<false>(s.u > 0 ? s.u : INT32_MAX);
  if (umax == umin) {
    // equal lengths: one round, the same number of partitions for each
    const int n = max(nonempty, a.sk_round);
    if (slot >= n) return false;
    const int q0 = n / nonempty;
    const int lam = max(a.sk_cmin, (umax + q0 - 1) / q0);
    const int qq = (umax + lam - 1) / lam;
    s.q = s.u > 0 ? qq : 0;
    s.qe = qq * __builtin_popcountll(live & ((uint64_t(1) << lane) - 1));
    s.total = qq * nonempty;
    return slot < s.total;
  }
  // unequal lengths: every planned round, finer partitions
  const int64_t W = wave_sum64(s.u);
  const int lam = sk_lam(s.u, W, umax, nonempty, a.sk_wgs, a.sk_cmin);
  s.q = s.u > 0 ? (s.u + lam - 1) / lam : 0;
  // Slots are dispatched in order, so the sequences are laid out largest
  // partition first (longest-processing-time order): the last workgroups to
  // start are the shortest, and the round ends evenly.  A sequence's
  // partitions stay consecutive; ties keep the sequence order.
  const int sz = s.q > 0 ? (s.u + s.q - 1) / s.q : 0;
  int qe = 0, total = 0;
  for (int k = 0; k < a.B; ++k) {
    const int szk = __builtin_amdgcn_readlane(sz, k);
    const int qk = __builtin_amdgcn_readlane(s.q, k);
    qe += (szk > sz || (szk == sz && k < lane)) ? qk : 0;
    total += qk;
  }
  s.qe = qe;
  s.total = total;
  return slot < s.total;
}

// Slot i < total of a KV head: sequence b, its partition p of q, units [x0, x1).
__device__ __forceinline__ void sk_part(const SkPlan &s, int i, int &b, int &p, int &q, int &x0,
                                        int &x1) {
  b = __builtin_ctzll(__builtin_amdgcn_ballot_w64(s.q > 0 && s.qe <= i && i < s.qe + s.q));
  p = i - __builtin_amdgcn_readlane(s.qe, b);
  q = __builtin_amdgcn_readlane(s.q, b);
  const int64_t u = __builtin_amdgcn_readlane(s.u, b);
  x0 = (int)(p * u / q);
  x1 = (int)((p + 1) * u / q);
}

struct PrefillArgs {
  const void *q;
  int64_t q_sb, q_sr, q_sh;
  const void *k, *v;
  int64_t k_sp, k_sh, v_sp, v_sh;
  const int32_t *page_table;
  int32_t pt_stride;
  int32_t capacity;
  const int32_t *lens;
  int32_t B, n_q, Hq, Hkv, G, D;
  int32_t kv_dtype, q_dtype, o_dtype;
  float score_scale;      // softmax_scale * k_scale * log2(e)
  float v_scale;
  const float *sinks;
  void *o;
  int64_t o_sb, o_sr, o_sh;
  float *lse;             // nullable [B][Hq][n_q]
  const uint8_t *mask;    // nullable
  int32_t mask_heads, mask_block, mask_nqb, mask_nkb;
  const int32_t *rows_b;  // nullable [B]: rows of each sequence (<= n_q); the rest are skipped
  int32_t q_tiles;        // ceil(n_q / 128)
  int32_t heads_per_wg;   // 1 or 2 query heads of one group per workgroup
  int32_t num_wg;         // total workgroups
  const float *k_vs, *v_vs;   // per-vector scales [page][head][16] (8-bit K/V), or null
  int64_t vs_sp, vs_sh;
  const uint64_t *k_frag, *v_frag;   // fragment tables (device addresses), or null
  int32_t frag_shift;
};

// K/V append: new rows [B][n_new][Hkv][D] (source strides) into the paged pool
struct AppendArgs {
  const void *k_src, *v_src;
  int32_t src_dtype;
  int64_t s_b, s_r, s_h;  // source strides (elements)
  void *k, *v;
  int64_t k_sp, k_sh, v_sp, v_sh;
  int32_t kv_dtype;
  const int32_t *page_table;
  int32_t pt_stride;
  int32_t capacity;
  const int32_t *lens;
  int32_t B, n_new, Hkv, D;
  float k_scale, v_scale;
  float *k_vs, *v_vs;         // per-vector scale pools (written), or null
  int64_t vs_sp, vs_sh;
  const uint64_t *k_frag, *v_frag;   // fragment tables (device addresses), or null
  int32_t frag_shift;
};

hipError_t launch_kv_append(const AppendArgs &a, hipStream_t s);

hipError_t launch_decode_valu(const DecodeArgs &a, hipStream_t s);
hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t s);
hipError_t launch_decode_merge(const DecodeArgs &a, hipStream_t s);
// Device address of the file-scope decode scratch array of the current device
// (kDecodeScratchBytes, 256-byte aligned); call with that device current.
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
hipError_t decode_scratch_address(void **ptr);
bool decode_mfma_supported(int kv_dtype, int q_dtype, int D, int rows);
bool decode_valu_supported(int kv_dtype, int q_dtype, int D);
// resident workgroups per CU of the partial kernel selected for these arguments
// (vs: per-vector scales)
int decode_blocks_per_cu(bool mfma, int kv_dtype, int q_dtype, int D, int rows, bool vs);

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s);
hipError_t launch_prefill_wide(const PrefillArgs &a, hipStream_t s);   // head_dim 256
// head_dim 256 multi-row verify partial (up to 64 rows per KV head)
hipError_t launch_decode_wide(const DecodeArgs &a, hipStream_t s);
bool decode_wide_supported(int kv_dtype, int q_dtype, int D, int rows);
int decode_wide_blocks_per_cu(int kv_dtype, int q_dtype, bool vs);
bool prefill_supported(int kv_dtype, int q_dtype, int D);

hipError_t launch_debug_gather(const void *k, const void *v, int64_t k_sp, int64_t k_sh,
                               int64_t v_sp, int64_t v_sh, int kv_dtype, int Hkv, int D,
                               float k_scale, float v_scale, const float *k_vs,
                               const float *v_vs, int64_t vs_sp, int64_t vs_sh,
                               const uint64_t *k_frag, const uint64_t *v_frag, int frag_shift,
                               const int32_t *pt_row, int seq_len, float *k_out, float *v_out,
                               hipStream_t s);

// read-only HBM probes (pattern 0: contiguous, 1: 4 KiB tiles in `order`)
hipError_t launch_read_probe(const void *buf, size_t bytes, int pattern, const int32_t *order,
                             uint32_t *sink, int num_cus, hipStream_t s);

}  // namespace pa
