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
