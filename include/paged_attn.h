/*
 * paged_attn.h - C ABI of the gfx950 (MI355X) paged grouped-query attention
 * library (libpaged_attn.so).
 *
 * Three attention operations, each defined by scaled dot-product attention
 * over a paged K/V cache with FP32 accumulation and FP32 softmax state, and
 * the K/V append that fills the cache (attn_kv_append, below):
 *
 *   attn_paged_decode        decode / speculative verify: 1-8 query rows per
 *                            sequence, K/V split into partitions and merged
 *                            with a log-sum-exp merge (Geramy/LSE releases,
 *                            v0.4.19 "Long-context split attention" and v0.4.20
 *                            "automatic split attention"; K/V reads shared by
 *                            the query heads and rows of a group, v0.4.21
 *                            "joint decode attention").
 *   attn_prefill             causal prefill with optional per-head attention
 *                            sinks (TokenSpeed-Kernel-AMD page, "Attention":
 *                            full causal attention with attention sinks).
 *   attn_prefill_blocksparse causal prefill restricted to the key blocks a
 *                            caller-supplied block mask keeps (Geramy/LSE
 *                            README, FlashPrefill V2 paragraph: attention runs
 *                            on selected blocks only; the selection rule is
 *                            the caller's).
 *
 * Semantics (identical for all three).  For sequence b with L = seq_lens[b]
 * keys and n = q_rows query rows, row i sits at absolute position
 * p = L - n + i and attends to keys j with j <= p (and, for the block-sparse
 * call, mask[b][mh][p / mask_block][j / mask_block] != 0).  Query head h reads
 * KV head h / (num_q_heads / num_kv_heads).  With s_j = softmax_scale * q.k_j
 * (k_j, v_j dequantised: code value * k_scale, code value * v_scale, each
 * also times its (token, head) vector's scale where the cache has per-vector
 * scales):
 *     m = max(max_j s_j, sink_h),  Z = sum_j e^{s_j - m} + e^{sink_h - m},
 *     o = sum_j e^{s_j - m} v_j / Z,  lse = m + ln Z.
 * No sink means sink_h = -inf.  A row with no allowed key gets o = 0 and
 * lse = sink_h (-inf without sinks).
 * Ragged rows: with attn_opts.rows_per_seq, sequence b has only its first
 * n_b = rows_per_seq[b] rows (n = n_b above, so they sit at its last n_b
 * positions); the O and lse entries of its rows n_b .. q_rows-1 are left
 * untouched.
 *
 * Memory layout (all device memory, element strides):
 *   K pool   tile (page, kv_head) at k_pages + page*k_stride_page +
 *            head*k_stride_head, laid out [page_size][head_dim] (token-major).
 *   V pool   tile at v_pages + page*v_stride_page + head*v_stride_head, laid
 *            out [head_dim][page_size] (token-minor), so the tokens of one
 *            value component are contiguous.
 *   page_table  int32 [batch][page_table_stride]; entry k of row b is the page
 *            holding tokens 16k..16k+15 of sequence b.  Entries at or past
 *            ceil(seq_lens[b]/16) are never read.
 *   seq_lens int32 [batch]; keys in the cache for each sequence, including the
 *            rows of this call.  Values above page_table_stride*page_size are
 *            clamped to it.
 *   Q, O     [batch][q_rows][num_q_heads][head_dim] through the given strides,
 *            head_dim contiguous.
 *   lse      optional float [batch][num_q_heads][q_rows] (natural log).
 *   fragments (optional): the K and/or V pool split into fragments of
 *            2^fragment_pages_log2 pages (Geramy/LSE releases, v0.4.20 "K/V
 *            memory management": K/V kept in 256 KiB fragments of shared
 *            256 MiB arenas, grown without moving existing data).  With
 *            k_fragments set, page p's tile (page, kv_head) is at
 *            k_fragments[p >> fragment_pages_log2] + (p & (2^log2 - 1)) *
 *            k_stride_page + head*k_stride_head (elements of the K dtype from
 *            that device address); k_pages is then ignored.  Likewise
 *            v_fragments for V.  Fragment addresses are device data (trusted),
 *            16-byte aligned.  The per-vector scale pools stay unfragmented.
 *   per-vector scales (optional, 8-bit K/V): float scale of slot t of tile
 *            (page, kv_head) at k_vscales + page*vscale_stride_page +
 *            head*vscale_stride_head + t (likewise v_vscales), the 16 slots
 *            of a tile contiguous (Geramy/LSE README, "K/V storage": fp8 and
 *            bf8 caches keep an FP32 scale per K and per V vector, 33,280
 *            bytes per token in its table; the architecture paragraph: FP8/BF8
 *            loads are decoded with per-vector scales).
 *   block_mask  uint8 [batch][mask_heads][mask_q_blocks][mask_k_blocks];
 *            entries outside that extent count as 0.
 *
 * Ownership and threading: the caller owns every buffer.  The library never
 * allocates or frees device memory and never synchronises: each call only
 * enqueues work on `hip_stream` (NULL = the null stream) and returns; buffers
 * must stay valid until the stream reaches that point.  A decode workspace
 * must not be shared by calls in flight at the same time.  An attn_ctx is
 * immutable after attn_open and may be used from several host threads.
 *
 * Errors: every call returns an attn_status.  On failure, if `err` is not
 * NULL, *err receives a message the caller releases with attn_free().
 *   ATTN_ERR_INVALID_ARGUMENT  null pointers, inconsistent shapes or strides,
 *                              num_q_heads % num_kv_heads != 0, misaligned
 *                              base pointers or strides (16 bytes), q_rows
 *                              outside [1, 8] for decode, a block mask passed
 *                              to a call that does not take one (or missing
 *                              where required), bad mask geometry.
 *   ATTN_ERR_UNSUPPORTED       a well-formed request this build does not
 *                              implement (head_dim not 64, 128 or 256 --
 *                              256 with 16-bit or 8-bit K/V only --,
 *                              page_size not 16, unsupported dtype
 *                              combination, page_table_stride * 16 above
 *                              2^30 tokens).
 *   ATTN_ERR_WORKSPACE_TOO_SMALL  decode workspace below the queried size.
 *   ATTN_ERR_DEVICE            no usable gfx950 device, or a HIP error while
 *                              enqueuing (its text in *err).
 * Device-side data (page ids, seq_lens, mask bytes) is trusted: page ids must
 * lie in [0, num_pages).
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 5

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARGUMENT = 1,
  ATTN_ERR_UNSUPPORTED = 2,
  ATTN_ERR_WORKSPACE_TOO_SMALL = 3,
  ATTN_ERR_DEVICE = 4
} attn_status;

/* Storage / compute types.  FP8 is OCP e4m3fn (bias 7, max 448, no inf); BF8 is
 * OCP e5m2 (bias 15, max 57344, IEEE infinities and NaNs): the cache formats
 * "fp8" and "bf8" of the Geramy/LSE README ("K/V storage"). */
typedef enum {
  ATTN_F32 = 0, ATTN_F16 = 1, ATTN_BF16 = 2, ATTN_FP8_E4M3 = 3, ATTN_BF8_E5M2 = 4
} attn_dtype;

typedef struct attn_ctx attn_ctx;

/* Paged K/V cache of one layer. */
typedef struct {
  const void *k_pages;          /* K tiles [page_size][head_dim] */
  const void *v_pages;          /* V tiles [head_dim][page_size] */
  int32_t dtype;                /* attn_dtype of K and V */
  int32_t num_pages;            /* pages in the pool */
  int32_t page_size;            /* tokens per page; must be 16 */
  int32_t num_kv_heads;
  int32_t head_dim;             /* 64, 128, or 256 (256: 16-bit or 8-bit K/V) */
  int32_t pad0;
  int64_t k_stride_page, k_stride_head;   /* elements */
  int64_t v_stride_page, v_stride_head;   /* elements */
  float k_scale, v_scale;       /* dequantisation multipliers (1.0 unless 8-bit) */
  const int32_t *page_table;    /* [batch][page_table_stride] */
  int32_t page_table_stride;
  int32_t pad1;
  const int32_t *seq_lens;      /* [batch] */
  const float *k_vscales;       /* nullable: per-vector K scales (8-bit K/V), see layout */
  const float *v_vscales;       /* nullable: per-vector V scales; both or neither */
  int64_t vscale_stride_page, vscale_stride_head;   /* floats, multiples of 4 */
  const uint64_t *k_fragments;  /* nullable: device array of K fragment addresses */
  const uint64_t *v_fragments;  /* nullable: device array of V fragment addresses */
  int32_t fragment_pages_log2;  /* pages per fragment = 2^this, 0..20 */
  int32_t num_fragments;        /* entries in each fragment array (covers num_pages) */
} attn_kv;

/* Queries and outputs. */
typedef struct {
  const void *q;
  int32_t q_dtype;              /* F32, F16 or BF16 (see each call) */
  int32_t batch;
  int32_t q_rows;               /* decode: 1..8 rows; prefill: rows per sequence */
  int32_t num_q_heads;
  int64_t q_stride_b, q_stride_row, q_stride_head;   /* elements */
  void *o;
  int32_t o_dtype;              /* F32, F16 or BF16 */
  int32_t pad0;
  int64_t o_stride_b, o_stride_row, o_stride_head;   /* elements */
  float *lse;                   /* nullable [batch][num_q_heads][q_rows] */
} attn_io;

typedef struct {
  float softmax_scale;          /* <= 0 selects 1/sqrt(head_dim) */
  int32_t num_splits;           /* decode: 0 = plan from capacity and LDS; > 0 forces it */
  const float *sinks;           /* nullable [num_q_heads], finite or -inf */
  const uint8_t *block_mask;    /* attn_prefill_blocksparse only, else NULL */
  int32_t mask_heads;           /* 1 (shared) or num_kv_heads */
  int32_t mask_block;           /* tokens per mask block: a multiple of 64 */
  int32_t mask_q_blocks, mask_k_blocks;
  const int32_t *rows_per_seq;  /* nullable device int32 [batch]: query rows of each
                                   sequence (ragged verify / chunked prefill), values
                                   clamped to [0, q_rows]; see "Semantics" */
} attn_opts;

/* ABI version of the loaded library (ATTN_ABI_VERSION). */
int attn_abi_version(void);

/* Open device `hip_device` (must be gfx950) and return an opaque context in
 * *ctx (Geramy/LSE README, libLSE C API section: a caller opens the library
 * once and gets an opaque handle, every later call takes that handle and
 * returns a status, and a failed open reports its reason through an error
 * string).  The context caches the device facts the kernels are shaped by
 * (CU count, LDS per workgroup, architecture), since the pages choose kernel
 * shapes from device facts (Geramy/LSE summary page, first paragraph) and plan
 * split attention from the device's limits (Geramy/LSE releases, v0.4.20
 * "automatic split attention": LDS check).  On failure *ctx is NULL and the
 * status is ATTN_ERR_DEVICE (no HIP device, index out of range, not gfx950)
 * or ATTN_ERR_INVALID_ARGUMENT (ctx NULL).  The caller releases the context
 * with attn_close. */
attn_status attn_open(int hip_device, attn_ctx **ctx, char **err);

/* A context for planning and argument checking only, describing a device
 * with `num_cus` compute units: every call validates and plans as usual and
 * then returns ATTN_ERR_DEVICE instead of enqueuing work. */
attn_status attn_open_host_only(int num_cus, attn_ctx **ctx, char **err);

/* Release a context from attn_open or attn_open_host_only (the close half of
 * the open/close pair of the libLSE C API section of the Geramy/LSE README).
 * NULL is ignored.  The caller must not close a context while work enqueued
 * with it may still use it from another thread; work already on a stream
 * does not reference the context. */
void attn_close(attn_ctx *ctx);

/* Release a string the library returned through an `err` argument (Geramy/LSE
 * README, libLSE C API section: strings the library hands out are released
 * with the library's own free function, not the caller's allocator).  NULL is
 * ignored. */
void attn_free(void *p);

/* Decode plan: number of KV partitions, tokens per partition and the
 * workspace bytes attn_paged_decode needs for these arguments.  The
 * partition count follows the page table's capacity (page_table_stride *
 * page_size), the rows that share each K/V read and the device's CU count
 * (Geramy/LSE releases, v0.4.20: partitions from K/V table capacity, with an
 * LDS check).  tokens_per_split is the size at full capacity: unless
 * opts->num_splits forces a split, the kernels apply the same rule to the
 * longest seq_lens entry of the call and use shorter partitions (never more
 * than num_splits of them) when every sequence is shorter than the
 * capacity. */
attn_status attn_paged_decode_plan(const attn_ctx *ctx, const attn_io *io, const attn_kv *kv,
                                   const attn_opts *opts, int32_t *num_splits,
                                   int32_t *tokens_per_split, size_t *workspace_bytes,
                                   char **err);

/* Workspace bytes for attn_paged_decode (0 if the arguments are invalid). */
size_t attn_paged_decode_workspace_bytes(const attn_ctx *ctx, const attn_io *io,
                                         const attn_kv *kv, const attn_opts *opts);

/* Decode / verify: q_rows in [1, 8].  Q dtype: F32/F16/BF16 with F32 K/V,
 * equal to the K/V dtype for F16/BF16 K/V, F16 or BF16 with 8-bit K/V.
 * `workspace` is device memory of at least the queried size (16-byte
 * aligned, contents irrelevant) for the partition partials; it may be reused
 * by consecutive calls on one stream but not by calls that can run
 * concurrently.  block_mask must be NULL. */
attn_status attn_paged_decode(attn_ctx *ctx, const attn_io *io, const attn_kv *kv,
                              const attn_opts *opts, void *workspace, size_t workspace_bytes,
                              void *hip_stream, char **err);

/* Bytes of device-resident scratch behind attn_paged_decode_noalloc, per device. */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* attn_paged_decode without a caller workspace and without any allocation,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Arguments,
 * semantics, plan and kernels are those of attn_paged_decode; the partition
 * partials go to a device-resident scratch array of ATTN_NOALLOC_SCRATCH_BYTES
 * that the library holds on every device it runs on until the process ends
 * (its address is looked up once per device by attn_open).  The call
 * allocates and frees nothing.  A decode whose partials need more than
 * ATTN_NOALLOC_SCRATCH_BYTES (attn_paged_decode_plan's workspace_bytes) is
 * rejected with ATTN_ERR_WORKSPACE_TOO_SMALL before anything is enqueued.
 * Every call on a device shares that device's scratch: calls that can run at
 * the same time on one device (other streams, other threads, other contexts
 * of the same device) race and must be serialised by the caller; consecutive
 * calls on one stream are fine.  A host-only context returns ATTN_ERR_DEVICE
 * after validation and planning. */
attn_status attn_paged_decode_noalloc(attn_ctx *ctx, const attn_io *io, const attn_kv *kv,
                                      const attn_opts *opts, void *hip_stream, char **err);

/* Causal prefill (q_rows rows at the end of each sequence, q_rows <= seq_len
 * expected).  K/V F16, BF16, FP8 or BF8; Q F16/BF16 (equal to K/V for 16-bit
 * K/V).
 * block_mask must be NULL. */
attn_status attn_prefill(attn_ctx *ctx, const attn_io *io, const attn_kv *kv,
                         const attn_opts *opts, void *hip_stream, char **err);

/* Block-sparse causal prefill: as attn_prefill, with block_mask required. */
attn_status attn_prefill_blocksparse(attn_ctx *ctx, const attn_io *io, const attn_kv *kv,
                                     const attn_opts *opts, void *hip_stream, char **err);

/* New K/V rows for attn_kv_append. */
typedef struct {
  const void *k, *v;            /* [batch][n_new][num_kv_heads][head_dim] through the strides */
  int32_t dtype;                /* F32, F16 or BF16 */
  int32_t batch;
  int32_t n_new;                /* rows per sequence, >= 1 */
  int32_t pad0;
  int64_t stride_b, stride_row, stride_head;   /* elements, shared by k and v */
} attn_kv_rows;

/* K/V append, the step before decode / verify (Geramy/LSE README, "K/V
 * storage": the cache is kept in 16-bit or FP8 storage; Geramy/LSE releases,
 * v0.4.20, "Correctness": K/V writes checked against CPU references).
 * Row i of sequence b (0 <= i < n_new) is written to position
 * p = L_b - n_new + i, L_b = min(seq_lens[b], page_table_stride * 16), i.e.
 * seq_lens already counts the new rows, as in the attention calls; rows with
 * p < 0 are skipped.  Its K row goes to slot p % 16 of K tile
 * (page_table[b][p / 16], head), its V row to the same slot of the V tile.
 * The stored value is src / scale (k_scale or v_scale; one IEEE
 * single-precision division) rounded to the pool's dtype to nearest, ties to
 * even: F16 and BF16 overflow to infinity, FP8 e4m3fn saturates at +-448, BF8
 * e5m2 saturates finite values at +-57344 and keeps infinities, NaN stays NaN
 * (F32 stores the quotient).  With per-vector scales (k_vscales/v_vscales set;
 * k_scale and v_scale must then be 1) each new K or V vector x gets the scale
 * u = amax / fmax (one single-precision division; amax the largest |x_i| over
 * its finite entries, fmax 448 for FP8 and 57344 for BF8; u = 1 when the
 * quotient is 0), written to the vector's scale slot, and its values are
 * stored as x_i / u rounded as above.  Only those slots are written: the pool
 * memory (k_pages / v_pages, and the scale pools) must be writable, and the
 * pages for the new positions must already be in the page table.  Base pointers and strides are
 * 16-byte aligned, head_dim contiguous.  Appends of one call must not target
 * the same slot twice (distinct sequences own distinct pages). */
attn_status attn_kv_append(attn_ctx *ctx, const attn_kv *kv, const attn_kv_rows *rows,
                           void *hip_stream, char **err);

/* Test hook: gather sequence b's K and V through the page table and
 * dequantise them exactly as the attention kernels do, into FP32 arrays
 * k_out, v_out of [num_kv_heads][seq_len][head_dim] (device memory): each
 * value is (code value * per-vector scale) * per-tensor scale, evaluated in
 * FP32 in that order (the per-vector factor only where the cache has one).
 * The operation is the read half of the paged cache: K/V kept in pages of a
 * pool in fp32/fp16/bf16/fp8/bf8 storage, fp8 and bf8 with their scales
 * (Geramy/LSE README, "K/V storage" paragraph and table), reached through
 * fragment addresses where the pool is fragmented (Geramy/LSE releases,
 * v0.4.20 "K/V memory management"); the pages check the cache's contents
 * against CPU references (v0.4.20, "Correctness"), which is what the hook is
 * for.  Arguments: b < batch of the page table, 0 <= seq_len <=
 * page_table_stride * 16 (tokens gathered; seq_lens is not read), k_out and
 * v_out caller-owned device buffers of num_kv_heads * seq_len * head_dim
 * floats.  Errors as for the attention calls (ATTN_ERR_INVALID_ARGUMENT for
 * NULL outputs, negative or out-of-range b / seq_len). */
attn_status attn_debug_gather_kv(attn_ctx *ctx, const attn_kv *kv, int32_t b, int32_t seq_len,
                                 float *k_out, float *v_out, void *hip_stream, char **err);

/* Measurement hook: a read-only HBM probe, the practical read ceiling the
 * decode kernels are compared with.  pattern 0 streams [buf, buf + bytes)
 * contiguously; pattern 1 reads the 4 KiB tiles buf + 4096 * tile_order[i],
 * i < bytes / 4096, in that order (tile_order: device int32 array whose
 * entries lie in [0, bytes / 4096), trusted), the access pattern of a paged
 * pool; pattern 2 does the same with 2 KiB tiles (buf + 2048 * tile_order[i],
 * i < bytes / 2048, entries in [0, bytes / 2048)), the size of one (page, KV
 * head) tile of 8-bit K or V at head_dim 128.  buf must be 16-byte aligned
 * and bytes a positive multiple of 4096.
 * `sink` (device, one word) is written only if the data XOR to a fixed
 * constant: it exists so that no load can be optimised away. */
attn_status attn_debug_read_probe(attn_ctx *ctx, const void *buf, size_t bytes, int32_t pattern,
                                  const int32_t *tile_order, uint32_t *sink, void *hip_stream,
                                  char **err);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
