// C ABI of the paged attention library: argument validation, split planning,
// workspace sizing and kernel launches.  The library never allocates device
// memory and never synchronises; every call only enqueues on the given stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "paged_attn.h"
#include "attn_internal.h"

struct attn_ctx {
  int device;
  int num_cus;
  size_t lds_per_block;
  bool host_only;
  char arch[64];
  void *scratch;   // this device's decode scratch array (attn_paged_decode_noalloc), or null
};

namespace {

using pa::DecodeArgs;
using pa::PrefillArgs;

constexpr int kPage = 16;
constexpr int64_t kMaxCapacity = int64_t(1) << 30;   // tokens a page-table row may address
constexpr int kMaxDevices = 64;
constexpr int64_t kLdsPerCu = 160 * 1024;   // gfx950 LDS per compute unit
constexpr int64_t kSkRounds = 2;            // balanced partitions: rounds of resident workgroups

int elt_bytes(int dt) {
  switch (dt) {
    case ATTN_F32: return 4;
    case ATTN_F16: return 2;
    case ATTN_BF16: return 2;
    case ATTN_FP8_E4M3: return 1;
    case ATTN_BF8_E5M2: return 1;
  }
  return 0;
}

attn_status fail(char **err, attn_status st, const char *fmt, ...) {
  if (err) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    *err = strdup(buf);
  }
  return st;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// ---- shared validation --------------------------------------------------------

attn_status check_kv(const attn_kv *kv, char **err) {
  if (!kv) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "kv is NULL");
  if ((!kv->k_pages && !kv->k_fragments) || (!kv->v_pages && !kv->v_fragments))
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "K/V pages are NULL (and no fragment table is given)");
  if (!kv->page_table || !kv->seq_lens)
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "page_table / seq_lens is NULL");
  if (elt_bytes(kv->dtype) == 0) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "bad K/V dtype %d", kv->dtype);
  if (kv->num_pages < 1 || kv->num_kv_heads < 1 || kv->page_table_stride < 1)
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "num_pages, num_kv_heads and page_table_stride must be >= 1");
  if (kv->head_dim < 1 || kv->page_size < 1)
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "head_dim and page_size must be >= 1");
  if (kv->page_size != kPage) return fail(err, ATTN_ERR_UNSUPPORTED, "page_size %d (only 16)", kv->page_size);
  // token positions, partition bounds and their sums are int32 in the kernels
  if ((int64_t)kv->page_table_stride * kPage > kMaxCapacity)
    return fail(err, ATTN_ERR_UNSUPPORTED, "page_table_stride %d: capacity above 2^30 tokens",
                kv->page_table_stride);
  if (kv->head_dim != 64 && kv->head_dim != 128 && kv->head_dim != 256)
    return fail(err, ATTN_ERR_UNSUPPORTED, "head_dim %d (only 64, 128 or 256)", kv->head_dim);
  if (!aligned16(kv->k_pages) || !aligned16(kv->v_pages))
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "K/V pages must be 16-byte aligned");
  if (kv->k_fragments || kv->v_fragments) {
    if (kv->fragment_pages_log2 < 0 || kv->fragment_pages_log2 > 20)
      return fail(err, ATTN_ERR_INVALID_ARGUMENT, "fragment_pages_log2 %d outside [0, 20]", kv->fragment_pages_log2);
    if ((reinterpret_cast<uintptr_t>(kv->k_fragments) | reinterpret_cast<uintptr_t>(kv->v_fragments)) & 7u)
      return fail(err, ATTN_ERR_INVALID_ARGUMENT, "fragment tables must be 8-byte aligned");
    const int64_t need = ceil_div(kv->num_pages, int64_t(1) << kv->fragment_pages_log2);
    if (kv->num_fragments < need)
      return fail(err, ATTN_ERR_INVALID_ARGUMENT, "%d fragments do not cover %d pages of 2^%d per fragment",
                  kv->num_fragments, kv->num_pages, kv->fragment_pages_log2);
  }
  const int64_t tile = (int64_t)kPage * kv->head_dim;
  const int eb = elt_bytes(kv->dtype);
  const int64_t s[4] = {kv->k_stride_page, kv->k_stride_head, kv->v_stride_page, kv->v_stride_head};
  for (int i = 0; i < 4; ++i) {
    if (s[i] < tile) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "K/V strides must be >= one page tile (%lld elements)", (long long)tile);
    if ((s[i] * eb) % 16) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "K/V strides must be multiples of 16 bytes");
  }
  if (!(kv->k_scale > 0.f) || !(kv->v_scale > 0.f) || !std::isfinite(kv->k_scale) || !std::isfinite(kv->v_scale))
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "k_scale and v_scale must be finite and > 0");
  if ((kv->k_vscales == nullptr) != (kv->v_vscales == nullptr))
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "k_vscales and v_vscales must both be set or both be NULL");
  if (kv->k_vscales) {
    if (eb != 1) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "per-vector scales need 8-bit K/V (FP8 or BF8)");
    if (!aligned16(kv->k_vscales) || !aligned16(kv->v_vscales))
      return fail(err, ATTN_ERR_INVALID_ARGUMENT, "per-vector scale pools must be 16-byte aligned");
    if (kv->vscale_stride_page < kPage || kv->vscale_stride_head < kPage ||
        kv->vscale_stride_page % 4 || kv->vscale_stride_head % 4)
      return fail(err, ATTN_ERR_INVALID_ARGUMENT, "per-vector scale strides must be >= 16 and multiples of 4 floats");
  }
  return ATTN_OK;
}

attn_status check_io(const attn_io *io, const attn_kv *kv, char **err) {
  if (!io) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "io is NULL");
  if (!io->q || !io->o) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "q / o is NULL");
  if (io->batch < 1 || io->q_rows < 1 || io->num_q_heads < 1)
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "batch, q_rows and num_q_heads must be >= 1");
  if (io->num_q_heads % kv->num_kv_heads)
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "num_q_heads %d is not a multiple of num_kv_heads %d", io->num_q_heads, kv->num_kv_heads);
  if (io->q_dtype != ATTN_F32 && io->q_dtype != ATTN_F16 && io->q_dtype != ATTN_BF16)
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "q_dtype must be F32, F16 or BF16");
  if (io->o_dtype != ATTN_F32 && io->o_dtype != ATTN_F16 && io->o_dtype != ATTN_BF16)
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "o_dtype must be F32, F16 or BF16");
  if (!aligned16(io->q) || !aligned16(io->o)) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "q and o must be 16-byte aligned");
  if (io->lse && (reinterpret_cast<uintptr_t>(io->lse) & 3u)) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "lse must be 4-byte aligned");
  const int qb = elt_bytes(io->q_dtype), ob = elt_bytes(io->o_dtype);
  const int64_t qs[3] = {io->q_stride_b, io->q_stride_row, io->q_stride_head};
  const int64_t os[3] = {io->o_stride_b, io->o_stride_row, io->o_stride_head};
  for (int i = 0; i < 3; ++i) {
    if (qs[i] < 0 || os[i] < 0) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "negative q/o stride");
    if ((qs[i] * qb) % 16 || (os[i] * ob) % 16) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "q/o strides must be multiples of 16 bytes");
  }
  if (io->q_stride_head < kv->head_dim || io->o_stride_head < kv->head_dim)
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "q/o head stride below head_dim");
  return ATTN_OK;
}

attn_status check_ctx(const attn_ctx *ctx, char **err) {
  if (!ctx) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "ctx is NULL");
  return ATTN_OK;
}

// ---- decode planning ------------------------------------------------------------

struct DecodePlan {
  bool mfma;
  bool wide;              // head_dim 256 with more than 8 rows per KV head
  int rows, rb, row_blocks, P, T;
  int t_dyn, t_target, t_min, t_cap;   // the device-side partition rule (DecodeArgs)
  int sk, sk_wgs, sk_cmin, sk_unit, sk_rbw, sk_lds, sk_round;   // balanced split (DecodeArgs)
  size_t ws_bytes, ws_o_bytes, ws_ml_bytes, ws_tab_bytes;
};

constexpr int kTGran = 128;   // partition granularity (tokens)
constexpr int kTMax = 8192;   // partition size limit (page ids a wave preloads)
constexpr int kValuWgPerCu = 2;   // decode_valu workgroups per CU the planner counts on
constexpr int kMfmaWgPerCu = 1;   // decode_mfma workgroups per CU the planner counts on
constexpr int kWideWgPerCu = 2;   // head_dim 256 verify workgroups per CU
constexpr int64_t kValuTAuto = 1024;   // planned partition size limit of the VALU kernel
constexpr int64_t kValuRounds = 16;    // ... unless it plans more rounds of workgroups than this

attn_status plan_decode(const attn_ctx *ctx, const attn_io *io, const attn_kv *kv, const attn_opts *opts,
                        DecodePlan *pl, char **err) {
  attn_status st;
  if ((st = check_ctx(ctx, err)) != ATTN_OK) return st;
  if ((st = check_kv(kv, err)) != ATTN_OK) return st;
  if ((st = check_io(io, kv, err)) != ATTN_OK) return st;
  if (!opts) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "opts is NULL");
  if (opts->block_mask) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "attn_paged_decode takes no block mask");
  if (opts->num_splits < 0) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "num_splits must be >= 0");
  if (reinterpret_cast<uintptr_t>(opts->rows_per_seq) & 3u)
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "rows_per_seq must be 4-byte aligned");
  if (io->q_rows > 8) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "decode q_rows %d outside [1, 8]", io->q_rows);
  const int G = io->num_q_heads / kv->num_kv_heads;
  const int rows = G * io->q_rows;
  const int D = kv->head_dim;
  pl->rows = rows;
  // more than 8 rows per KV head go to the MFMA kernel where it exists for
  // these arguments; otherwise the VALU kernel runs them in blocks of 8 rows
  pl->mfma = kv->dtype != ATTN_F32 && rows > 8 &&
             pa::decode_mfma_supported(kv->dtype, io->q_dtype, D, rows);
  pl->wide = !pl->mfma && rows > 8 && pa::decode_wide_supported(kv->dtype, io->q_dtype, D, rows);
  if (pl->mfma || pl->wide) {
    pl->rb = rows;
    pl->row_blocks = 1;
  } else {
    if (!pa::decode_valu_supported(kv->dtype, io->q_dtype, D))
      return fail(err, ATTN_ERR_UNSUPPORTED, "decode: K/V dtype %d with Q dtype %d is not supported", kv->dtype, io->q_dtype);
    pl->rb = rows <= 4 ? 4 : 8;
    pl->row_blocks = (int)ceil_div(rows, pl->rb);
  }
  // LDS the partial kernel needs for its rows (merge buffer + softmax state)
  const size_t lds = pl->wide ? (size_t)2 * 32 * (256 + 16) * 2 + (size_t)2 * 256 * 32 * 2 + 128
                 : pl->mfma ? (size_t)round_up(rows, 16) * (D + 4) * 4 + 2 * 4 * 64 * 4
                            : (size_t)pl->rb * D * 4 + 4 * 16 * pl->rb * 4 + 3 * 4 * pl->rb * 4;
  if (lds > ctx->lds_per_block)
    return fail(err, ATTN_ERR_UNSUPPORTED, "decode needs %zu bytes of LDS, the device has %zu", lds, ctx->lds_per_block);

  // Partitions: the K/V table capacity is cut so that one round of resident
  // workgroups covers every (sequence, KV head, row block) once (a second,
  // partly filled round would run at a fraction of the occupancy); the VALU
  // kernel then cuts further, to partitions of at most kValuTAuto tokens.
  const int64_t cap = (int64_t)kv->page_table_stride * kPage;
  const int rows_per_wg = (pl->mfma || pl->wide) ? rows : pl->rb;
  // at least 32 tokens per row of a workgroup: a partition's FP32 partials (written
  // once, read back by the merge) stay within 1/16 of its K/V bytes at 16-bit K/V
  const int64_t tmin = round_up(std::max<int64_t>(256, 32 * (int64_t)rows_per_wg), kTGran);
  int64_t T;
  pl->t_dyn = 0;
  pl->t_target = 1;
  pl->t_min = (int)tmin;
  pl->t_cap = kTMax;
  if (opts->num_splits > 0) {
    T = round_up(ceil_div(cap, opts->num_splits), kTGran);
  } else {
    const int64_t groups = (int64_t)io->batch * kv->num_kv_heads * pl->row_blocks;
    // Resident workgroups are counted at no more than kValuWgPerCu (VALU
    // kernel) or kMfmaWgPerCu (MFMA kernel) per CU: that many already reach
    // the HBM read rate, and the longer partitions leave fewer idle
    // workgroups when sequences are shorter than the capacity.
    const int cap_cu = pl->wide ? kWideWgPerCu : pl->mfma ? kMfmaWgPerCu : kValuWgPerCu;
    int per_cu = ctx->host_only ? cap_cu
                 : pl->wide ? pa::decode_wide_blocks_per_cu(kv->dtype, io->q_dtype, kv->k_vscales != nullptr)
                            : pa::decode_blocks_per_cu(pl->mfma, kv->dtype, io->q_dtype, D, rows,
                                                       kv->k_vscales != nullptr);
    per_cu = std::max(1, std::min(per_cu, cap_cu));
    const int64_t slots = (int64_t)ctx->num_cus * per_cu;
    const int64_t target = std::max<int64_t>(1, slots / groups);
    T = std::max(tmin, round_up(ceil_div(cap, target), kTGran));
    // VALU kernel: partitions of at most kValuTAuto tokens.  Sequences
    // shorter than the capacity leave long partitions unevenly filled; with
    // short ones the workgroups that finish early take the remaining ones.
    // Measured (16 sequences, 32 query / 8 KV heads, d 128): lengths
    // U[8K,16K] +6%, U[4K,32K] +20%, 32 x U[2K,16K] +28%; all 16K equal;
    // 4 x 64K -2.5%.
    // The limit is lifted where it would plan more than kValuRounds rounds
    // of resident workgroups: with many sequences it only multiplies the
    // grid, and every launched workgroup costs, even one that exits at once
    // past its sequence's end (measured, 512 x 1,024 tokens in 1,024-token
    // tables: 372 us at 1 partition per sequence, 541 us at 2, 940 us at 8).
    if (!pl->mfma && !pl->wide)
      T = std::max(std::min(T, std::max(tmin, kValuTAuto)),
                   round_up(ceil_div(cap, std::max<int64_t>(1, kValuRounds * slots / groups)), kTGran));
    // the kernels apply the same rule to the batch's longest sequence, so
    // that sequences far shorter than the capacity still fill the CUs
    pl->t_dyn = 1;
    pl->t_target = (int)std::min<int64_t>(target, INT32_MAX);
    pl->t_cap = (int)std::min<int64_t>(kTMax, (!pl->mfma && !pl->wide) ? std::max(tmin, kValuTAuto)
                                                                         : kTMax);
  }
  // a wave of the head_dim 256 verify kernel preloads the page ids of its
  // pages: at most 8192 tokens per partition (the VALU and MFMA kernels load
  // them in blocks as their walk reaches them)
  if (pl->wide) T = std::min<int64_t>(T, kTMax);
  T = std::min<int64_t>(T, std::min<int64_t>(round_up(cap, kTGran), int64_t(1) << 30));
  int64_t P = ceil_div(cap, T);
  pl->sk = 0;
  pl->sk_wgs = pl->sk_cmin = pl->sk_unit = pl->sk_rbw = pl->sk_lds = pl->sk_round = 0;
  int64_t slots = (int64_t)io->batch * kv->num_kv_heads * rows * P;
  if (opts->num_splits == 0 && !pl->wide && io->batch <= 64 && pl->row_blocks == 1) {
    // Balanced partitions (up to 64 sequences, one row block): per KV head,
    // each sequence is cut into partitions of at most lam units (pages, or
    // page pairs for the MFMA kernel), lam the smallest size that needs one
    // round of resident workgroups, or two if one round leaves the partitions
    // unequal; the kernels compute lam from seq_lens on the device, so
    // sequences of different lengths cost their length (with one partition
    // size for all, set by the longest, short sequences leave workgroups idle
    // or empty).
    const int cap_cu = pl->mfma ? kMfmaWgPerCu : kValuWgPerCu;
    int per_cu = ctx->host_only ? cap_cu
                                : pa::decode_blocks_per_cu(pl->mfma, kv->dtype, io->q_dtype, D, rows,
                                                           kv->k_vscales != nullptr);
    per_cu = std::max(1, std::min(per_cu, cap_cu));
    const int64_t wgs = (int64_t)ctx->num_cus * per_cu;
    const int unit = pl->mfma ? 32 : kPage;
    pl->sk = 1;
    // partitions per KV head: kSkRounds rounds of the resident workgroups
    const int64_t round = ceil_div(wgs, kv->num_kv_heads);
    const int64_t rph = std::max<int64_t>(io->batch, kSkRounds * round);
    pl->sk_wgs = (int)std::min<int64_t>(rph, INT32_MAX);
    // Equal lengths (one round): the VALU kernel with page tiles of at least
    // 4 KiB takes one workgroup per CU, half the partitions of twice the
    // length (fewer prologues, epilogues and partials; measured on one box,
    // alternating runs: 16 x 16,384 bf16 R=1 +2%, one KV head of it +7%).
    // With smaller tiles (8-bit K/V, head_dim 64 at 16 bits) one workgroup
    // per CU cannot keep enough bytes in flight (e4m3fn 4 x 65,536: -20%),
    // and unequal lengths keep the finer partitions of two rounds (-4%).
    // Fragment-addressed pools keep two as well: each page's fragment-table
    // lookup is a dependent load that half the waves hide poorly (the
    // headline in 256 KiB fragments: 19% over the contiguous call at one
    // workgroup per CU, 3% at two).
    const bool big_tiles = (int64_t)kPage * D * elt_bytes(kv->dtype) >= 4096;
    const bool fragmented = kv->k_fragments || kv->v_fragments;
    const int64_t round_eq = (!pl->mfma && big_tiles && !fragmented && per_cu > 1)
                                 ? ceil_div((int64_t)ctx->num_cus, kv->num_kv_heads)
                                 : rph / kSkRounds;
    pl->sk_round = (int)std::min<int64_t>(round_eq, INT32_MAX);
    pl->sk_unit = unit;
    pl->sk_cmin = (int)ceil_div(tmin, unit);
    pl->sk_rbw = rows_per_wg;
    // dynamic LDS that keeps per_cu + 1 workgroups from sharing a CU (the
    // kernels' own LDS is far below what that leaves for per_cu of them)
    pl->sk_lds = (int)(kLdsPerCu / (per_cu + 1) + 256);
    if ((size_t)pl->sk_lds + lds > ctx->lds_per_block) pl->sk_lds = 0;
    // the partition size at full capacity (one round), reported as the plan's
    const int64_t c_full = std::max<int64_t>(
        pl->sk_cmin, ceil_div(ceil_div(cap, unit), std::max<int64_t>(1, pl->sk_round / io->batch)));
    T = std::min<int64_t>(c_full * unit, int64_t(1) << 30);
    P = ceil_div(cap, T);
    slots = rph * kv->num_kv_heads * rows_per_wg;
  }
  if (P > 65535) return fail(err, ATTN_ERR_UNSUPPORTED, "too many partitions (%lld)", (long long)P);
  pl->P = (int)P;
  pl->T = (int)T;
  pl->ws_o_bytes = (size_t)round_up(slots * D * 4, 256);
  pl->ws_ml_bytes = (size_t)round_up(slots * 2 * 4, 256);
  pl->ws_tab_bytes = pl->sk ? (size_t)round_up((int64_t)kv->num_kv_heads * io->batch * 2 * 4, 256) : 0;
  pl->ws_bytes = pl->ws_o_bytes + pl->ws_ml_bytes + pl->ws_tab_bytes;
  return ATTN_OK;
}

float score_scale(const attn_opts *opts, const attn_kv *kv) {
  const float s = opts->softmax_scale > 0.f ? opts->softmax_scale : 1.0f / std::sqrt((float)kv->head_dim);
  return s * kv->k_scale * 1.4426950408889634f;
}

struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) { ok = false; return; }
    if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
  }
  ~DeviceGuard() {
    int cur;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

// Device address of the decode scratch array on device `dev`, looked up once
// per device with that device current and kept for every later context.
attn_status device_scratch(int dev, void **ptr, char **err) {
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  if (dev < 0 || dev >= kMaxDevices) return fail(err, ATTN_ERR_DEVICE, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    DeviceGuard g(dev);
    if (!g.ok) return fail(err, ATTN_ERR_DEVICE, "cannot select device %d", dev);
    void *p = nullptr;
    const hipError_t e = pa::decode_scratch_address(&p);
    if (e != hipSuccess || !p)
      return fail(err, ATTN_ERR_DEVICE, "hipGetSymbolAddress(decode scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return ATTN_OK;
}

attn_status launched(hipError_t e, char **err, const char *what) {
  if (e != hipSuccess) return fail(err, ATTN_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return ATTN_OK;
}

// ---- prefill ------------------------------------------------------------------------

attn_status prefill_common(attn_ctx *ctx, const attn_io *io, const attn_kv *kv, const attn_opts *opts,
                           bool sparse, void *stream, char **err) {
  attn_status st;
  if ((st = check_ctx(ctx, err)) != ATTN_OK) return st;
  if ((st = check_kv(kv, err)) != ATTN_OK) return st;
  if ((st = check_io(io, kv, err)) != ATTN_OK) return st;
  if (!opts) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "opts is NULL");
  if (!sparse && opts->block_mask) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "attn_prefill takes no block mask (use attn_prefill_blocksparse)");
  if (reinterpret_cast<uintptr_t>(opts->rows_per_seq) & 3u)
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "rows_per_seq must be 4-byte aligned");
  if (sparse) {
    if (!opts->block_mask) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "attn_prefill_blocksparse needs a block mask");
    if (opts->mask_block < 64 || opts->mask_block % 64)
      return fail(err, ATTN_ERR_INVALID_ARGUMENT, "mask_block %d must be a positive multiple of 64", opts->mask_block);
    if (opts->mask_heads != 1 && opts->mask_heads != kv->num_kv_heads)
      return fail(err, ATTN_ERR_INVALID_ARGUMENT, "mask_heads must be 1 or num_kv_heads");
    if (opts->mask_q_blocks < 1 || opts->mask_k_blocks < 1)
      return fail(err, ATTN_ERR_INVALID_ARGUMENT, "mask_q_blocks and mask_k_blocks must be >= 1");
  }
  const int G = io->num_q_heads / kv->num_kv_heads;
  if (!pa::prefill_supported(kv->dtype, io->q_dtype, kv->head_dim))
    return fail(err, ATTN_ERR_UNSUPPORTED, "prefill: K/V dtype %d with Q dtype %d is not supported", kv->dtype, io->q_dtype);
  PrefillArgs a{};
  a.q = io->q;
  a.q_sb = io->q_stride_b; a.q_sr = io->q_stride_row; a.q_sh = io->q_stride_head;
  a.k = kv->k_pages; a.v = kv->v_pages;
  a.k_sp = kv->k_stride_page; a.k_sh = kv->k_stride_head;
  a.v_sp = kv->v_stride_page; a.v_sh = kv->v_stride_head;
  a.page_table = kv->page_table;
  a.pt_stride = kv->page_table_stride;
  a.capacity = (int32_t)std::min<int64_t>((int64_t)kv->page_table_stride * kPage, INT32_MAX);
  a.lens = kv->seq_lens;
  a.B = io->batch; a.n_q = io->q_rows; a.Hq = io->num_q_heads; a.Hkv = kv->num_kv_heads;
  a.G = G; a.D = kv->head_dim;
  a.kv_dtype = kv->dtype; a.q_dtype = io->q_dtype; a.o_dtype = io->o_dtype;
  a.score_scale = score_scale(opts, kv);
  a.v_scale = kv->v_scale;
  a.sinks = opts->sinks;
  a.o = io->o;
  a.o_sb = io->o_stride_b; a.o_sr = io->o_stride_row; a.o_sh = io->o_stride_head;
  a.lse = io->lse;
  a.rows_b = opts->rows_per_seq;
  a.mask = sparse ? opts->block_mask : nullptr;
  a.mask_heads = opts->mask_heads; a.mask_block = opts->mask_block;
  a.mask_nqb = opts->mask_q_blocks; a.mask_nkb = opts->mask_k_blocks;
  a.k_vs = kv->k_vscales; a.v_vs = kv->v_vscales;
  a.vs_sp = kv->vscale_stride_page; a.vs_sh = kv->vscale_stride_head;
  a.k_frag = kv->k_fragments; a.v_frag = kv->v_fragments;
  a.frag_shift = kv->fragment_pages_log2;
  a.q_tiles = (int)ceil_div(io->q_rows, 128);
  // head_dim 256 runs one query head per workgroup (16 rows per wave)
  a.heads_per_wg = (kv->head_dim == 256 || G % 2) ? 1 : 2;
  // groups dealt over 8 XCDs (padded), each with q_tiles tasks of G/HPW workgroups
  const int64_t groups = (int64_t)a.B * a.Hkv;
  const int64_t nwg = round_up(groups, 8) * a.q_tiles * (G / a.heads_per_wg);
  if (nwg > INT32_MAX) return fail(err, ATTN_ERR_UNSUPPORTED, "prefill grid too large");
  a.num_wg = (int)nwg;
  if (ctx->host_only) return fail(err, ATTN_ERR_DEVICE, "host-only context: nothing enqueued");
  DeviceGuard g(ctx->device);
  if (!g.ok) return fail(err, ATTN_ERR_DEVICE, "cannot select device %d", ctx->device);
  return launched(pa::launch_prefill(a, (hipStream_t)stream), err, "prefill launch");
}

// Enqueue a planned decode with its partials in `workspace` (>= pl.ws_bytes).
attn_status decode_enqueue(attn_ctx *ctx, const attn_io *io, const attn_kv *kv, const attn_opts *opts,
                           const DecodePlan &pl, void *workspace, void *hip_stream, char **err) {
  DecodeArgs a{};
  a.q = io->q;
  a.q_sb = io->q_stride_b; a.q_sr = io->q_stride_row; a.q_sh = io->q_stride_head;
  a.k = kv->k_pages; a.v = kv->v_pages;
  a.k_sp = kv->k_stride_page; a.k_sh = kv->k_stride_head;
  a.v_sp = kv->v_stride_page; a.v_sh = kv->v_stride_head;
  a.page_table = kv->page_table;
  a.pt_stride = kv->page_table_stride;
  a.capacity = (int32_t)std::min<int64_t>((int64_t)kv->page_table_stride * kPage, INT32_MAX);
  a.lens = kv->seq_lens;
  a.B = io->batch; a.R = io->q_rows; a.Hq = io->num_q_heads; a.Hkv = kv->num_kv_heads;
  a.G = io->num_q_heads / kv->num_kv_heads; a.D = kv->head_dim;
  a.rows = pl.rows;
  a.kv_dtype = kv->dtype; a.q_dtype = io->q_dtype; a.o_dtype = io->o_dtype;
  a.score_scale = score_scale(opts, kv);
  a.v_scale = kv->v_scale;
  a.sinks = opts->sinks;
  a.o = io->o;
  a.o_sb = io->o_stride_b; a.o_sr = io->o_stride_row; a.o_sh = io->o_stride_head;
  a.lse = io->lse;
  a.rows_b = opts->rows_per_seq;
  a.k_vs = kv->k_vscales; a.v_vs = kv->v_vscales;
  a.vs_sp = kv->vscale_stride_page; a.vs_sh = kv->vscale_stride_head;
  a.k_frag = kv->k_fragments; a.v_frag = kv->v_fragments;
  a.frag_shift = kv->fragment_pages_log2;
  a.P = pl.P; a.T = pl.T;
  a.t_dyn = pl.t_dyn; a.t_target = pl.t_target; a.t_min = pl.t_min; a.t_cap = pl.t_cap;
  a.row_blocks = pl.row_blocks;
  a.sk = pl.sk; a.sk_wgs = pl.sk_wgs; a.sk_cmin = pl.sk_cmin; a.sk_unit = pl.sk_unit;
  a.sk_rbw = pl.sk_rbw; a.sk_lds = pl.sk_lds; a.sk_round = pl.sk_round;
  a.ws_o = reinterpret_cast<float *>(workspace);
  a.ws_ml = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + pl.ws_o_bytes);
  a.sk_tab = reinterpret_cast<int32_t *>(reinterpret_cast<char *>(workspace) + pl.ws_o_bytes +
                                         pl.ws_ml_bytes);
  if (ctx->host_only) return fail(err, ATTN_ERR_DEVICE, "host-only context: nothing enqueued");
  DeviceGuard g(ctx->device);
  if (!g.ok) return fail(err, ATTN_ERR_DEVICE, "cannot select device %d", ctx->device);
  hipStream_t s = (hipStream_t)hip_stream;
  attn_status st = launched(pl.wide ? pa::launch_decode_wide(a, s)
                : pl.mfma ? pa::launch_decode_mfma(a, s) : pa::launch_decode_valu(a, s),
                err, "decode partial launch");
  if (st != ATTN_OK) return st;
  return launched(pa::launch_decode_merge(a, s), err, "decode merge launch");
}

}  // namespace

extern "C" {

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

void attn_free(void *p) { free(p); }

attn_status attn_open(int hip_device, attn_ctx **ctx, char **err) {
  if (!ctx) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "ctx is NULL");
  *ctx = nullptr;
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess || n == 0) return fail(err, ATTN_ERR_DEVICE, "no HIP device visible (%s)", hipGetErrorString(e));
  if (hip_device < 0 || hip_device >= n) return fail(err, ATTN_ERR_DEVICE, "device %d out of range (%d visible)", hip_device, n);
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, hip_device);
  if (e != hipSuccess) return fail(err, ATTN_ERR_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(err, ATTN_ERR_DEVICE, "device %d is %s; this library is built for gfx950", hip_device, prop.gcnArchName);
  attn_ctx *c = (attn_ctx *)calloc(1, sizeof(attn_ctx));
  if (!c) return fail(err, ATTN_ERR_DEVICE, "out of host memory");
  c->device = hip_device;
  c->num_cus = prop.multiProcessorCount;
  c->lds_per_block = prop.sharedMemPerBlock;
  c->host_only = false;
  snprintf(c->arch, sizeof c->arch, "%s", prop.gcnArchName);
  attn_status st = device_scratch(hip_device, &c->scratch, err);
  if (st != ATTN_OK) {
    free(c);
    return st;
  }
  *ctx = c;
  return ATTN_OK;
}

attn_status attn_open_host_only(int num_cus, attn_ctx **ctx, char **err) {
  if (!ctx) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "ctx is NULL");
  *ctx = nullptr;
  if (num_cus < 1) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "num_cus must be >= 1");
  attn_ctx *c = (attn_ctx *)calloc(1, sizeof(attn_ctx));
  if (!c) return fail(err, ATTN_ERR_DEVICE, "out of host memory");
  c->device = -1;
  c->num_cus = num_cus;
  c->lds_per_block = 160 * 1024;
  c->host_only = true;
  snprintf(c->arch, sizeof c->arch, "gfx950 (host-only)");
  *ctx = c;
  return ATTN_OK;
}

void attn_close(attn_ctx *ctx) { free(ctx); }

attn_status attn_paged_decode_plan(const attn_ctx *ctx, const attn_io *io, const attn_kv *kv,
                                   const attn_opts *opts, int32_t *num_splits,
                                   int32_t *tokens_per_split, size_t *workspace_bytes, char **err) {
  DecodePlan pl;
  attn_status st = plan_decode(ctx, io, kv, opts, &pl, err);
  if (st != ATTN_OK) return st;
  if (num_splits) *num_splits = pl.P;
  if (tokens_per_split) *tokens_per_split = pl.T;
  if (workspace_bytes) *workspace_bytes = pl.ws_bytes;
  return ATTN_OK;
}

size_t attn_paged_decode_workspace_bytes(const attn_ctx *ctx, const attn_io *io, const attn_kv *kv,
                                         const attn_opts *opts) {
  DecodePlan pl;
  if (plan_decode(ctx, io, kv, opts, &pl, nullptr) != ATTN_OK) return 0;
  return pl.ws_bytes;
}

attn_status attn_paged_decode(attn_ctx *ctx, const attn_io *io, const attn_kv *kv, const attn_opts *opts,
                              void *workspace, size_t workspace_bytes, void *hip_stream, char **err) {
  DecodePlan pl;
  attn_status st = plan_decode(ctx, io, kv, opts, &pl, err);
  if (st != ATTN_OK) return st;
  if (!workspace) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (!aligned16(workspace)) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  if (workspace_bytes < pl.ws_bytes)
    return fail(err, ATTN_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes, pl.ws_bytes);
  return decode_enqueue(ctx, io, kv, opts, pl, workspace, hip_stream, err);
}

attn_status attn_paged_decode_noalloc(attn_ctx *ctx, const attn_io *io, const attn_kv *kv,
                                      const attn_opts *opts, void *hip_stream, char **err) {
  DecodePlan pl;
  attn_status st = plan_decode(ctx, io, kv, opts, &pl, err);
  if (st != ATTN_OK) return st;
  static_assert(pa::kDecodeScratchBytes == ATTN_NOALLOC_SCRATCH_BYTES, "scratch size");
  if (pl.ws_bytes > pa::kDecodeScratchBytes)
    return fail(err, ATTN_ERR_WORKSPACE_TOO_SMALL,
                "this decode needs %zu bytes of partials; the library's device-resident scratch "
                "holds %zu (ATTN_NOALLOC_SCRATCH_BYTES): use attn_paged_decode with a workspace",
                pl.ws_bytes, (size_t)pa::kDecodeScratchBytes);
  if (ctx->host_only) return fail(err, ATTN_ERR_DEVICE, "host-only context: nothing enqueued");
  if (!ctx->scratch) return fail(err, ATTN_ERR_DEVICE, "no device scratch for device %d", ctx->device);
  return decode_enqueue(ctx, io, kv, opts, pl, ctx->scratch, hip_stream, err);
}

attn_status attn_prefill(attn_ctx *ctx, const attn_io *io, const attn_kv *kv, const attn_opts *opts,
                         void *hip_stream, char **err) {
  return prefill_common(ctx, io, kv, opts, false, hip_stream, err);
}

attn_status attn_prefill_blocksparse(attn_ctx *ctx, const attn_io *io, const attn_kv *kv,
                                     const attn_opts *opts, void *hip_stream, char **err) {
  return prefill_common(ctx, io, kv, opts, true, hip_stream, err);
}

attn_status attn_debug_gather_kv(attn_ctx *ctx, const attn_kv *kv, int32_t b, int32_t seq_len,
                                 float *k_out, float *v_out, void *hip_stream, char **err) {
  attn_status st;
  if ((st = check_ctx(ctx, err)) != ATTN_OK) return st;
  if ((st = check_kv(kv, err)) != ATTN_OK) return st;
  if (!k_out || !v_out) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "k_out / v_out is NULL");
  if (b < 0 || seq_len < 0) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "negative b or seq_len");
  if ((int64_t)seq_len > (int64_t)kv->page_table_stride * kPage)
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "seq_len beyond the page-table capacity");
  if (ctx->host_only) return fail(err, ATTN_ERR_DEVICE, "host-only context: nothing enqueued");
  DeviceGuard g(ctx->device);
  if (!g.ok) return fail(err, ATTN_ERR_DEVICE, "cannot select device %d", ctx->device);
  return launched(pa::launch_debug_gather(kv->k_pages, kv->v_pages, kv->k_stride_page, kv->k_stride_head,
                                          kv->v_stride_page, kv->v_stride_head, kv->dtype,
                                          kv->num_kv_heads, kv->head_dim, kv->k_scale, kv->v_scale,
                                          kv->k_vscales, kv->v_vscales, kv->vscale_stride_page,
                                          kv->vscale_stride_head, kv->k_fragments, kv->v_fragments,
                                          kv->fragment_pages_log2,
                                          kv->page_table + (int64_t)b * kv->page_table_stride, seq_len,
                                          k_out, v_out, (hipStream_t)hip_stream),
                  err, "debug gather launch");
}

attn_status attn_kv_append(attn_ctx *ctx, const attn_kv *kv, const attn_kv_rows *rows,
                           void *hip_stream, char **err) {
  attn_status st;
  if ((st = check_ctx(ctx, err)) != ATTN_OK) return st;
  if ((st = check_kv(kv, err)) != ATTN_OK) return st;
  if (!rows) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "rows is NULL");
  if (!rows->k || !rows->v) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "rows k / v is NULL");
  if (rows->dtype != ATTN_F32 && rows->dtype != ATTN_F16 && rows->dtype != ATTN_BF16)
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "rows dtype must be F32, F16 or BF16");
  if (rows->batch < 1 || rows->n_new < 1)
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "batch and n_new must be >= 1");
  if (!aligned16(rows->k) || !aligned16(rows->v))
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "rows k and v must be 16-byte aligned");
  const int sb = elt_bytes(rows->dtype);
  const int64_t rs[3] = {rows->stride_b, rows->stride_row, rows->stride_head};
  for (int i = 0; i < 3; ++i) {
    if (rs[i] < 0) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "negative rows stride");
    if ((rs[i] * sb) % 16) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "rows strides must be multiples of 16 bytes");
  }
  if (rows->stride_head < kv->head_dim)
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "rows head stride below head_dim");
  if (kv->k_vscales && (kv->k_scale != 1.0f || kv->v_scale != 1.0f))
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "an append with per-vector scales needs k_scale = v_scale = 1");
  if (ctx->host_only) return fail(err, ATTN_ERR_DEVICE, "host-only context: nothing enqueued");
  DeviceGuard g(ctx->device);
  if (!g.ok) return fail(err, ATTN_ERR_DEVICE, "cannot select device %d", ctx->device);
  pa::AppendArgs a{};
  a.k_src = rows->k;
  a.v_src = rows->v;
  a.src_dtype = rows->dtype;
  a.s_b = rows->stride_b;
  a.s_r = rows->stride_row;
  a.s_h = rows->stride_head;
  a.k = const_cast<void *>(kv->k_pages);
  a.v = const_cast<void *>(kv->v_pages);
  a.k_sp = kv->k_stride_page;
  a.k_sh = kv->k_stride_head;
  a.v_sp = kv->v_stride_page;
  a.v_sh = kv->v_stride_head;
  a.kv_dtype = kv->dtype;
  a.page_table = kv->page_table;
  a.pt_stride = kv->page_table_stride;
  a.capacity = (int32_t)std::min<int64_t>((int64_t)kv->page_table_stride * kPage, INT32_MAX);
  a.lens = kv->seq_lens;
  a.B = rows->batch;
  a.n_new = rows->n_new;
  a.Hkv = kv->num_kv_heads;
  a.D = kv->head_dim;
  a.k_scale = kv->k_scale;
  a.v_scale = kv->v_scale;
  a.k_vs = const_cast<float *>(kv->k_vscales);
  a.v_vs = const_cast<float *>(kv->v_vscales);
  a.vs_sp = kv->vscale_stride_page;
  a.vs_sh = kv->vscale_stride_head;
  a.k_frag = kv->k_fragments;
  a.v_frag = kv->v_fragments;
  a.frag_shift = kv->fragment_pages_log2;
  return launched(pa::launch_kv_append(a, (hipStream_t)hip_stream), err, "K/V append launch");
}

attn_status attn_debug_read_probe(attn_ctx *ctx, const void *buf, size_t bytes, int32_t pattern,
                                  const int32_t *tile_order, uint32_t *sink, void *hip_stream,
                                  char **err) {
  attn_status st;
  if ((st = check_ctx(ctx, err)) != ATTN_OK) return st;
  if (!buf || !sink) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "buf / sink is NULL");
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "buf is not 16-byte aligned");
  if (bytes == 0 || bytes % 4096 != 0)
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "bytes must be a positive multiple of 4096");
  if (pattern < 0 || pattern > 2)
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "pattern must be 0, 1 or 2");
  if (pattern != 0 && !tile_order) return fail(err, ATTN_ERR_INVALID_ARGUMENT, "tile_order is NULL");
  if (pattern != 0 && bytes / (pattern == 1 ? 4096 : 2048) > (size_t)INT32_MAX)
    return fail(err, ATTN_ERR_INVALID_ARGUMENT, "too many tiles");
  if (ctx->host_only) return fail(err, ATTN_ERR_DEVICE, "host-only context: nothing enqueued");
  DeviceGuard g(ctx->device);
  if (!g.ok) return fail(err, ATTN_ERR_DEVICE, "cannot select device %d", ctx->device);
  return launched(pa::launch_read_probe(buf, bytes, pattern, tile_order, sink, ctx->num_cus,
                                        (hipStream_t)hip_stream),
                  err, "read probe launch");
}

}  // extern "C"
