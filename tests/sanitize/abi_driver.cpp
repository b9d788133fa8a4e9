// Drives the library's host side (argument validation, split planning,
// workspace sizing, error strings) under AddressSanitizer and
// UndefinedBehaviorSanitizer through a planning-only context: every call
// validates and plans, then returns ATTN_ERR_DEVICE instead of enqueuing.
// Device pointers are fake (never dereferenced on the host).  Exits non-zero
// when a call returns an unexpected status.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "paged_attn.h"

namespace {

int failures = 0;

void expect(attn_status got, attn_status want, char *err, const char *what) {
  if (got != want) {
    std::printf("%s: status %d, expected %d (%s)\n", what, (int)got, (int)want, err ? err : "-");
    ++failures;
  }
  if (err) attn_free(err);
}

void *fake(uintptr_t a) { return reinterpret_cast<void *>(a); }

struct Case {
  attn_kv kv{};
  attn_io io{};
  attn_opts op{};
};

Case make(int B, int R, int Hq, int Hkv, int d, int stride, int dtype, int q_dtype) {
  Case c;
  const int eb = dtype == ATTN_F32 ? 4 : dtype <= ATTN_BF16 ? 2 : 1;
  const int qb = q_dtype == ATTN_F32 ? 4 : 2;
  c.kv.k_pages = fake(0x100000);
  c.kv.v_pages = fake(0x200000);
  c.kv.dtype = dtype;
  c.kv.num_pages = 4096;
  c.kv.page_size = 16;
  c.kv.num_kv_heads = Hkv;
  c.kv.head_dim = d;
  c.kv.k_stride_page = c.kv.v_stride_page = (int64_t)Hkv * 16 * d;
  c.kv.k_stride_head = c.kv.v_stride_head = (int64_t)16 * d;
  c.kv.k_scale = c.kv.v_scale = 1.0f;
  c.kv.page_table = static_cast<const int32_t *>(fake(0x300000));
  c.kv.page_table_stride = stride;
  c.kv.seq_lens = static_cast<const int32_t *>(fake(0x400000));
  c.io.q = fake(0x500000);
  c.io.q_dtype = q_dtype;
  c.io.batch = B;
  c.io.q_rows = R;
  c.io.num_q_heads = Hq;
  c.io.q_stride_head = d;
  c.io.q_stride_row = (int64_t)Hq * d;
  c.io.q_stride_b = (int64_t)R * Hq * d;
  c.io.o = fake(0x600000);
  c.io.o_dtype = q_dtype;
  c.io.o_stride_head = d;
  c.io.o_stride_row = (int64_t)Hq * d;
  c.io.o_stride_b = (int64_t)R * Hq * d;
  (void)eb;
  (void)qb;
  c.op.mask_heads = 1;
  c.op.mask_block = 128;
  c.op.mask_q_blocks = c.op.mask_k_blocks = 1;
  return c;
}

}  // namespace

int main() {
  attn_ctx *ctx = nullptr;
  char *err = nullptr;
  expect(attn_open_host_only(0, &ctx, &err), ATTN_ERR_INVALID_ARGUMENT, err, "open 0 CUs");
  err = nullptr;
  expect(attn_open_host_only(256, &ctx, &err), ATTN_OK, err, "open host-only");
  if (!ctx) return 1;

  const int dts[5] = {ATTN_F32, ATTN_F16, ATTN_BF16, ATTN_FP8_E4M3, ATTN_BF8_E5M2};
  const int ds[3] = {64, 128, 256};
  for (int dt : dts)
    for (int d : ds)
      for (int R = 1; R <= 8; R *= 2)
        for (int G = 1; G <= 8; G *= 2)
          for (int stride : {1, 64, 1024, 1 << 20, 1 << 26}) {
            const int q = dt == ATTN_F32 ? ATTN_F32 : dt == ATTN_F16 ? ATTN_F16 : ATTN_BF16;
            Case c = make(16, R, 8 * G, 8, d, stride, dt, q);
            int32_t P = 0, T = 0;
            size_t W = 0;
            err = nullptr;
            attn_status st = attn_paged_decode_plan(ctx, &c.io, &c.kv, &c.op, &P, &T, &W, &err);
            if (err) attn_free(err);
            if (st == ATTN_OK) {
              if (P < 1 || T < 1 || (int64_t)P * T < (int64_t)stride * 16 || W == 0) {
                std::printf("bad plan dt %d d %d R %d G %d stride %d: P %d T %d W %zu\n", dt, d, R,
                            G, stride, P, T, W);
                ++failures;
              }
              err = nullptr;
              expect(attn_paged_decode(ctx, &c.io, &c.kv, &c.op, fake(0x700000), W, nullptr, &err),
                     ATTN_ERR_DEVICE, err, "decode on host-only");
              err = nullptr;
              attn_status na = attn_paged_decode_noalloc(ctx, &c.io, &c.kv, &c.op, nullptr, &err);
              expect(na, W > ATTN_NOALLOC_SCRATCH_BYTES ? ATTN_ERR_WORKSPACE_TOO_SMALL
                                                        : ATTN_ERR_DEVICE,
                     err, "noalloc on host-only");
            } else if (st != ATTN_ERR_UNSUPPORTED) {
              std::printf("plan status %d for dt %d d %d\n", (int)st, dt, d);
              ++failures;
            }
            // prefill with and without a mask
            Case p = make(2, 256, 8 * G, 8, d, 16, dt, q);
            err = nullptr;
            st = attn_prefill(ctx, &p.io, &p.kv, &p.op, nullptr, &err);
            if (err) attn_free(err);
            if (st != ATTN_ERR_DEVICE && st != ATTN_ERR_UNSUPPORTED) {
              std::printf("prefill status %d\n", (int)st);
              ++failures;
            }
            p.op.block_mask = static_cast<const uint8_t *>(fake(0x800000));
            p.op.mask_q_blocks = p.op.mask_k_blocks = 2;
            err = nullptr;
            st = attn_prefill_blocksparse(ctx, &p.io, &p.kv, &p.op, nullptr, &err);
            if (err) attn_free(err);
            if (st != ATTN_ERR_DEVICE && st != ATTN_ERR_UNSUPPORTED) {
              std::printf("blocksparse status %d\n", (int)st);
              ++failures;
            }
          }

  // invalid arguments, each with an error string released by attn_free
  Case c = make(2, 1, 8, 2, 128, 64, ATTN_BF16, ATTN_BF16);
  err = nullptr;
  expect(attn_paged_decode(ctx, nullptr, &c.kv, &c.op, fake(0x700000), 1 << 24, nullptr, &err),
         ATTN_ERR_INVALID_ARGUMENT, err, "io NULL");
  err = nullptr;
  expect(attn_paged_decode(ctx, &c.io, nullptr, &c.op, fake(0x700000), 1 << 24, nullptr, &err),
         ATTN_ERR_INVALID_ARGUMENT, err, "kv NULL");
  c.io.q_rows = 9;
  err = nullptr;
  expect(attn_paged_decode(ctx, &c.io, &c.kv, &c.op, fake(0x700000), 1 << 24, nullptr, &err),
         ATTN_ERR_INVALID_ARGUMENT, err, "q_rows 9");
  c.io.q_rows = 1;
  c.kv.page_table_stride = (1 << 26) + 1;
  err = nullptr;
  expect(attn_paged_decode(ctx, &c.io, &c.kv, &c.op, fake(0x700000), 1 << 24, nullptr, &err),
         ATTN_ERR_UNSUPPORTED, err, "capacity above 2^30");
  c.kv.page_table_stride = 64;
  c.kv.k_pages = fake(0x100004);
  err = nullptr;
  expect(attn_paged_decode(ctx, &c.io, &c.kv, &c.op, fake(0x700000), 1 << 24, nullptr, &err),
         ATTN_ERR_INVALID_ARGUMENT, err, "misaligned K");
  c.kv.k_pages = fake(0x100000);
  err = nullptr;
  expect(attn_paged_decode(ctx, &c.io, &c.kv, &c.op, fake(0x700000), 16, nullptr, &err),
         ATTN_ERR_WORKSPACE_TOO_SMALL, err, "workspace too small");
  // append and gather validation
  attn_kv_rows rows{};
  rows.k = fake(0x900000);
  rows.v = fake(0xa00000);
  rows.dtype = ATTN_F32;
  rows.batch = 2;
  rows.n_new = 3;
  rows.stride_head = 128;
  rows.stride_row = 8 * 128;
  rows.stride_b = 3 * 8 * 128;
  c.kv.num_kv_heads = 8;
  err = nullptr;
  expect(attn_kv_append(ctx, &c.kv, &rows, nullptr, &err), ATTN_ERR_DEVICE, err, "append");
  rows.n_new = 0;
  err = nullptr;
  expect(attn_kv_append(ctx, &c.kv, &rows, nullptr, &err), ATTN_ERR_INVALID_ARGUMENT, err,
         "append n_new 0");
  err = nullptr;
  expect(attn_debug_gather_kv(ctx, &c.kv, 0, 64 * 16 + 1, static_cast<float *>(fake(0xb00000)),
                              static_cast<float *>(fake(0xc00000)), nullptr, &err),
         ATTN_ERR_INVALID_ARGUMENT, err, "gather past capacity");
  (void)attn_paged_decode_workspace_bytes(ctx, &c.io, &c.kv, &c.op);
  attn_close(ctx);
  attn_close(nullptr);
  attn_free(nullptr);
  std::printf("abi driver: %d failures\n", failures);
  return failures != 0;
}
