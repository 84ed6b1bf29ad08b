/* Host-side argument checks of the C ABI (include/blk.h), built with the
 * host AddressSanitizer and UndefinedBehaviorSanitizer together with a
 * host-only build of the library (tests/test_abi_sanitize.py does both).
 * Every call below must be refused before it touches the GPU: the data
 * pointers are fake, never-dereferenced addresses.  Exit status 0 when every
 * call returned the expected status. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../include/blk.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

#define P(a) ((void*)(uintptr_t)(a))
#define A 0x10000u
#define MIS 0x10008u

static blk_cfg d20(void) {
  blk_cfg c;
  memset(&c, 0, sizeof c);
  c.B = 32; c.T = 2048; c.C = 1280; c.H = 10; c.D = 128; c.F = 5120;
  c.eps = 1e-6f; c.rope_base = 10000.f; c.dtype = BLK_BF16; c.gemm = BLK_GEMM_NATIVE;
  return c;
}

static int fwd(const blk_cfg* c, void* x, void* w_o, void* y, void* saved, size_t saved_sz, void* scratch,
               size_t scratch_sz) {
  return block_fwd(c, x, P(A + 0x100), w_o, P(A + 0x300), P(A + 0x400), y, saved, saved_sz, scratch, scratch_sz, 0);
}

static int bwd(const blk_cfg* c, void* saved, size_t saved_sz, void* dx, float* dw_fc, int acc, void* scratch,
               size_t scratch_sz) {
  return block_bwd(c, P(A), P(A), P(A), P(A), P(A), P(A), saved, saved_sz, dx, (float*)P(A), (float*)P(A), dw_fc,
                   (float*)P(A), acc, scratch, scratch_sz, 0);
}

int main(void) {
  const size_t big = (size_t)1 << 40;
  blk_cfg c = d20(), bad;

  /* size queries */
  const size_t saved = block_saved_bytes(&c);
  expect("saved bytes nonzero", saved > 0, 1);
  expect("scratch >= saved", block_scratch_bytes(&c) >= saved, 1);
  expect("null cfg saved", (int)block_saved_bytes(NULL), 0);
  bad = c; bad.D = 64;
  expect("D=64 saved", (int)block_saved_bytes(&bad), 0);
  bad = c; bad.n_kv_head = 3;
  expect("groups of 3", (int)block_scratch_bytes(&bad), 0);

  /* block_fwd */
  expect("fwd null cfg", fwd(NULL, P(A), P(A + 0x200), P(A + 0x500), P(A + 0x600), big, P(A + 0x700), big),
         BLK_EINVAL);
  expect("fwd null x", fwd(&c, NULL, P(A + 0x200), P(A + 0x500), P(A + 0x600), big, P(A + 0x700), big), BLK_EINVAL);
  expect("fwd y aliases x", fwd(&c, P(A), P(A + 0x200), P(A), P(A + 0x600), big, P(A + 0x700), big), BLK_EINVAL);
  expect("fwd misaligned", fwd(&c, P(A), P(MIS), P(A + 0x500), P(A + 0x600), big, P(A + 0x700), big), BLK_EALIGN);
  expect("fwd short saved", fwd(&c, P(A), P(A + 0x200), P(A + 0x500), P(A + 0x600), 10, P(A + 0x700), big),
         BLK_ENOSPC);
  expect("fwd no scratch", fwd(&c, P(A), P(A + 0x200), P(A + 0x500), NULL, 0, NULL, 0), BLK_EINVAL);
  bad = c; bad.gemm = BLK_GEMM_FP8_E4M3; bad.dtype = BLK_F32;
  expect("fwd fp8 f32", fwd(&bad, P(A), P(A + 0x200), P(A + 0x500), P(A + 0x600), big, P(A + 0x700), big),
         BLK_EUNSUPPORTED);
  bad = c; bad.window = -1;
  expect("fwd window", fwd(&bad, P(A), P(A + 0x200), P(A + 0x500), P(A + 0x600), big, P(A + 0x700), big),
         BLK_EINVAL);
  /* four-wave weight-gradient operands of 4 GiB or more */
  bad = c; bad.B = 1; bad.T = 209716; bad.dtype = BLK_F32;
  expect("fwd f32 4 GiB operand", fwd(&bad, P(A), P(A + 0x200), P(A + 0x500), P(A + 0x600), big, P(A + 0x700), big),
         BLK_EUNSUPPORTED);
  bad.T = 209715;
  expect("f32 below 4 GiB", block_saved_bytes(&bad) > 0, 1);
  bad = c; bad.B = 1; bad.T = 419431;
  expect("bf16 ragged 4 GiB operand", (int)block_scratch_bytes(&bad), 0);

  /* block_bwd */
  expect("bwd null saved", bwd(&c, NULL, big, P(A + 0x800), (float*)P(A), 0, P(A), big), BLK_EINVAL);
  expect("bwd null dw", bwd(&c, P(A), big, P(A + 0x800), NULL, 0, P(A), big), BLK_EINVAL);
  expect("bwd accumulate 2", bwd(&c, P(A), big, P(A + 0x800), (float*)P(A), 2, P(A), big), BLK_EINVAL);
  expect("bwd misaligned dx", bwd(&c, P(A), big, P(MIS), (float*)P(A), 0, P(A), big), BLK_EALIGN);
  expect("bwd short scratch", bwd(&c, P(A), big, P(A + 0x800), (float*)P(A), 0, P(A), 100), BLK_ENOSPC);
  expect("bwd short saved", bwd(&c, P(A), 100, P(A + 0x800), (float*)P(A), 0, P(A), big), BLK_ENOSPC);

  /* decode_step */
  blk_dcfg d;
  memset(&d, 0, sizeof d);
  d.B = 64; d.C = 1280; d.H = 10; d.D = 128; d.F = 5120; d.S_max = 2049; d.eps = 1e-6f; d.rope_base = 10000.f;
  d.dtype = BLK_BF16;
  const size_t dneed = decode_scratch_bytes(&d);
  expect("decode scratch nonzero", dneed > 0, 1);
  expect("decode null cfg", (int)decode_scratch_bytes(NULL), 0);
  expect("decode null x", decode_step(&d, NULL, P(A), P(A), P(A), P(A), P(A + 0x100), P(A + 0x200), (int32_t*)P(A),
                                      NULL, P(A), P(A), big, 0), BLK_EINVAL);
  expect("decode caches alias", decode_step(&d, P(A), P(A), P(A), P(A), P(A), P(A + 0x100), P(A + 0x100),
                                            (int32_t*)P(A), NULL, P(A), P(A), big, 0), BLK_EINVAL);
  expect("decode misaligned len", decode_step(&d, P(A), P(A), P(A), P(A), P(A), P(A + 0x100), P(A + 0x200),
                                              (int32_t*)P(A + 2), NULL, P(A), P(A), big, 0), BLK_EALIGN);
  expect("decode short scratch", decode_step(&d, P(A), P(A), P(A), P(A), P(A), P(A + 0x100), P(A + 0x200),
                                             (int32_t*)P(A), NULL, P(A), P(A), dneed - 1, 0), BLK_ENOSPC);
  expect("decode misaligned status", decode_step(&d, P(A), P(A), P(A), P(A), P(A), P(A + 0x100), P(A + 0x200),
                                                 (int32_t*)P(A), (int32_t*)P(A + 6), P(A), P(A), big, 0), BLK_EALIGN);
  blk_dcfg dbad = d;
  dbad.dtype = BLK_F32;
  expect("decode f32", decode_step(&dbad, P(A), P(A), P(A), P(A), P(A), P(A + 0x100), P(A + 0x200), (int32_t*)P(A), NULL,
                                   P(A), P(A), big, 0), BLK_EUNSUPPORTED);

  /* head */
  blk_hcfg h;
  memset(&h, 0, sizeof h);
  h.N = 65536; h.C = 1280; h.V = 65536; h.eps = 1e-6f; h.dtype = BLK_BF16;
  expect("head scratch nonzero", head_scratch_bytes(&h) > 0, 1);
  blk_hcfg hb = h;
  hb.V = 1000;
  expect("head V", (int)head_scratch_bytes(&hb), 0);
  expect("head fwd null targets", head_loss_fwd(&h, P(A), P(A), NULL, (float*)P(A), (float*)P(A), P(A), big, 0),
         BLK_EINVAL);
  expect("head fwd short scratch", head_loss_fwd(&h, P(A), P(A), (int32_t*)P(A), (float*)P(A), (float*)P(A), P(A),
                                                 4096, 0), BLK_ENOSPC);
  expect("head bwd dx aliases x", head_loss_bwd(&h, P(A), P(A), (int32_t*)P(A), (float*)P(A), 1.f, P(A),
                                                (float*)P(A), 0, P(A), big, 0), BLK_EINVAL);
  expect("head bwd accumulate 2", head_loss_bwd(&h, P(A), P(A), (int32_t*)P(A), (float*)P(A), 1.f, P(A + 0x100),
                                                (float*)P(A), 2, P(A), big, 0), BLK_EINVAL);

  /* fp8 quantiser */
  expect("quantize n", block_fp8_quantize(P(A), 7, P(A), (uint32_t*)P(A), 0), BLK_EINVAL);
  expect("quantize null", block_fp8_quantize(NULL, 8, P(A), (uint32_t*)P(A), 0), BLK_EINVAL);
  expect("quantize_2d ldt", block_fp8_quantize_2d(P(A), 300, 384, P(A), P(A), 299, (uint32_t*)P(A), 0), BLK_EINVAL);
  expect("quantize_2d align", block_fp8_quantize_2d(P(MIS), 300, 384, P(A), P(A), 320, (uint32_t*)P(A), 0),
         BLK_EALIGN);

  /* strings */
  for (int code = 0; code < 8; ++code) expect("strerror", block_strerror(code) != NULL, 1);

  if (failures) return 1;
  printf("abi checks passed under the host sanitizers\n");
  return 0;
}
