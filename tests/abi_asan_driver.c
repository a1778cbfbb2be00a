/*
 * Host-side driver for the address-sanitized build of the C ABI's argument
 * checks (tests/test_abi_asan.py). Every call here is answered by the
 * validation and workspace arithmetic before any HIP launch, so it runs
 * without a GPU; the ABI layer itself is compiled with AddressSanitizer on
 * the host side. Each expected status is checked; the program prints one
 * summary line and exits non-zero on a mismatch (ASan aborts on a bad access).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../include/engram.h"

static int g_fail = 0, g_checks = 0;

static void expect(int got, int want, const char* what) {
  ++g_checks;
  if (got != want) {
    printf("FAIL %s: got %d want %d\n", what, got, want);
    ++g_fail;
  }
}

static void expect_sz(size_t got, size_t want, const char* what) {
  ++g_checks;
  if (got != want) {
    printf("FAIL %s: got %zu want %zu\n", what, got, want);
    ++g_fail;
  }
}

int main(void) {
  /* heap blocks standing in for device buffers: never dereferenced by the
     checks, only compared, aligned-tested and passed through */
  char* base = (char*)aligned_alloc(256, 1 << 16);
  void* p16 = base + 256;
  void* mis = base + 258; /* 2 bytes off a 16-byte boundary */
  uint8_t* u8 = (uint8_t*)(base + 512);
  int32_t* ids = (int32_t*)(base + 1024);
  float* part = (float*)(base + 2048);
  const int OK = ENGRAM_OK, INV = ENGRAM_EINVAL, UNS = ENGRAM_EUNSUPPORTED;

  expect(engram_abi_version(), ENGRAM_ABI_VERSION, "abi version");
  for (int s = -1; s < 8; ++s) {
    const char* t = engram_status_string(s);
    ++g_checks;
    if (!t || !*t) { printf("FAIL status string %d\n", s); ++g_fail; }
  }

  /* lookup (and its background form): T = 0 no-op, bad sizes, NULLs, alignment */
  expect(engram_lookup(NULL, 10, 128, NULL, 16, 1, 0, 16, NULL, NULL, NULL), OK, "lookup T=0");
  expect(engram_lookup(p16, 10, 128, ids, 16, 1, -1, 16, p16, NULL, NULL), INV, "lookup T<0");
  expect(engram_lookup(p16, 10, 12, ids, 16, 1, 4, 16, p16, NULL, NULL), UNS, "lookup hd%8");
  expect(engram_lookup(p16, 10, 2048, ids, 16, 1, 4, 16, p16, NULL, NULL), UNS, "lookup hd>1024");
  expect(engram_lookup(NULL, 10, 128, ids, 16, 1, 4, 16, p16, NULL, NULL), INV, "lookup NULL table");
  expect(engram_lookup(mis, 10, 128, ids, 16, 1, 4, 16, p16, NULL, NULL), INV, "lookup misaligned");
  expect(engram_lookup(p16, 10, 128, ids, -16, 1, 4, 16, p16, NULL, NULL), INV, "lookup negative stride");
  expect(engram_lookup(p16, -1, 128, ids, 16, 1, 4, 16, p16, NULL, NULL), INV, "lookup negative rows");
  expect(engram_lookup(p16, 10, 128, ids, 16, 1, 4, 0, p16, NULL, NULL), INV, "lookup no columns");
  expect(engram_lookup_background(NULL, 10, 128, NULL, 16, 1, 0, 16, NULL, NULL, NULL), OK, "bg T=0");
  expect(engram_lookup_background(p16, 10, 12, ids, 16, 1, 4, 16, p16, NULL, NULL), UNS, "bg hd%8");
  expect(engram_lookup_background(p16, 10, 128, (const int32_t*)(base + 1026), 16, 1, 4, 16, p16, NULL, NULL),
         INV, "bg misaligned ids");
  expect(engram_lookup_fp8(p16, u8, 10, 72, ids, 16, 1, 4, 16, p16, NULL, NULL), UNS, "fp8 hd%32");
  expect(engram_lookup_fp8(p16, NULL, 10, 128, ids, 16, 1, 4, 16, p16, NULL, NULL), INV, "fp8 NULL scales");

  /* MX quantize */
  expect(engram_mx_quantize(NULL, 0, 2048, NULL, NULL, NULL), OK, "mxq T=0");
  expect(engram_mx_quantize(p16, 4, 100, u8, u8, NULL), UNS, "mxq K%32");
  expect(engram_mx_quantize(p16, 4, 0, u8, u8, NULL), INV, "mxq K=0");
  expect(engram_mx_quantize(mis, 4, 64, u8, u8, NULL), INV, "mxq misaligned");

  /* wkv */
  expect_sz(engram_wkv_workspace_size(0, 2048, 20480, ENGRAM_W_MXFP8), 0, "wkv ws T=0");
  expect_sz(engram_wkv_workspace_size(16, 2048, 20480, ENGRAM_W_BF16), 0, "wkv ws bf16");
  expect_sz(engram_wkv_workspace_size(16, 2048, 20480, ENGRAM_W_MXFP8), 32768 + 1024, "wkv ws mxfp8");
  expect(engram_wkv(NULL, 0, 2048, NULL, NULL, ENGRAM_W_BF16, 20480, NULL, NULL, 0, NULL), OK, "wkv T=0");
  expect(engram_wkv(p16, 4, 100, p16, NULL, ENGRAM_W_BF16, 64, p16, NULL, 0, NULL), UNS, "wkv K%8");
  expect(engram_wkv(p16, 4, 256, p16, NULL, ENGRAM_W_BF16, 66, p16, NULL, 0, NULL), UNS, "wkv N%4");
  expect(engram_wkv(p16, 4, 256, p16, NULL, ENGRAM_W_MXFP8, 64, p16, p16, 1 << 12, NULL), INV, "wkv mx NULL scales");
  expect(engram_wkv(p16, 4, 200, p16, u8, ENGRAM_W_MXFP8, 64, p16, p16, 1 << 12, NULL), UNS, "wkv mx K%128");
  expect(engram_wkv(p16, 4, 256, p16, u8, 7, 64, p16, NULL, 0, NULL), INV, "wkv bad format");
  expect(engram_wkv(p16, 4, 1 << 21, p16, NULL, ENGRAM_W_BF16, 64, p16, NULL, 0, NULL), UNS, "wkv K too large");
  expect(engram_wkv(p16, 64, 256, p16, u8, ENGRAM_W_MXFP8, 64, p16, p16, 16, NULL), INV, "wkv short workspace");

  /* gate, gate finish, partials */
  expect(engram_gate(NULL, NULL, NULL, NULL, NULL, 0, 4, 4096, 1e-6f, 1e-6f, NULL, NULL, NULL), OK, "gate T=0");
  expect(engram_gate(p16, p16, p16, p16, NULL, 4, 4, 4100, 1e-6f, 1e-6f, p16, NULL, NULL), UNS, "gate dim%8");
  expect(engram_gate(p16, p16, p16, p16, NULL, 4, 9, 4096, 1e-6f, 1e-6f, p16, NULL, NULL), UNS, "gate hc>8");
  expect(engram_gate(p16, p16, p16, p16, NULL, 4, 0, 4096, 1e-6f, 1e-6f, p16, NULL, NULL), INV, "gate hc=0");
  expect(engram_gate(p16, NULL, p16, p16, NULL, 4, 4, 4096, 1e-6f, 1e-6f, p16, NULL, NULL), INV, "gate NULL kv");
  expect(engram_gate(mis, p16, p16, p16, NULL, 4, 4, 4096, 1e-6f, 1e-6f, p16, NULL, NULL), INV, "gate misaligned");
  expect(engram_gate(p16, p16, p16, p16, NULL, 4, 4, 32768, 1e-6f, 1e-6f, p16, NULL, NULL), UNS, "gate dim>16384");
  expect(engram_gate_finish(p16, p16, part, NULL, 4, 4, 4000, 1e-6f, 1e-6f, p16, NULL, NULL), UNS, "finish dim%256");
  expect(engram_gate_finish(p16, p16, NULL, NULL, 4, 4, 4096, 1e-6f, 1e-6f, p16, NULL, NULL), INV, "finish NULL partials");
  expect(engram_gate_finish(p16, p16, (const float*)(base + 2052), NULL, 4, 4, 4096, 1e-6f, 1e-6f, p16, NULL, NULL),
         INV, "finish misaligned partials");
  expect(engram_gate_finish(NULL, NULL, NULL, NULL, 0, 4, 4096, 1e-6f, 1e-6f, NULL, NULL, NULL), OK, "finish T=0");
  expect(engram_wkv_gate_partials(p16, 4, 256, p16, NULL, ENGRAM_W_BF16, 4, 4000, p16, p16, p16, p16, part, NULL, 0,
                                  NULL), UNS, "partials dim%256");
  expect(engram_wkv_gate_partials(p16, 4, 256, p16, NULL, ENGRAM_W_BF16, 9, 256, p16, p16, p16, p16, part, NULL, 0,
                                  NULL), UNS, "partials hc>8");
  expect(engram_wkv_gate_partials(p16, 4, 256, p16, NULL, ENGRAM_W_BF16, 2, 256, p16, p16, p16, p16, NULL, NULL, 0,
                                  NULL), INV, "partials NULL partials");

  /* forward: argument struct checks, workspace sizes, options, no-alloc limit */
  engram_forward_args a;
  memset(&a, 0, sizeof(a));
  a.table = p16; a.num_rows = 100; a.hash_ids = ids; a.ids_stride_t = 16; a.ids_stride_c = 1;
  a.w = p16; a.w_scales = u8; a.w_format = ENGRAM_W_MXFP8;
  a.hidden = p16; a.q_weight = p16; a.k_weight = p16; a.out = p16;
  a.T = 16; a.hc = 4; a.dim = 4096; a.n_cols = 16; a.head_dim = 128; a.eps = 1e-6f; a.clamp = 1e-6f;
  const size_t ws = engram_forward_workspace_size(&a);
  ++g_checks;
  if (ws < 65536 + 16 * 2048 * 2 + 16 * 20480 * 2) { printf("FAIL forward workspace %zu\n", ws); ++g_fail; }
  expect(engram_forward(&a, NULL, ws, NULL), INV, "forward NULL workspace");
  expect(engram_forward(&a, p16, ws - 1, NULL), INV, "forward short workspace");
  expect(engram_forward(&a, base + 16, ws, NULL), INV, "forward misaligned workspace");
  a.options = 6;
  expect(engram_forward(&a, p16, ws, NULL), INV, "forward unknown options");
  a.options = 0;
  expect(engram_forward(NULL, p16, ws, NULL), INV, "forward NULL args");
  expect_sz(engram_forward_workspace_size(NULL), 0, "forward ws NULL");
  a.T = 0;
  expect_sz(engram_forward_workspace_size(&a), 0, "forward ws T=0");
  expect(engram_forward(&a, NULL, 0, NULL), OK, "forward T=0");
  expect(engram_forward_noalloc(&a, NULL), OK, "noalloc T=0");
  a.T = 16;
  a.dim = 4100;
  expect(engram_forward(&a, p16, 1u << 30, NULL), UNS, "forward dim%8");
  a.dim = 4096;
  a.n_cols = 1 << 20; a.head_dim = 1024;    /* K past 2^31 */
  expect(engram_forward(&a, p16, 1u << 30, NULL), UNS, "forward K too large");
  a.n_cols = 16; a.head_dim = 128;
  a.hc = 1 << 20;                            /* N past 2^31 */
  expect(engram_forward(&a, p16, 1u << 30, NULL), UNS, "forward N overflow");
  a.hc = 4;
  a.T = 100000;                              /* the no-alloc scratch is too small */
  expect(engram_forward_noalloc(&a, NULL), ENGRAM_ENOSPACE, "noalloc too large");
  a.T = 16;
  a.w_format = ENGRAM_W_BF16;
  a.w_scales = NULL;
  expect(engram_forward_single_launch(&a, p16, 1u << 30, NULL), UNS, "single launch bf16 wkv");

  /* host tables and probes: bad arguments answered before the runtime */
  void* h = base;
  void* d = base;
  expect(engram_host_alloc(0, &h, &d), INV, "host alloc 0 bytes");
  expect(engram_host_alloc(4096, NULL, &d), INV, "host alloc NULL host");
  expect(engram_host_alloc(4096, &h, NULL), INV, "host alloc NULL device");
  expect(engram_host_free(NULL), OK, "host free NULL");
  expect(engram_probe_mfma(7, 10, (float*)p16, NULL, NULL), INV, "probe mfma format");
  expect(engram_probe_mfma(ENGRAM_W_BF16, 0, (float*)p16, NULL, NULL), INV, "probe mfma iters");
  expect(engram_probe_read(p16, 100, (uint32_t*)p16, NULL), INV, "probe read size");
  expect(engram_probe_stream(p16, p16, 64, 5, NULL), INV, "probe stream ratio");
  expect(engram_probe_stream(p16, p16, 0, 1, NULL), OK, "probe stream empty");

  free(base);
  printf("abi checks under ASan: %d checks, %d failures\n", g_checks, g_fail);
  return g_fail ? 1 : 0;
}
