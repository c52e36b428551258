/*
 * c_abi_caller.c -- a plain C11 caller of the decode library's C ABI
 * (include/fd.h): no C++ and no Python between the caller and libfd.so.
 * Test infrastructure, driven by tests/test_c_abi.py.
 *
 *   c_abi_caller host
 *       The planner, the status strings and the argument checks, all of
 *       which answer before the library touches a GPU.  Prints one
 *       "name value" line per check and exits 0 when every check holds.
 *   c_abi_caller run IN OUT
 *       Reads a problem from IN and decodes it on device 0 twice --
 *       fd_decode (library workspace) and fd_decode_ex (a workspace this
 *       program allocates, with IN's split count) -- then writes both
 *       results to OUT.
 *
 * IN (little-endian): int32 B, Hq, Hkv, D, Lmax, num_splits, has_seqlens;
 * float32 scale; bf16 q[B][Hq][D]; bf16 k[B][Hkv][Lmax][D]; bf16 v, the
 * same; int32 seqlens[B] when has_seqlens.
 * OUT: int32 status of fd_decode, of fd_decode_ex, of fd_decode_ex with a
 * workspace one byte too small (1 when the plan needs none), and 1 if
 * fd_plan's workspace size equals fd_workspace_bytes' (else 0); then bf16
 * out[B][Hq][D] and float32
 * lse[B][Hq] of fd_decode, then those of fd_decode_ex.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "fd.h"

static int failures = 0;

/* A HIP runtime call that must succeed in run mode. */
#define HIP_OK(call)                                                  \
  do {                                                                \
    if ((call) != hipSuccess) {                                       \
      fprintf(stderr, "%s failed at line %d\n", #call, __LINE__);     \
      return 3;                                                       \
    }                                                                 \
  } while (0)

static void check(const char *name, long got, long want) {
  printf("%s %ld%s\n", name, got, got == want ? "" : "  MISMATCH");
  if (got != want) ++failures;
}

static int host_checks(void) {
  /* placeholder device addresses: every call below fails validation
     before the library would dereference or hand them to HIP */
  void *p = (void *)(uintptr_t)0x100000;
  float *pl = (float *)p;
  fd_plan_t plan;

  check("version_positive", fd_version() > 0, 1);
  check("status_ok_text", fd_status_string(FD_OK) != NULL &&
                              strlen(fd_status_string(FD_OK)) > 0, 1);
  check("status_unknown_text", fd_status_string(-999) != NULL, 1);

  /* batch 1, 64k keys, 64 query heads on 8 KV heads, 256 compute units */
  check("plan_rc", fd_plan(1, 64, 8, 128, 65536, FD_BF16, 0, 0,
                           FD_VARIANT_AUTO, 0, 256, &plan), FD_OK);
  check("plan_splits", plan.num_splits, 32);
  check("plan_chunk", plan.chunk, 2048);
  check("plan_grid", plan.grid, 256);
  check("plan_variant", plan.variant, FD_VARIANT_MFMA);
  check("plan_merge", plan.merge, FD_MERGE_SEPARATE);
  check("plan_workspace", (long)plan.workspace_bytes,
        (long)(64 * 32 * 128 * 4 + 64 * 32 * 4));
  /* 64 sequences of 4k keys fill the chip without splitting */
  check("plan_b64_rc", fd_plan(64, 32, 8, 128, 4096, FD_BF16, 0, 0,
                               FD_VARIANT_AUTO, 0, 256, &plan), FD_OK);
  check("plan_b64_splits", plan.num_splits, 1);
  check("plan_b64_merge", plan.merge, FD_MERGE_NONE);
  check("plan_b64_workspace", (long)plan.workspace_bytes, 0);

  check("plan_group_not_dividing",
        fd_plan(1, 6, 4, 128, 1024, FD_BF16, 0, 0, 0, 0, 256, &plan),
        FD_ERR_INVALID_ARG);
  check("plan_head_dim_96",
        fd_plan(1, 8, 8, 96, 1024, FD_BF16, 0, 0, 0, 0, 256, &plan),
        FD_ERR_UNSUPPORTED);
  check("plan_bad_dtype",
        fd_plan(1, 8, 8, 128, 1024, (fd_dtype_t)7, 0, 0, 0, 0, 256, &plan),
        FD_ERR_UNSUPPORTED);
  check("plan_unknown_flag",
        fd_plan(1, 8, 8, 128, 1024, FD_BF16, 0, 0, 0, 1 << 20, 256, &plan),
        FD_ERR_INVALID_ARG);

  check("decode_null_q",
        fd_decode(NULL, p, p, NULL, 1, 8, 8, 128, 1024, 0.1f, FD_BF16, p, pl,
                  NULL),
        FD_ERR_INVALID_ARG);
  check("decode_misaligned_k",
        fd_decode(p, (char *)p + 2, p, NULL, 1, 8, 8, 128, 1024, 0.1f,
                  FD_BF16, p, pl, NULL),
        FD_ERR_INVALID_ARG);
  check("decode_nan_scale",
        fd_decode(p, p, p, NULL, 1, 8, 8, 128, 1024, nanf(""), FD_BF16, p,
                  pl, NULL),
        FD_ERR_INVALID_ARG);
  check("decode_zero_batch",
        fd_decode(p, p, p, NULL, 0, 8, 8, 128, 1024, 0.1f, FD_BF16, p, pl,
                  NULL),
        FD_ERR_INVALID_ARG);
  check("decode_ex_bytes_without_workspace",
        fd_decode_ex(p, p, p, NULL, 1, 8, 8, 128, 1024, 0.1f, FD_BF16, p, pl,
                     0, FD_VARIANT_AUTO, 0, NULL, 64, NULL),
        FD_ERR_INVALID_ARG);
  check("decode_ex_negative_splits",
        fd_decode_ex(p, p, p, NULL, 1, 8, 8, 128, 1024, 0.1f, FD_BF16, p, pl,
                     -1, FD_VARIANT_AUTO, 0, NULL, 0, NULL),
        FD_ERR_INVALID_ARG);
  return failures == 0 ? 0 : 1;
}

static int read_all(FILE *f, void *dst, size_t bytes) {
  return fread(dst, 1, bytes, f) == bytes;
}

static int run_case(const char *in_path, const char *out_path) {
  FILE *f = fopen(in_path, "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", in_path);
    return 2;
  }
  int32_t hdr[7];
  float scale;
  if (!read_all(f, hdr, sizeof hdr) || !read_all(f, &scale, sizeof scale)) {
    fprintf(stderr, "short header\n");
    fclose(f);
    return 2;
  }
  const int B = hdr[0], Hq = hdr[1], Hkv = hdr[2], D = hdr[3], Lmax = hdr[4];
  const int splits = hdr[5], has_sl = hdr[6];
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Lmax <= 0) {
    fprintf(stderr, "bad sizes\n");
    fclose(f);
    return 2;
  }
  const size_t nq = (size_t)B * Hq * D, nkv = (size_t)B * Hkv * Lmax * D;
  const size_t nlse = (size_t)B * Hq;
  uint16_t *hq = malloc(nq * 2), *hk = malloc(nkv * 2), *hv = malloc(nkv * 2);
  uint16_t *hout = malloc(nq * 2);
  float *hlse = malloc(nlse * 4);
  int32_t *hsl = malloc((size_t)B * 4);
  if (!hq || !hk || !hv || !hout || !hlse || !hsl) {
    fprintf(stderr, "out of host memory\n");
    fclose(f);
    return 2;
  }
  int ok = read_all(f, hq, nq * 2) && read_all(f, hk, nkv * 2) &&
           read_all(f, hv, nkv * 2) &&
           (!has_sl || read_all(f, hsl, (size_t)B * 4));
  fclose(f);
  if (!ok) {
    fprintf(stderr, "short input\n");
    return 2;
  }

  if (hipSetDevice(0) != hipSuccess) {
    fprintf(stderr, "no HIP device\n");
    return 3;
  }
  void *dq, *dk, *dv, *dout, *dws = NULL;
  float *dlse;
  int32_t *dsl = NULL;
  hipStream_t st;
  if (hipMalloc(&dq, nq * 2) != hipSuccess ||
      hipMalloc(&dk, nkv * 2) != hipSuccess ||
      hipMalloc(&dv, nkv * 2) != hipSuccess ||
      hipMalloc(&dout, nq * 2) != hipSuccess ||
      hipMalloc((void **)&dlse, nlse * 4) != hipSuccess ||
      (has_sl && hipMalloc((void **)&dsl, (size_t)B * 4) != hipSuccess) ||
      hipStreamCreate(&st) != hipSuccess) {
    fprintf(stderr, "device allocation failed\n");
    return 3;
  }
  HIP_OK(hipMemcpy(dq, hq, nq * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dk, hk, nkv * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dv, hv, nkv * 2, hipMemcpyHostToDevice));
  if (has_sl)
    HIP_OK(hipMemcpy(dsl, hsl, (size_t)B * 4, hipMemcpyHostToDevice));

  FILE *o = fopen(out_path, "wb");
  if (!o) {
    fprintf(stderr, "cannot open %s\n", out_path);
    return 2;
  }
  int32_t status[4];
  status[0] = fd_decode(dq, dk, dv, dsl, B, Hq, Hkv, D, Lmax, scale, FD_BF16,
                        dout, dlse, st);
  HIP_OK(hipStreamSynchronize(st));
  HIP_OK(hipMemcpy(hout, dout, nq * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hlse, dlse, nlse * 4, hipMemcpyDeviceToHost));

  fd_plan_t plan;
  const size_t ws = fd_workspace_bytes(B, Hq, Hkv, D, Lmax, FD_BF16, has_sl,
                                       splits, FD_VARIANT_AUTO, 0);
  const int prc = fd_plan(B, Hq, Hkv, D, Lmax, FD_BF16, has_sl, splits,
                          FD_VARIANT_AUTO, 0, 0, &plan);
  status[3] = prc == FD_OK && plan.workspace_bytes == ws;
  if (ws && hipMalloc(&dws, ws) != hipSuccess) {
    fprintf(stderr, "workspace allocation failed\n");
    return 3;
  }
  status[2] = ws ? fd_decode_ex(dq, dk, dv, dsl, B, Hq, Hkv, D, Lmax, scale,
                                FD_BF16, dout, dlse, splits, FD_VARIANT_AUTO,
                                0, dws, ws - 1, st)
                 : 1; /* the plan needs no workspace */
  status[1] = fd_decode_ex(dq, dk, dv, dsl, B, Hq, Hkv, D, Lmax, scale,
                           FD_BF16, dout, dlse, splits, FD_VARIANT_AUTO, 0,
                           dws, ws, st);
  HIP_OK(hipStreamSynchronize(st));
  fwrite(status, 4, 4, o);
  fwrite(hout, 2, nq, o);
  fwrite(hlse, 4, nlse, o);
  HIP_OK(hipMemcpy(hout, dout, nq * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hlse, dlse, nlse * 4, hipMemcpyDeviceToHost));
  fwrite(hout, 2, nq, o);
  fwrite(hlse, 4, nlse, o);
  fclose(o);

  hipFree(dq);
  hipFree(dk);
  hipFree(dv);
  hipFree(dout);
  hipFree(dlse);
  if (dsl) hipFree(dsl);
  if (dws) hipFree(dws);
  hipStreamDestroy(st);
  free(hq);
  free(hk);
  free(hv);
  free(hout);
  free(hlse);
  free(hsl);
  printf("decode %d decode_ex %d small_workspace %d workspace_size_agrees %d\n",
         status[0], status[1], status[2], status[3]);
  return 0;
}

int main(int argc, char **argv) {
  if (argc == 2 && strcmp(argv[1], "host") == 0) return host_checks();
  if (argc == 4 && strcmp(argv[1], "run") == 0)
    return run_case(argv[2], argv[3]);
  fprintf(stderr, "usage: %s host | run IN OUT\n", argv[0]);
  return 2;
}
