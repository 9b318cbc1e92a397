/* Host-side AddressSanitizer run of the C ABI (no GPU needed): argument checks over
 * a grid of valid and invalid values, every entry point with a NULL handle, gemm_create (with
 * no device present it must fail and leave the handle NULL), and every status string. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include "gemm.h"

#define P(x) ((void*)(uintptr_t)(x))

int main(void) {
  long calls = 0, ok = 0;
  for (int s = -40; s <= 40; ++s) { const char* t = gemm_status_string((gemm_status_t)s); calls++; if (t && strlen(t)) ok++; }
  const int64_t dims[] = {0, 1, 7, 1000, 4096, -1, (int64_t)1 << 31, (int64_t)1 << 40};
  const int types[] = {GEMM_F32, GEMM_F16, GEMM_BF16, GEMM_E4M3, GEMM_E5M2, GEMM_E2M1, GEMM_E2M3, GEMM_E3M2, 99, -1};
  const uint32_t epis[] = {0, GEMM_EPI_BIAS, GEMM_EPI_GELU, GEMM_EPI_BIAS | GEMM_EPI_GELU, 0xFFFFFFFFu};
  for (int im = 0; im < 8; ++im) for (int in = 0; in < 8; ++in) for (int ik = 0; ik < 8; ++ik)
    for (int t = 0; t < 4; ++t) for (int ia = 0; ia < 10; ++ia) for (int ic = 0; ic < 10; ic += 3)
      for (int ie = 0; ie < 5; ++ie) {
        const int64_t M = dims[im], N = dims[in], K = dims[ik];
        const int ta = t & 1, tb = t >> 1;
        const int64_t lda = ta ? M : K, ldb = tb ? K : N, ldc = N;
        const float* bias = (ie & 1) ? (const float*)P(0x900000) : NULL;
        int st = gemm_check_args(M, N, K, ta, tb, P(0x100000), lda, P(0x200000), ldb, P(0x300000), ldc,
                                 (gemm_dtype_t)types[ia], (gemm_dtype_t)types[ia], (gemm_dtype_t)types[ic], epis[ie], bias);
        calls++; ok += (st == GEMM_OK);
        st = gemm_check_args(M, N, K, ta, tb, NULL, lda - 1, P(0x300000), ldb, P(0x300000), ldc - 1,
                             (gemm_dtype_t)types[ia], (gemm_dtype_t)types[ia], (gemm_dtype_t)types[ic], epis[ie], NULL);
        calls++;
        st = gemm_check_args_mx(M, N, K, ta, tb, P(0x100000), lda, P(0x400000), K / 32, P(0x200000), ldb,
                                P(0x500000), K / 32, P(0x300000), ldc, (gemm_dtype_t)types[ia],
                                (gemm_dtype_t)types[ia], (gemm_dtype_t)types[ic], epis[ie], bias);
        calls++; ok += (st == GEMM_OK);
      }
  const int bits[] = {3, 4, 8, 0};
  const int64_t groups[] = {0, 7, 16, 32, 64, 128, -64};
  for (int im = 0; im < 8; ++im) for (int in = 0; in < 8; ++in) for (int ik = 0; ik < 8; ++ik)
    for (int ib = 0; ib < 4; ++ib) for (int ig = 0; ig < 7; ++ig) for (int ix = 0; ix < 4; ++ix) {
      const int64_t M = dims[im], N = dims[in], K = dims[ik], G = groups[ig];
      const int64_t ldg = G > 0 ? K / G : 0;
      int st = gemm_check_args_q(M, N, K, P(0x100000), K, (const uint8_t*)P(0x200000), K * bits[ib] / 8,
                                 bits[ib], G, P(0x300000), P(0x400000), ldg, P(0x500000), N,
                                 (gemm_dtype_t)types[ix], GEMM_EPI_BIAS | GEMM_EPI_GELU,
                                 (const float*)P(0x600000));
      calls++; ok += (st == GEMM_OK);
    }
  /* no handle */
  int e = 0;
  e |= gemm_run(NULL, NULL, 8, 8, 8, 0, 0, 1.f, P(16), 8, 1.f, P(16), 8, 1.f, 0.f, P(4096), 8, GEMM_F32, GEMM_F32, GEMM_F32, 0, NULL) != GEMM_ERR_INVALID_HANDLE;
  e |= gemm_run_kernel(NULL, GEMM_KERNEL_MFMA_256, NULL, 8, 8, 8, 0, 0, 1.f, P(16), 8, 1.f, P(16), 8, 1.f, 0.f, P(4096), 8, GEMM_F32, GEMM_F32, GEMM_F32, 0, NULL) != GEMM_ERR_INVALID_HANDLE;
  e |= gemm_run_ws(NULL, NULL, 8, 8, 8, 0, 0, 1.f, P(16), 8, 1.f, P(16), 8, 1.f, 0.f, P(4096), 8, GEMM_F16, GEMM_F16, GEMM_F16, 0, NULL, P(8192), 256) != GEMM_ERR_INVALID_HANDLE;
  e |= gemm_run_ws_kernel(NULL, GEMM_KERNEL_MFMA_256_SK, NULL, 8, 8, 8, 0, 0, 1.f, P(16), 8, 1.f, P(16), 8, 1.f, 0.f, P(4096), 8, GEMM_F16, GEMM_F16, GEMM_F16, 0, NULL, P(8192), 256) != GEMM_ERR_INVALID_HANDLE;
  e |= gemm_run_noalloc(NULL, GEMM_KERNEL_MFMA_256x128_SK2, NULL, 8, 8, 8, 0, 0, 1.f, P(16), 8, 1.f, P(16), 8, 1.f, 0.f, P(4096), 8, GEMM_F16, GEMM_F16, GEMM_F16, 0, NULL) != GEMM_ERR_INVALID_HANDLE;
  e |= gemm_workspace_bytes(NULL, 8, 8, 8, 0, 0, P(16), 8, P(16), 8, P(4096), 8, GEMM_F16, GEMM_F16, GEMM_F16, 0, NULL) != GEMM_ERR_INVALID_HANDLE;
  e |= gemm_kernel_workspace_bytes(NULL, GEMM_KERNEL_MFMA_256_SK, 512, 512) != GEMM_ERR_INVALID_HANDLE;
  e |= gemm_run_mx(NULL, NULL, 32, 32, 32, 0, 0, 1.f, P(16), 32, P(16), 1, P(16), 32, P(16), 1, 0.f, P(4096), 32, GEMM_E4M3, GEMM_E4M3, GEMM_BF16, 0, NULL) != GEMM_ERR_INVALID_HANDLE;
  e |= gemm_run_mx_kernel(NULL, GEMM_KERNEL_MFMA_64, NULL, 32, 32, 32, 0, 0, 1.f, P(16), 32, P(16), 1, P(16), 32, P(16), 1, 0.f, P(4096), 32, GEMM_E4M3, GEMM_E4M3, GEMM_BF16, 0, NULL) != GEMM_ERR_INVALID_HANDLE;
  e |= gemm_select_kernel(NULL, 8, 8, 8, 0, 0, P(16), 8, P(16), 8, P(4096), 8, GEMM_F32, GEMM_F32, GEMM_F32, 0, NULL) != GEMM_ERR_INVALID_HANDLE;
  e |= gemm_bias_gelu(NULL, NULL, 8, 8, P(4096), 8, GEMM_BF16, (const float*)P(16), GEMM_EPI_BIAS) != GEMM_ERR_INVALID_HANDLE;
  e |= gemm_run_q(NULL, NULL, 1, 64, 64, 1.f, P(16), 64, (const uint8_t*)P(16), 32, 4, 64, P(16), P(16), 1, 0.f, P(4096), 64, GEMM_BF16, 0, NULL) != GEMM_ERR_INVALID_HANDLE;
  e |= gemm_run_q_kernel(NULL, GEMM_KERNEL_QGEMV, NULL, 1, 64, 64, 1.f, P(16), 64, (const uint8_t*)P(16), 32, 4, 64, P(16), P(16), 1, 0.f, P(4096), 64, GEMM_BF16, 0, NULL) != GEMM_ERR_INVALID_HANDLE;
  e |= gemm_select_kernel_q(NULL, 1, 64, 64, P(16), 64, (const uint8_t*)P(16), 32, 4, 64, P(16), P(16), 1, P(4096), 64, GEMM_BF16, 0, NULL) != GEMM_ERR_INVALID_HANDLE;
  e |= gemm_probe_clock(NULL, NULL, (uint64_t*)P(4096), 256, 40) != GEMM_ERR_INVALID_HANDLE;
  e |= gemm_wall_clock_khz(NULL) != GEMM_ERR_INVALID_HANDLE;
  e |= gemm_probe_bandwidth(NULL, NULL, P(4096), NULL, 1 << 20, P(8192)) != GEMM_ERR_INVALID_HANDLE;
  e |= gemm_destroy(NULL) != GEMM_OK;
  calls += 18;
  /* without a GPU, gemm_create must fail cleanly */
  gemm_handle_t h = (gemm_handle_t)P(1);
  const int cst = gemm_create(&h, 0);
  if (cst == GEMM_OK) {  /* a machine with a gfx950 */
    e |= h == NULL;
    e |= gemm_destroy(h) != GEMM_OK;
  } else {
    e |= h != NULL;
  }
  e |= gemm_create(NULL, 0) != GEMM_ERR_INVALID_VALUE;
  calls += 2;
  printf("[asan] %ld calls, %ld argument sets valid, gemm_create without a GPU: %s, null-handle checks %s\n",
         calls, ok, gemm_status_string((gemm_status_t)cst), e ? "FAILED" : "ok");
  return e;
}
