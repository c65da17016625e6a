/* A plain C99 program that uses the library through include/abg.h alone (no
 * Python, no torch): checks the version, the status names and that invalid
 * requests are rejected on the host with their status code and a message.
 * Every call here fails validation, so it runs without a GPU. */
#include "abg.h"

#include <stdint.h>
#include <stdio.h>
#include <string.h>

static int failures = 0;

static void expect(int cond, const char* what) {
  if (!cond) {
    fprintf(stderr, "FAIL: %s\n", what);
    ++failures;
  }
}

int main(void) {
  /* Distinct, aligned stand-ins for device addresses; validation never
   * dereferences them. */
  const void* q = (const void*)(uintptr_t)0x100000000ull;
  const void* k = (const void*)(uintptr_t)0x200000000ull;
  const void* v = (const void*)(uintptr_t)0x300000000ull;
  const float* bias = (const float*)(uintptr_t)0x400000000ull;
  void* out = (void*)(uintptr_t)0x500000000ull;
  const void* weight = (const void*)(uintptr_t)0x600000000ull;
  abg_status st;

  expect(abg_abi_version() == ABG_ABI_VERSION, "abi version");
  expect(strcmp(abg_status_string(ABG_OK), "ABG_OK") == 0, "status name");
  /* The status codes are part of the ABI: the first seven keep the values
   * of the library's first contract, ABG_ERR_ALIAS was appended after them. */
  expect(ABG_ERR_NULL == 1 && ABG_ERR_SHAPE == 2 && ABG_ERR_UNSUPPORTED == 3 &&
             ABG_ERR_ALIGN == 4 && ABG_ERR_VALUE == 5 && ABG_ERR_DEVICE == 6 &&
             ABG_ERR_ALIAS == 7,
         "status code values");
  expect(strcmp(abg_status_string(6), "ABG_ERR_DEVICE") == 0, "code 6 is ABG_ERR_DEVICE");

  /* Eight query heads are required. */
  st = abg_biased_mqa_fwd(q, k, v, bias, out, 1, 8192, 4, 128, 128, 0, 1,
                          0.088f, 5.0f, ABG_BF16, NULL);
  expect(st != ABG_OK, "Hq = 4 rejected");
  expect(strlen(abg_last_error()) > 0, "message after a rejection");

  /* A null query pointer. */
  st = abg_biased_mqa_fwd(NULL, k, v, bias, out, 1, 8192, 8, 128, 128, 0, 1,
                          0.088f, 5.0f, ABG_BF16, NULL);
  expect(st == ABG_ERR_NULL, "null q");

  /* The output overlapping an input. */
  st = abg_biased_mqa_fwd(q, k, v, bias, (void*)q, 1, 8192, 8, 128, 128, 0, 1,
                          0.088f, 5.0f, ABG_BF16, NULL);
  expect(st == ABG_ERR_ALIAS, "out overlapping q");

  /* The projection needs C % 8 == 0. */
  st = abg_pair_bias_project(q, weight, (float*)out, 1, 512, 127, 8, ABG_BF16, NULL);
  expect(st == ABG_ERR_SHAPE || st == ABG_ERR_UNSUPPORTED, "C = 127 rejected");

  /* The fused pair form needs C == 128. */
  st = abg_pair_biased_mqa_fwd(q, k, v, bias, weight, out, NULL, 0, 1, 8192, 8192, 0,
                               8, 128, 128, 64, 0, 1, 1, 0.088f, 5.0f, ABG_BF16,
                               NULL);
  expect(st != ABG_OK, "pair form with C = 64 rejected");

  if (failures == 0) printf("c consumer ok\n");
  return failures == 0 ? 0 : 1;
}
