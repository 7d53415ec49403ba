/* The C ABI from C: the header compiles as strict C99, its structs have the
 * layout the Python binding mirrors, and the host-side entry points (sizes,
 * descriptors, validation that runs before any device access) behave as
 * documented.  Needs no GPU.  Prints "ok" and exits 0 on success. */
#include <stddef.h>
#include <stdio.h>

#include "qlora_nf4.h"

#define CHECK(x)                                                        \
  do {                                                                  \
    if (!(x)) {                                                         \
      printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #x);               \
      return 1;                                                         \
    }                                                                   \
  } while (0)

int main(void) {
  qlora_nf4_weight w;
  size_t a, b, c, d;

  CHECK(sizeof(qlora_nf4_weight) == 64);
  CHECK(offsetof(qlora_nf4_weight, dq_blocksize) == 8);
  CHECK(offsetof(qlora_nf4_weight, quant_type) == 12);
  CHECK(offsetof(qlora_nf4_weight, compute_dtype) == 14);
  CHECK(offsetof(qlora_nf4_weight, rows) == 16);
  CHECK(offsetof(qlora_nf4_weight, codes) == 32);
  CHECK(offsetof(qlora_nf4_weight, absmax_offset) == 56);
  CHECK(sizeof(qlora_dropout) == 24);
  CHECK(offsetof(qlora_dropout, seed) == 8 && offsetof(qlora_dropout, offset) == 16);

  /* default format: NF4, double quantisation, bf16 */
  CHECK(qlora_nf4_weight_init(&w, 1024, 1024) == QLORA_OK);
  CHECK(w.format_version == QLORA_NF4_FORMAT_VERSION && w.blocksize == QLORA_NF4_BLOCKSIZE);
  CHECK(w.dq_blocksize == QLORA_NF4_DQ_BLOCKSIZE && w.quant_type == QLORA_QUANT_NF4 &&
        w.compute_dtype == QLORA_COMPUTE_BF16);
  CHECK(qlora_nf4_buffer_sizes(1024, 1024, &a, &b, &c, &d) == QLORA_OK);
  CHECK(a == 524288 && b == 16384 && c == 4 * 64 && d == 4);
  CHECK(qlora_nf4_weight_buffer_sizes(&w, &a, &b, &c, &d) == QLORA_OK);
  CHECK(a == 524288 && b == 16384 && c == 4 * 64 && d == 4);
  CHECK(qlora_nf4_weight_init(&w, 8, 64) == QLORA_ERR_SHAPE);

  /* variant: INT4, float32 constants (4.5 bits), fp16 */
  CHECK(qlora_nf4_weight_init_ex(&w, 1024, 1024, QLORA_QUANT_INT4, 0, QLORA_COMPUTE_FP16) ==
        QLORA_OK);
  CHECK(w.dq_blocksize == QLORA_NF4_DQ_OFF);
  CHECK(qlora_nf4_weight_buffer_sizes(&w, &a, &b, &c, &d) == QLORA_OK);
  CHECK(a == 524288 && b == 0 && c == 4 * 16384 && d == 0);
  CHECK(qlora_nf4_weight_init_ex(&w, 1024, 1024, 7, 1, 0) == QLORA_ERR_FORMAT);

  /* sizes */
  CHECK(qlora_nf4_quantize_workspace(1024, 1024) > 0);
  CHECK(qlora_linear_workspace(512, 1024, 1024, 16, 1) > qlora_linear_workspace(512, 1024, 1024, 16, 0));
  CHECK(qlora_pre_dequant_min_tokens() == 2048);
  CHECK(qlora_set_pre_dequant_min_tokens(-5) == -1);
  CHECK(qlora_linear_workspace(2048, 1024, 1024, 16, 0) >=
        qlora_linear_workspace(2047, 1024, 1024, 16, 0) + (size_t)2 * 1024 * 1024);
  CHECK(qlora_linear_workspace(512, 1024, 1024, 24, 0) == 0);
  CHECK(qlora_linear_workspace_dropout(512, 1024, 1024, 16, 0) >
        qlora_linear_workspace(512, 1024, 1024, 16, 0));
  CHECK(qlora_dropout_mask_bytes(5, 64) == 64);

  /* validation before any device access */
  CHECK(qlora_nf4_dequantize(NULL, NULL, NULL) == QLORA_ERR_NULL);
  CHECK(qlora_set_timing_events(QLORA_TIMING_DROPOUT + 1, NULL, NULL) == QLORA_ERR_SHAPE);
  CHECK(qlora_status_string(QLORA_ERR_FORMAT) != NULL);
  printf("ok\n");
  return 0;
}
