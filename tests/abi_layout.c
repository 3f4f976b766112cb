/* Prints the size and field offsets of the C-ABI structs (include/fp4.h),
 * one "struct.field offset" per line, for the Python binding's layout test. */
#include <stddef.h>
#include <stdio.h>

#include "fp4.h"

#define F(S, f) printf(#S "." #f " %zu\n", offsetof(S, f))

int main(void) {
  printf("fp4_quant_desc.__size__ %zu\n", sizeof(fp4_quant_desc));
  F(fp4_quant_desc, format);
  F(fp4_quant_desc, block);
  F(fp4_quant_desc, orient);
  F(fp4_quant_desc, round);
  F(fp4_quant_desc, seed);
  F(fp4_quant_desc, offset);
  F(fp4_quant_desc, rht);
  F(fp4_quant_desc, rht_signs);
  F(fp4_quant_desc, target);
  F(fp4_quant_desc, amax_given);
  F(fp4_quant_desc, emit_transpose);
  F(fp4_quant_desc, scale_layout);
  F(fp4_quant_desc, rht_n);
  F(fp4_quant_desc, rht_signs_hi);
  F(fp4_quant_desc, scale_round);
  F(fp4_quant_desc, global_scope);
  F(fp4_quant_desc, count_level);
  printf("fp4_operand.__size__ %zu\n", sizeof(fp4_operand));
  F(fp4_operand, format);
  F(fp4_operand, codes);
  F(fp4_operand, ld_codes);
  F(fp4_operand, scales);
  F(fp4_operand, scale_stride_row);
  F(fp4_operand, scale_stride_kblk);
  F(fp4_operand, scale_row_group);
  F(fp4_operand, s_dec);
  F(fp4_operand, scale_layout);
  F(fp4_operand, s_dec_scope);
  printf("fp4_counters.__size__ %zu\n", sizeof(fp4_counters));
  return 0;
}
