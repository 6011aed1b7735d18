/* A plain C99 caller of the library's host-side entry points: the header compiles
 * as strict C, and the shape check, padding, RoPE table and workspace sizes answer
 * as documented without a GPU.  Built and run by tests/test_abi_host.py.  Exit
 * status 0 when every check holds; otherwise the number of the first failed check. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rotattn.h"

int main(void) {
  /* the Wan-720p-like layer: 21 x 45 x 80 tokens, D = 128 split 44/42/42 */
  rotattn_shape s = {1, 40, 21, 45, 80, 128, 44, 42, 42, 64, 64};
  rotattn_shape bad = s;
  size_t nf;
  float* tab;
  if (rotattn_check_shape(&s) != ROTATTN_OK) return 1;
  bad.Dw = 40; /* 44 + 42 + 40 != 128 */
  if (rotattn_check_shape(&bad) != ROTATTN_E_SHAPE) return 2;
  if (rotattn_padded_tokens(&s) != 75776) return 3; /* 75600 rounded up to 256 */
  if (rotattn_quantize_qk_workspace(&s) == 0 || rotattn_int4_attention_workspace(&s) == 0) return 4;
  if (rotattn_quantize_qk_workspace(&bad) != 0) return 5;
  nf = rotattn_rope_table_floats(&s);
  /* per axis and pair: (cos, sin) for every position of that axis */
  if (nf != (size_t)2 * (21 * 22 + 45 * 21 + 80 * 21)) return 6;
  tab = (float*)malloc(nf * sizeof(float));
  if (!tab) return 7;
  if (rotattn_build_rope_table(&s, ROTATTN_ROT_HALF, 10000.0, tab) != ROTATTN_OK) return 8;
  /* position 0 of every axis: angle 0, so (cos, sin) = (1, 0) */
  if (tab[0] != 1.0f || tab[1] != 0.0f) return 9;
  free(tab);
  if (strlen(rotattn_status_str(ROTATTN_E_SHAPE)) == 0) return 10;
  printf("c abi ok\n");
  return 0;
}
