/* A plain C99 caller of libradial.so: includes the header, builds the Wan-shaped mask
 * on the host and prints its sizes, and queries the element-table size and an error
 * string. Host calls only, so it runs without a GPU. */
#include <stdio.h>
#include <stdlib.h>

#include "radial_attn.h"

int main(void) {
  int32_t nb = 0;
  int64_t nnz = 0;
  if (radial_mask_dims(21, 1560, 1560, RADIAL_BLOCK, &nb, &nnz) != RADIAL_OK) return 1;
  int32_t* row_ptr = malloc(sizeof(int32_t) * (size_t)(nb + 1));
  int32_t* col_idx = malloc(sizeof(int32_t) * (size_t)nnz);
  if (!row_ptr || !col_idx) return 2;
  if (radial_build_mask(21, 1560, 1560, RADIAL_BLOCK, row_ptr, col_idx, nnz) != RADIAL_OK)
    return 3;
  int64_t table_bytes = 0;
  if (radial_element_table_bytes(nnz, &table_bytes) != RADIAL_OK) return 4;
  printf("nb=%d nnz=%lld last_row=%d table_bytes=%lld err=%s\n", nb, (long long)nnz,
         row_ptr[nb] - row_ptr[nb - 1], (long long)table_bytes,
         radial_error_string(RADIAL_ERR_SHAPE_MISMATCH));
  free(row_ptr);
  free(col_idx);
  return 0;
}
