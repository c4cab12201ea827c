// The one-row-per-lane panel, one quantization group per block (group size = block size).
#include "panel_row.h"

namespace gptq {

hipError_t row_panel_launch_group(dim3 grid, dim3 block, hipStream_t s, float* W, int d_row, int d_col, int i1,
                                 const float* U, int maxq, int gwide, int ngroups, uint8_t* codes,
                                 float* scales, int32_t* zeros, float* E, double* part_e) {
  return rowpanel::launch<true>(grid, block, s, W, d_row, d_col, i1, U, maxq, gwide, ngroups, codes, scales,
                                zeros, E, part_e);
}

}  // namespace gptq
