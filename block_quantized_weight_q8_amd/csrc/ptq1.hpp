// Internal entry points of the PTQ1_0 kernels, for the stacked-projection
// dispatch and the launch-shape query of q8gemv.hip.
#pragma once

#include <stdint.h>

#include "q8gemv.h"

namespace q8g {

// gemv_stacked for Q8G_PTQ1_0 parts (x = rotated codes int8 [K], dx = binary16 [K/128]).
q8g_status ptq1_stacked(const q8g_part *parts, int nparts, const int8_t *qx, const uint16_t *dx, int64_t K,
                        void *stream);

// rows per wave step and waves per workgroup of the PTQ1_0 GEMV over n_total rows of K.
q8g_status ptq1_config(int64_t n_total, int64_t K, int *rows_per_wave, int *waves_per_group);

}  // namespace q8g
