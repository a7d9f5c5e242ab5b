// Split-K GQA decode attention, MFMA path (16 or more query rows per KV
// head, e.g. GQA group 16 x 4 draft tokens in speculative verification).
// Placeholder dispatch: runs the VALU partial kernel over groups of 8 rows.
#include <hip/hip_runtime.h>

#include "attn_internal.h"

namespace had {

hipError_t launch_attn_mfma(const ValuArgs& a_in, int head_dim, dim3 grid, hipStream_t stream) {
  ValuArgs a = a_in;
  hipError_t e = hipSuccess;
  for (int rb = 0; rb < a.rows && e == hipSuccess; rb += 8) {
    a.row_base = rb;
    e = launch_attn_valu(a, head_dim, grid, stream);
  }
  return e;
}

}  // namespace had
