// Selector kernels (placeholder).
#include "common.h"
namespace bsa {
size_t select_workspace_bytes(int, int, int, int, int, int) { return 0; }
int launch_select_scores(const void *, const void *, int, int, int, int, int, int, int, float *,
                         float *, float *, void *, hipStream_t) {
  return BSA_ERR_UNSUPPORTED;
}
}  // namespace bsa
