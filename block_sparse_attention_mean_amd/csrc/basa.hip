// BASA list construction (placeholder).
#include "common.h"
namespace bsa {
int basa_layout(int, int, int, int, int, int, int, int, int, int, int, int, int *, int *, int *,
                int *, int *, size_t *) {
  return BSA_ERR_UNSUPPORTED;
}
int launch_basa_plan(const void *, const void *, const void *, int, int, int, int, int, int, int,
                     int, int, int, int, int, int, int, void *, void *, void *, int32_t *,
                     int32_t *, int32_t *, void *, hipStream_t) {
  return BSA_ERR_UNSUPPORTED;
}
int launch_window_unpermute(const void *, void *, int, int, int, int, int, int, int, int, int,
                            int, hipStream_t) {
  return BSA_ERR_UNSUPPORTED;
}
}  // namespace bsa
