// Allocation-free variant of the BASA list builder.
//
// bsa_basa_plan takes a caller workspace for its scratch: the fp32 window
// means of Q and K ([BH][2][nwin][d]) and the routed windows
// ([BH][nwin][topk] int32).  bsa_basa_plan_noalloc runs the same kernels with
// that scratch in the file-scope device array below, so the call needs no
// allocation of any kind.  Each GPU holds its own copy of the array for the
// life of the process.  The host never passes the array's name to a kernel:
// the device address of the current GPU's copy is looked up once per device
// with hipGetSymbolAddress and that address is what the kernels receive.
//
// Every byte the kernels read from the scratch is written earlier in the
// same call (means before routing, routes before the lists), so nothing has
// to be cleared between calls.  Two calls that overlap on one GPU share the
// array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/bsa.h"

namespace bsa {
int launch_basa_plan(const void *q, const void *k, const void *v, int B, int H, int T, int Hg,
                     int Wg, int d, int wh, int ww, int dy, int dx, int ph, int pw, int topk,
                     int kv_block, void *qp, void *kp, void *vp, int32_t *idx, int32_t *count,
                     int32_t *routes, void *workspace, hipStream_t stream);

namespace {

static __device__ __align__(256) unsigned char scratch[BSA_BASA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_dev[kMaxDevices];  // device address of `scratch` on each GPU

}  // namespace

// Device address of the current GPU's copy of `scratch`.
int basa_noalloc_scratch(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return BSA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return BSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BSA_ERR_HIP;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return BSA_OK;
}

int launch_basa_plan_noalloc(const void *q, const void *k, const void *v, int B, int H, int T,
                             int Hg, int Wg, int d, int wh, int ww, int dy, int dx, int ph,
                             int pw, int topk, int kv_block, void *qp, void *kp, void *vp,
                             int32_t *idx, int32_t *count, int32_t *routes, hipStream_t stream) {
  void *ws = nullptr;
  const int st = basa_noalloc_scratch(&ws);
  if (st != BSA_OK) return st;
  return launch_basa_plan(q, k, v, B, H, T, Hg, Wg, d, wh, ww, dy, dx, ph, pw, topk, kv_block, qp,
                          kp, vp, idx, count, routes, ws, stream);
}

}  // namespace bsa
