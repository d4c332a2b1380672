// C ABI entry points: host-side validation and kernel dispatch.
//
// Every check here runs before any HIP call so that invalid calls return a
// status without touching the GPU (and can be tested on a machine without
// one).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/bsa.h"

namespace bsa {
int launch_attn_fwd(const void *q, const void *k, const void *v, int B, int H, int Nq, int Nk,
                    int d, int kv_block, const int32_t *idx, const float *bias,
                    const int32_t *count, int max_blocks, float scale, void *out, float *lse,
                    hipStream_t stream);
int launch_sip_plan(const float *scores, int rows, int nqb, int M, int budget, int mode,
                    uint64_t seed, const uint64_t *offsets, int32_t *idx, float *bias,
                    int32_t *count, double *lambda, int32_t *status, hipStream_t stream);
int launch_select_scores(const void *q, const void *k, int B, int H, int N, int d, int kv_block,
                         int n_clusters, int kmeans_iters, float *scores, float *centroids,
                         float *weights, void *workspace, hipStream_t stream);
size_t select_workspace_bytes(int B, int H, int N, int d, int kv_block, int n_clusters);
int basa_layout(int T, int Hg, int Wg, int d, int wh, int ww, int ph, int pw, int topk,
                int kv_block, int B, int H, int *nwin, int *Nq_pad, int *Nk, int *max_blocks,
                size_t *workspace);
int launch_basa_plan(const void *q, const void *k, const void *v, int B, int H, int T, int Hg,
                     int Wg, int d, int wh, int ww, int dy, int dx, int ph, int pw, int topk,
                     int kv_block, void *qp, void *kp, void *vp, int32_t *idx, int32_t *count,
                     int32_t *routes, void *workspace, hipStream_t stream);
int launch_basa_plan_noalloc(const void *q, const void *k, const void *v, int B, int H, int T,
                             int Hg, int Wg, int d, int wh, int ww, int dy, int dx, int ph,
                             int pw, int topk, int kv_block, void *qp, void *kp, void *vp,
                             int32_t *idx, int32_t *count, int32_t *routes, hipStream_t stream);
int launch_window_unpermute(const void *out_perm, void *out, int B, int H, int T, int Hg,
                            int Wg, int d, int wh, int ww, int dy, int dx, hipStream_t stream);
uint64_t sampling_offset(uint64_t seed, uint64_t row);
int mass_chunk_keys(int kv_block);
int launch_attn_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
                    const float *lse, int B, int H, int Nq, int Nk, int d, int kv_block,
                    const int32_t *idx, const float *bias, const int32_t *count, int max_blocks,
                    float scale, float *dq, float *dk, float *dv, hipStream_t stream);
size_t attn_bwd_slab_bytes(int Nq, int Nk, int d, int kv_block, int max_blocks);
long long attn_bwd_union_entries(int Nq, int kv_block, int max_blocks);
int launch_attn_bwd_ws(const void *q, const void *k, const void *v, const void *o,
                       const void *dout, const float *lse, int B, int H, int Nq, int Nk, int d,
                       int kv_block, const int32_t *idx, const float *bias, const int32_t *count,
                       int max_blocks, float scale, float *dq, float *dk, float *dv,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);
void basa_offsets(int w, int L, int *b);
void basa_shifts(int wh, int ww, int L, int S, const int *c_h, const int *c_w, int *dy, int *dx);
int launch_block_mass(const void *q, const void *k, const float *lse, int B, int H, int Nq, int Nk,
                      int d, int kv_block, float scale, float *mass, hipStream_t stream);
int launch_plan_coverage(const float *mass, const int32_t *idx, const int32_t *count, int rows,
                         int M, int max_blocks, double *cov, hipStream_t stream);
int launch_output_error(const void *out, const void *ref, int slabs, long long n, double *sums,
                        hipStream_t stream);
long long mfma_peak_flops(int workgroups, int iters);
int launch_mfma_peak(int workgroups, int iters, int operands, float *sink, hipStream_t stream);
}  // namespace bsa

namespace {

constexpr long long kMaxIndex = 0x7fffffffLL;

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
bool pow2_block(int b) { return b >= 1 && b <= 128 && (b & (b - 1)) == 0; }
bool head_dim_ok(int d) { return d == 64 || d == 128; }
bool clusters_ok(int c) { return c >= 1 && c <= 16 && (c & (c - 1)) == 0; }

// Checks shared by both backward entry points.
int attn_bwd_check(const void *q, const void *k, const void *v, const void *o, const void *dout,
                   const float *lse, int B, int H, int Nq, int Nk, int d, int q_block,
                   int kv_block, const int32_t *idx, const float *bias, const int32_t *count,
                   int max_blocks, float softmax_scale, float *dq, float *dk, float *dv) {
  if (!q || !k || !v || !o || !dout || !lse || !idx || !count || !dq || !dk || !dv)
    return BSA_ERR_ARG;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || max_blocks < 1) return BSA_ERR_ARG;
  if (!std::isfinite(softmax_scale)) return BSA_ERR_ARG;
  if (!head_dim_ok(d) || q_block != 128 || !pow2_block(kv_block)) return BSA_ERR_UNSUPPORTED;
  if (dk == dv || dq == dk || dq == dv) return BSA_ERR_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4) || !aligned(idx, 4) || !aligned(count, 4) || (bias && !aligned(bias, 4)))
    return BSA_ERR_ALIGN;
  const long long nqb = (Nq + 127) / 128;
  if ((long long)B * H * nqb > kMaxIndex) return BSA_ERR_SIZE;
  if ((long long)max_blocks * kv_block > kMaxIndex) return BSA_ERR_SIZE;
  if ((long long)Nk + kv_block > kMaxIndex) return BSA_ERR_SIZE;
  return BSA_OK;
}

float bwd_scale(float softmax_scale, int d) {
  return softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)d);
}

}  // namespace

extern "C" {

const char *bsa_status_string(int status) {
  switch (status) {
    case BSA_OK: return "ok";
    case BSA_ERR_ARG: return "invalid argument (null pointer, non-positive size or bad mode)";
    case BSA_ERR_UNSUPPORTED: return "unsupported head dim, block size or cluster count";
    case BSA_ERR_BUDGET: return "budget outside [1, M]";
    case BSA_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
    case BSA_ERR_HIP: return "HIP runtime call or kernel launch failed";
    case BSA_ERR_WORKSPACE: return "workspace missing or too small";
    case BSA_ERR_SIZE: return "size product exceeds the supported index range";
    case BSA_ERR_NONFINITE: return "a score row holds a NaN, an infinity or a negative value";
    case BSA_ERR_SCRATCH:
      return "problem needs more scratch than the allocation-free entry point's fixed array";
    default: return "unknown status";
  }
}

const char *bsa_version(void) { return "bsa 0.1 gfx950"; }

uint64_t bsa_sampling_offset(uint64_t seed, uint64_t row) { return bsa::sampling_offset(seed, row); }

int bsa_attn_fwd(const void *q, const void *k, const void *v, int B, int H, int Nq, int Nk,
                 int d, int q_block, int kv_block, const int32_t *idx, const float *bias,
                 const int32_t *count, int max_blocks, float softmax_scale, void *out,
                 float *lse, void *stream) {
  if (!q || !k || !v || !idx || !count || !out) return BSA_ERR_ARG;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || max_blocks < 1) return BSA_ERR_ARG;
  if (!std::isfinite(softmax_scale)) return BSA_ERR_ARG;
  if (!head_dim_ok(d) || q_block != 128 || !pow2_block(kv_block)) return BSA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(idx, 4) || !aligned(count, 4) || (bias && !aligned(bias, 4)) ||
      (lse && !aligned(lse, 4)))
    return BSA_ERR_ALIGN;
  const long long nqb = (Nq + 127) / 128;
  if ((long long)B * H * nqb > kMaxIndex) return BSA_ERR_SIZE;
  if ((long long)max_blocks * kv_block > kMaxIndex) return BSA_ERR_SIZE;
  if ((long long)Nk + kv_block > kMaxIndex) return BSA_ERR_SIZE;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)d);
  return bsa::launch_attn_fwd(q, k, v, B, H, Nq, Nk, d, kv_block, idx, bias, count, max_blocks,
                              scale, out, lse, (hipStream_t)stream);
}

int bsa_sip_plan(const float *scores, int B, int H, int nQB, int M, int budget, int mode,
                 uint64_t seed, const uint64_t *offsets, int32_t *idx, float *bias,
                 int32_t *count, double *lambda, int32_t *status, void *stream) {
  if (!scores || !idx || !count) return BSA_ERR_ARG;
  if (B < 1 || H < 1 || nQB < 1 || M < 1) return BSA_ERR_ARG;
  if (mode != BSA_PLAN_SIP && mode != BSA_PLAN_TOPK) return BSA_ERR_ARG;
  if (budget < 1 || budget > M) return BSA_ERR_BUDGET;
  if (!aligned(scores, 16) || !aligned(idx, 4) || !aligned(count, 4) ||
      (bias && !aligned(bias, 4)) || (lambda && !aligned(lambda, 8)) ||
      (offsets && !aligned(offsets, 8)) || (status && !aligned(status, 4)))
    return BSA_ERR_ALIGN;
  if ((long long)B * H * nQB > kMaxIndex) return BSA_ERR_SIZE;
  if (M > (1 << 20)) return BSA_ERR_SIZE;  // one row must fit the on-chip sampler
  if (mode == BSA_PLAN_SIP && M > BSA_SIP_MAX_BLOCKS) return BSA_ERR_SIZE;
  return bsa::launch_sip_plan(scores, B * H * nQB, nQB, M, budget, mode, seed, offsets, idx,
                              bias, count, lambda, status, (hipStream_t)stream);
}

int bsa_select_workspace_bytes(int B, int H, int N, int d, int q_block, int kv_block,
                               int n_clusters, size_t *bytes) {
  if (!bytes) return BSA_ERR_ARG;
  if (B < 1 || H < 1 || N < 1) return BSA_ERR_ARG;
  if (!head_dim_ok(d) || q_block != 128 || !pow2_block(kv_block) || !clusters_ok(n_clusters))
    return BSA_ERR_UNSUPPORTED;
  *bytes = bsa::select_workspace_bytes(B, H, N, d, kv_block, n_clusters);
  return BSA_OK;
}

int bsa_select_scores(const void *q, const void *k, int B, int H, int N, int d, int q_block,
                      int kv_block, int n_clusters, int kmeans_iters, float *scores,
                      float *centroids, float *weights, void *workspace, size_t workspace_bytes,
                      void *stream) {
  if (!q || !k || !scores) return BSA_ERR_ARG;
  if (B < 1 || H < 1 || N < 1 || kmeans_iters < 0 || kmeans_iters > 16) return BSA_ERR_ARG;
  if (!head_dim_ok(d) || q_block != 128 || !pow2_block(kv_block) || !clusters_ok(n_clusters))
    return BSA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(scores, 16) ||
      (centroids && !aligned(centroids, 16)) || (weights && !aligned(weights, 4)))
    return BSA_ERR_ALIGN;
  const long long nqb = (N + 127) / 128;
  const long long M = (N + kv_block - 1) / kv_block;
  if ((long long)B * H * nqb * n_clusters > kMaxIndex) return BSA_ERR_SIZE;
  if ((long long)B * H * M > kMaxIndex) return BSA_ERR_SIZE;
  if (nqb * M > 0xffffffffLL) return BSA_ERR_SIZE;  // one head's scores, 32-bit offsets
  const size_t need = bsa::select_workspace_bytes(B, H, N, d, kv_block, n_clusters);
  if (!workspace || workspace_bytes < need) return BSA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return BSA_ERR_ALIGN;
  return bsa::launch_select_scores(q, k, B, H, N, d, kv_block, n_clusters, kmeans_iters, scores,
                                   centroids, weights, workspace, (hipStream_t)stream);
}

int bsa_basa_layout(int T, int Hg, int Wg, int d, int wh, int ww, int ph, int pw, int topk,
                    int kv_block, int B, int H, int *nwin, int *Nq_pad, int *Nk,
                    int *max_blocks, size_t *workspace) {
  if (!nwin || !Nq_pad || !Nk || !max_blocks || !workspace) return BSA_ERR_ARG;
  if (T < 1 || Hg < 1 || Wg < 1 || wh < 1 || ww < 1 || ph < 1 || pw < 1 || topk < 0 || B < 1 ||
      H < 1)
    return BSA_ERR_ARG;
  if (wh > Hg || ww > Wg) return BSA_ERR_ARG;
  if (!head_dim_ok(d) || !pow2_block(kv_block)) return BSA_ERR_UNSUPPORTED;
  return bsa::basa_layout(T, Hg, Wg, d, wh, ww, ph, pw, topk, kv_block, B, H, nwin, Nq_pad, Nk,
                          max_blocks, workspace);
}

// Checks shared by bsa_basa_plan and bsa_basa_plan_noalloc; *ws receives the
// scratch bytes the call needs.
static int check_basa_plan(const void *q, const void *k, const void *v, int B, int H, int T,
                           int Hg, int Wg, int d, int wh, int ww, int ph, int pw, int topk,
                           int kv_block, const void *qp, const void *kp, const void *vp,
                           const int32_t *idx, const int32_t *count, const int32_t *routes,
                           size_t *ws) {
  if (!q || !k || !v || !qp || !kp || !vp || !idx || !count) return BSA_ERR_ARG;
  int nwin, nqp, nk, mb;
  int st = bsa_basa_layout(T, Hg, Wg, d, wh, ww, ph, pw, topk, kv_block, B, H, &nwin, &nqp, &nk,
                           &mb, ws);
  if (st != BSA_OK) return st;
  if (topk > nwin - 1) return BSA_ERR_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(qp, 16) ||
      !aligned(kp, 16) || !aligned(vp, 16) || !aligned(idx, 4) || !aligned(count, 4) ||
      (routes && !aligned(routes, 4)))
    return BSA_ERR_ALIGN;
  return BSA_OK;
}

int bsa_basa_plan(const void *q, const void *k, const void *v, int B, int H, int T, int Hg,
                  int Wg, int d, int wh, int ww, int dy, int dx, int ph, int pw, int topk,
                  int kv_block, void *qp, void *kp, void *vp, int32_t *idx, int32_t *count,
                  int32_t *routes, void *workspace, size_t workspace_bytes, void *stream) {
  size_t ws;
  const int st = check_basa_plan(q, k, v, B, H, T, Hg, Wg, d, wh, ww, ph, pw, topk, kv_block, qp,
                                 kp, vp, idx, count, routes, &ws);
  if (st != BSA_OK) return st;
  if (!workspace || workspace_bytes < ws) return BSA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return BSA_ERR_ALIGN;
  return bsa::launch_basa_plan(q, k, v, B, H, T, Hg, Wg, d, wh, ww, dy, dx, ph, pw, topk,
                               kv_block, qp, kp, vp, idx, count, routes, workspace,
                               (hipStream_t)stream);
}

int bsa_basa_plan_noalloc(const void *q, const void *k, const void *v, int B, int H, int T,
                          int Hg, int Wg, int d, int wh, int ww, int dy, int dx, int ph, int pw,
                          int topk, int kv_block, void *qp, void *kp, void *vp, int32_t *idx,
                          int32_t *count, int32_t *routes, void *stream) {
  size_t ws;
  const int st = check_basa_plan(q, k, v, B, H, T, Hg, Wg, d, wh, ww, ph, pw, topk, kv_block, qp,
                                 kp, vp, idx, count, routes, &ws);
  if (st != BSA_OK) return st;
  if (ws > BSA_BASA_NOALLOC_SCRATCH_BYTES) return BSA_ERR_SCRATCH;
  return bsa::launch_basa_plan_noalloc(q, k, v, B, H, T, Hg, Wg, d, wh, ww, dy, dx, ph, pw, topk,
                                       kv_block, qp, kp, vp, idx, count, routes,
                                       (hipStream_t)stream);
}

int bsa_window_unpermute(const void *out_perm, void *out, int B, int H, int T, int Hg, int Wg,
                         int d, int wh, int ww, int dy, int dx, void *stream) {
  if (!out_perm || !out) return BSA_ERR_ARG;
  if (B < 1 || H < 1 || T < 1 || Hg < 1 || Wg < 1 || wh < 1 || ww < 1 || wh > Hg || ww > Wg)
    return BSA_ERR_ARG;
  if (!head_dim_ok(d)) return BSA_ERR_UNSUPPORTED;
  if (!aligned(out_perm, 16) || !aligned(out, 16)) return BSA_ERR_ALIGN;
  return bsa::launch_window_unpermute(out_perm, out, B, H, T, Hg, Wg, d, wh, ww, dy, dx,
                                      (hipStream_t)stream);
}

int bsa_block_mass(const void *q, const void *k, const float *lse, int B, int H, int Nq, int Nk,
                   int d, int q_block, int kv_block, float softmax_scale, float *mass,
                   void *stream) {
  if (!q || !k || !lse || !mass) return BSA_ERR_ARG;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || kv_block < 1) return BSA_ERR_ARG;
  if (!std::isfinite(softmax_scale)) return BSA_ERR_ARG;
  if (!head_dim_ok(d) || q_block != 128 || kv_block > 1024) return BSA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(lse, 4) || !aligned(mass, 4))
    return BSA_ERR_ALIGN;
  const long long nqb = (Nq + 127) / 128, M = ((long long)Nk + kv_block - 1) / kv_block;
  const long long ck = bsa::mass_chunk_keys(kv_block);
  const long long wgs = (long long)B * H * nqb * ((Nk + ck - 1) / ck);
  if ((long long)B * H * Nq * d > kMaxIndex * 8 || (long long)B * H * Nk * d > kMaxIndex * 8 ||
      (long long)B * H * nqb * M > kMaxIndex || wgs > kMaxIndex)
    return BSA_ERR_SIZE;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)d);
  return bsa::launch_block_mass(q, k, lse, B, H, Nq, Nk, d, kv_block, scale, mass,
                                (hipStream_t)stream);
}

int bsa_plan_coverage(const float *mass, const int32_t *idx, const int32_t *count, int rows,
                      int M, int max_blocks, double *coverage, void *stream) {
  if (!mass || !idx || !count || !coverage) return BSA_ERR_ARG;
  if (rows < 1 || M < 1 || max_blocks < 1) return BSA_ERR_ARG;
  if (!aligned(mass, 4) || !aligned(idx, 4) || !aligned(count, 4) || !aligned(coverage, 8))
    return BSA_ERR_ALIGN;
  if ((long long)rows * M > kMaxIndex * 8 || (long long)rows * max_blocks > kMaxIndex * 8)
    return BSA_ERR_SIZE;
  return bsa::launch_plan_coverage(mass, idx, count, rows, M, max_blocks, coverage,
                                   (hipStream_t)stream);
}

int bsa_output_error(const void *out, const void *ref, int slabs, long long n, double *sums,
                     void *stream) {
  if (!out || !ref || !sums) return BSA_ERR_ARG;
  if (slabs < 1 || n < 8 || n % 8 != 0) return BSA_ERR_ARG;
  if (!aligned(out, 16) || !aligned(ref, 16) || !aligned(sums, 8)) return BSA_ERR_ALIGN;
  if ((long long)slabs * n > kMaxIndex * 16) return BSA_ERR_SIZE;
  return bsa::launch_output_error(out, ref, slabs, n, sums, (hipStream_t)stream);
}

int bsa_basa_offsets(int w, int L, int *offsets) {
  if (!offsets || w < 1 || L < 1) return BSA_ERR_ARG;
  bsa::basa_offsets(w, L, offsets);
  return BSA_OK;
}

int bsa_basa_shifts(int wh, int ww, int L, int S, const int *c_h, const int *c_w, int *dy,
                    int *dx) {
  if (!dy || !dx || wh < 1 || ww < 1 || L < 1 || S < 1) return BSA_ERR_ARG;
  if ((long long)L * S > kMaxIndex) return BSA_ERR_SIZE;
  bsa::basa_shifts(wh, ww, L, S, c_h, c_w, dy, dx);
  return BSA_OK;
}

int bsa_attn_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
                 const float *lse, int B, int H, int Nq, int Nk, int d, int q_block, int kv_block,
                 const int32_t *idx, const float *bias, const int32_t *count, int max_blocks,
                 float softmax_scale, float *dq, float *dk, float *dv, void *stream) {
  const int st = attn_bwd_check(q, k, v, o, dout, lse, B, H, Nq, Nk, d, q_block, kv_block, idx,
                                bias, count, max_blocks, softmax_scale, dq, dk, dv);
  if (st != BSA_OK) return st;
  return bsa::launch_attn_bwd(q, k, v, o, dout, lse, B, H, Nq, Nk, d, kv_block, idx, bias, count,
                              max_blocks, bwd_scale(softmax_scale, d), dq, dk, dv,
                              (hipStream_t)stream);
}

// The workspace form's index space: slot numbers of one slab's union
// entries (pairs of query blocks x (2 max_blocks + 3 passes' padding)) and
// key positions inside one pair's union list stay below 2^31.
static bool bwd_ws_sizes_ok(int Nq, int kv_block, int max_blocks) {
  const long long bpp = kv_block >= 128 ? 1 : 128 / kv_block;
  if (bsa::attn_bwd_union_entries(Nq, kv_block, max_blocks) > kMaxIndex - 63) return false;
  return (2LL * max_blocks + 3 * bpp) * kv_block <= kMaxIndex;
}

int bsa_attn_bwd_workspace_bytes(int Nq, int Nk, int d, int q_block, int kv_block,
                                 int max_blocks, size_t *bytes) {
  if (!bytes) return BSA_ERR_ARG;
  if (Nq < 1 || Nk < 1 || max_blocks < 1) return BSA_ERR_ARG;
  if (!head_dim_ok(d) || q_block != 128 || !pow2_block(kv_block)) return BSA_ERR_UNSUPPORTED;
  if (!bwd_ws_sizes_ok(Nq, kv_block, max_blocks)) return BSA_ERR_SIZE;
  if ((long long)max_blocks * kv_block > kMaxIndex) return BSA_ERR_SIZE;
  if ((long long)Nk + kv_block > kMaxIndex) return BSA_ERR_SIZE;
  *bytes = bsa::attn_bwd_slab_bytes(Nq, Nk, d, kv_block, max_blocks);
  return BSA_OK;
}

int bsa_attn_bwd_ws(const void *q, const void *k, const void *v, const void *o, const void *dout,
                    const float *lse, int B, int H, int Nq, int Nk, int d, int q_block,
                    int kv_block, const int32_t *idx, const float *bias, const int32_t *count,
                    int max_blocks, float softmax_scale, float *dq, float *dk, float *dv,
                    void *workspace, size_t workspace_bytes, void *stream) {
  const int st = attn_bwd_check(q, k, v, o, dout, lse, B, H, Nq, Nk, d, q_block, kv_block, idx,
                                bias, count, max_blocks, softmax_scale, dq, dk, dv);
  if (st != BSA_OK) return st;
  if (!bwd_ws_sizes_ok(Nq, kv_block, max_blocks)) return BSA_ERR_SIZE;
  // one wave per KV block of every slab in the per-block sums' grid
  if ((long long)B * H * (((long long)Nk + kv_block - 1) / kv_block) > kMaxIndex * 4)
    return BSA_ERR_SIZE;
  if (!workspace) return BSA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return BSA_ERR_ALIGN;
  if (workspace_bytes < bsa::attn_bwd_slab_bytes(Nq, Nk, d, kv_block, max_blocks))
    return BSA_ERR_WORKSPACE;
  return bsa::launch_attn_bwd_ws(q, k, v, o, dout, lse, B, H, Nq, Nk, d, kv_block, idx, bias,
                                 count, max_blocks, bwd_scale(softmax_scale, d), dq, dk, dv,
                                 workspace, workspace_bytes, (hipStream_t)stream);
}

int bsa_mfma_peak_probe(int workgroups, int iters, int operands, float *sink, long long *flops,
                        void *stream) {
  if (!sink || workgroups < 1 || iters < 1) return BSA_ERR_ARG;
  if (operands != BSA_PROBE_RANDOM && operands != BSA_PROBE_LOW_ENTROPY) return BSA_ERR_ARG;
  if (!aligned(sink, 4)) return BSA_ERR_ALIGN;
  if (flops) *flops = bsa::mfma_peak_flops(workgroups, iters);
  return bsa::launch_mfma_peak(workgroups, iters, operands, sink, (hipStream_t)stream);
}

}  // extern "C"
