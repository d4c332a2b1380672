/*
 * bsa.h -- C ABI of the block-sparse attention forward library for AMD
 * MI355X (gfx950).
 *
 * The library computes the hot path of training-free dynamic block-sparse
 * attention for video diffusion transformers:
 *
 *   bsa_select_scores  KV-block mean pooling, k-means inside every 128-query
 *                      block, block scores (AB-Attention page, onedev.kr/
 *                      papers/1521, section "무엇과 다른가": the
 *                      Intra-Block Clustering Selector);
 *   bsa_sip_plan       SIP inclusion probabilities pi = min(1, lambda * S)
 *                      fitted to the budget, systematic sample of exactly s
 *                      distinct blocks; or top-k (same page, section
 *                      "어떻게 쓰나", and the ablation paragraph of
 *                      "전제와 한계");
 *   bsa_attn_fwd       one fused pass that gathers the listed small KV
 *                      blocks into full tiles, shifts logits by -log pi,
 *                      and runs online softmax with P.V accumulation (same
 *                      page, section "전제와 한계", first paragraph);
 *   bsa_attn_bwd,      its gradients dQ, dK, dV with the plan held fixed
 *   bsa_attn_bwd_ws    (dK and dV by atomic adds, or by sums of partial
 *                      rows in a caller's workspace, one per entry of the
 *                      union of two neighbouring query blocks' lists);
 *   bsa_basa_*         the shifted-window + routed-window + pooled-memory
 *                      structure of the BASA page (onedev.kr/papers/688,
 *                      sections "어떻게 동작하나" and "무엇과 다른가") turned
 *                      into block lists for bsa_attn_fwd, and its per-layer
 *                      shift schedule;
 *   bsa_block_mass,    accuracy diagnostics of a plan: the true attention
 *   bsa_plan_coverage, mass of every KV block, the mass a plan retains, and
 *   bsa_output_error   the output error against dense attention
 *                      (AB-Attention page, sections "무엇과 다른가" and
 *                      "어떻게 쓰나").
 *
 * Conventions for every entry point:
 *   - Tensors are dense, row-major and contiguous.  [B,H,N,d] means
 *     element (b,h,n,c) sits at ((b*H + h)*N + n)*d + c.  bf16 tensors are
 *     passed as `const void*` / `void*` holding IEEE bfloat16 bit patterns.
 *   - Every pointer argument is a DEVICE pointer unless its comment says
 *     host.  The caller allocates and owns every buffer; the library never
 *     allocates, frees or keeps device memory and holds no state between
 *     calls (the one exception: the fixed scratch array that
 *     bsa_basa_plan_noalloc uses instead of a workspace).
 *   - `stream` is a hipStream_t passed as `void *`, so that this header
 *     needs no HIP include (NULL = the null stream).  All work is enqueued
 *     asynchronously on it; no entry point synchronises.
 *   - All argument checks run on the host before any HIP call, so an
 *     invalid call returns an error code without touching the GPU.  A HIP
 *     launch failure returns BSA_ERR_HIP (an error that an earlier HIP call
 *     outside the library left pending on the thread is cleared first, so
 *     the status speaks of the call's own launches).  Errors that only the device can
 *     see (non-finite scores, out-of-range block indices) are reported in
 *     the outputs as documented per call; they never fault.
 *   - Supported sizes: head dim d in {64, 128}; q_block = 128; kv_block a
 *     power of two in [1, 128]; B, H >= 1; N >= 1; every 16-byte vector
 *     access requires bf16 tensors to be 16-byte aligned.
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  BSA_OK = 0,
  BSA_ERR_ARG = -1,         /* null pointer, non-positive size, bad mode   */
  BSA_ERR_UNSUPPORTED = -2, /* head dim, block size or cluster count       */
  BSA_ERR_BUDGET = -3,      /* budget outside [1, M]                       */
  BSA_ERR_ALIGN = -4,       /* a tensor pointer is not 16-byte aligned     */
  BSA_ERR_HIP = -5,         /* a HIP runtime call or launch failed         */
  BSA_ERR_WORKSPACE = -6,   /* workspace missing or smaller than required  */
  BSA_ERR_SIZE = -7,        /* a size product overflows the index range    */
  BSA_ERR_SCRATCH = -8,     /* more than an allocation-free call's fixed scratch */
  BSA_ERR_NONFINITE = -9    /* (device status word) a score row is not finite / >= 0 */
};

enum { BSA_PLAN_SIP = 0, BSA_PLAN_TOPK = 1 };

/* Human-readable text of a status code (static storage, never NULL). */
const char *bsa_status_string(int status);

/* Library version string, e.g. "bsa 0.1 gfx950" (static storage). */
const char *bsa_version(void);

/* ------------------------------------------------------------------------
 * Selector (AB-Attention page, section "무엇과 다른가").
 *
 * For every (b, h) and query block i (rows [128 i, min(N, 128 i + 128))):
 *   pooled key   kbar_j = mean of K rows of KV block j (the last block
 *                averages its valid rows only), j < M = ceil(N / kv_block);
 *   k-means      n_clusters clusters start from contiguous segment means
 *                (segment c = rows [floor(c n / C), floor((c+1) n / C)));
 *                each of kmeans_iters iterations assigns every query to the
 *                nearest centroid (squared Euclidean distance, ties to the
 *                lowest cluster) and moves every non-empty cluster to its
 *                members' mean; share w_c = members / n.  This runs in fp32
 *                in a fixed operation order (ascending-row member sums, one
 *                IEEE division, distances summed over dims in ascending
 *                order without fused multiply-add), so its decisions are
 *                reproducible bit for bit;
 *   scores       S_ij = sum_c w_c softmax_j(mu_c . kbar_j / sqrt(d)), the
 *                softmax running over all M KV blocks of the head.
 *
 * q, k        [B,H,N,d] bf16, 16-byte aligned.
 * scores      out: [B,H,nQB,M] fp32, nQB = ceil(N / q_block).
 * centroids   optional out (NULL = not written): [B,H,nQB,C,d] fp32.
 * weights     optional out (NULL = not written): [B,H,nQB,C] fp32.
 * workspace   device scratch of at least bsa_select_workspace_bytes() bytes,
 *             256-byte aligned; its contents are undefined after the call.
 * n_clusters  1, 2, 4, 8 or 16; kmeans_iters 0..16 (0 = segment means).
 * Sizes: B*H*M and B*H*nQB*n_clusters at most 2^31 - 1, and one head's
 * score matrix (nQB * M entries) below 2^32; larger problems return
 * BSA_ERR_SIZE before any HIP call.
 * --------------------------------------------------------------------- */
int bsa_select_workspace_bytes(int B, int H, int N, int d, int q_block, int kv_block,
                               int n_clusters, size_t *bytes /* host out */);

int bsa_select_scores(const void *q, const void *k, int B, int H, int N, int d,
                      int q_block, int kv_block, int n_clusters, int kmeans_iters,
                      float *scores, float *centroids, float *weights,
                      void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Sampling plan (AB-Attention page, section "어떻게 쓰나").
 *
 * One row = one (b, h, i).  mode BSA_PLAN_SIP:
 *   M+ = number of positive scores.  If budget >= M+, every positive block
 *   is taken with pi = 1 (count = M+, lambda = +inf).  Otherwise r is the
 *   smallest number of saturated blocks with (s - r) * S_(r+1) <= T_r
 *   decided exactly (S_(1) >= S_(2) >= ... sorted scores, T_r the exact sum
 *   of all but the r largest), found by bisection; lambda = (s - r) / T_r
 *   with T_r correctly rounded to fp64 and one IEEE fp64 division;
 *   pi_j = min(1, lambda * S_j) (one IEEE fp64 multiply);
 *   Pi_j = floor(pi_j * 2^44), C_j = Pi_0 + ... + Pi_j (exact integers);
 *   block j is drawn when some x_k = U + k * 2^44 (k = 0..s-1) falls in
 *   [C_{j-1}, C_j).  Exactly s distinct blocks are drawn; every block with
 *   pi = 1 is among them.  (The floors lose less than one unit per block
 *   and the fp64 rounding of lambda and pi less than 3 s 2^-9 units in all,
 *   so C_M >= s 2^44 - 2^16 > x_{s-1} whenever M <= BSA_SIP_MAX_BLOCKS;
 *   SIP rows longer than that are refused with BSA_ERR_SIZE.)
 * mode BSA_PLAN_TOPK: the s largest scores, ties to the lowest index, pi = 1,
 *   count = s.
 *
 * scores   [B,H,nQB,M] fp32, finite and >= 0.
 * budget   s, 1 <= s <= M.
 * seed     used when offsets == NULL: U of row r = (b*H + h)*nQB + i is
 *          bsa_sampling_offset(seed, r).
 * offsets  optional [B*H*nQB] uint64 offsets U, each < 2^44 - 2^16.
 * idx      out: [B,H,nQB,budget] int32, the drawn blocks in ascending order,
 *          entries beyond count set to -1.
 * bias     out: [B,H,nQB,budget] fp32 logit shift -ln(pi_j) of each drawn
 *          block (0 for top-k and for saturated blocks), 0 beyond count.
 *          May be NULL.
 * count    out: [B,H,nQB] int32 blocks drawn.  A row holding a NaN, an
 *          infinity or a negative score gets count = -1 and no blocks
 *          (bsa_attn_fwd then gives its queries zero outputs).
 * lambda   optional out (NULL = not written): [B,H,nQB] fp64; +inf when
 *          every positive block is taken, 0 for top-k, NaN for an invalid
 *          row.
 * status   optional out (NULL = not written): one device int32, set to
 *          BSA_OK by the call and to BSA_ERR_NONFINITE if any row was
 *          invalid, so that a caller can check a whole call with one read
 *          once the stream has reached it.
 * M        at most 2^20; in SIP mode at most BSA_SIP_MAX_BLOCKS.
 * The plan is caller-owned and stays valid for any number of later
 * bsa_attn_fwd calls (the page rebuilds it every 4 denoising steps).
 * --------------------------------------------------------------------- */
#define BSA_SIP_MAX_BLOCKS 65024

int bsa_sip_plan(const float *scores, int B, int H, int nQB, int M, int budget, int mode,
                 uint64_t seed, const uint64_t *offsets, int32_t *idx, float *bias,
                 int32_t *count, double *lambda, int32_t *status, void *stream);

/* Host helper, no GPU needed: U = floor((x >> 20) * (2^44 - 2^16) / 2^44)
 * where x is output number `row` (0-based) of SplitMix64 (Steele, Lea and
 * Flood 2014) seeded with `seed`. */
uint64_t bsa_sampling_offset(uint64_t seed, uint64_t row);

/* ------------------------------------------------------------------------
 * Fused sparse attention (AB-Attention page, section "전제와 한계", first
 * paragraph; the shift of section "어떻게 쓰나").
 *
 * For query row n of query block i = n / q_block of (b, h):
 *   keys  = tokens j*kv_block + t (t < kv_block) of every listed block
 *           j = idx[b,h,i,e], e < count[b,h,i], with token index < Nk;
 *   logit = scale * q_n . k_t + bias[b,h,i,e]   (bias = -ln pi; NULL = 0);
 *   out_n = softmax(logits) . V_keys;  lse_n = ln sum exp(logits).
 *
 * q        [B,H,Nq,d] bf16.   k, v  [B,H,Nk,d] bf16.  16-byte aligned.
 * idx      [B,H,nQB,max_blocks] int32, nQB = ceil(Nq / q_block).  Order is
 *          free (ascending gives the best gather locality).  Entries outside
 *          [0, ceil(Nk / kv_block)) are skipped.
 * bias     optional [B,H,nQB,max_blocks] fp32 added to every logit of the
 *          listed block.
 * count    [B,H,nQB] int32, clamped to [0, max_blocks] (negative = 0).
 * scale    softmax_scale <= 0 selects 1/sqrt(d).
 * out      [B,H,Nq,d] bf16 (round to nearest even).  A row with no valid
 *          key gets zeros (and lse = -inf).
 * lse      optional [B,H,Nq] fp32 natural-log sum of exponentials.
 * --------------------------------------------------------------------- */
int bsa_attn_fwd(const void *q, const void *k, const void *v, int B, int H, int Nq, int Nk,
                 int d, int q_block, int kv_block, const int32_t *idx, const float *bias,
                 const int32_t *count, int max_blocks, float softmax_scale, void *out,
                 float *lse, void *stream);

/* ------------------------------------------------------------------------
 * Backward of bsa_attn_fwd (AB-Attention page: the fused pass of section
 * "전제와 한계" with the shift of section "어떻게 쓰나"; the page's closing
 * paragraph names a trainable version, with a backward pass, as future
 * work).  With the plan and its shifts held fixed, the gradients of
 * sum(dout * out) for every query n of query block i and every gathered key
 * t (each listed occurrence of a block is its own set of keys):
 *   P_nt = exp(scale q_n . k_t + bias - lse_n),   D_n = dout_n . out_n,
 *   dS_nt = P_nt (dout_n . v_t - D_n),
 *   dq_n  = scale sum_t dS_nt k_t,
 *   dk_t += scale sum_n dS_nt q_n,   dv_t += sum_n P_nt dout_n.
 * q, k, v, idx, bias, count, Nq, Nk, kv_block, max_blocks and
 * softmax_scale are those of the forward call; out [B,H,Nq,d] bf16 and
 * lse [B,H,Nq] fp32 are its outputs (P is recomputed from lse; a row with
 * lse = -inf gets zero gradients); dout [B,H,Nq,d] bf16.
 * dq [B,H,Nq,d], dk, dv [B,H,Nk,d] fp32 (16-byte aligned, three distinct
 * buffers: BSA_ERR_ARG if two are the same); dk and dv are zeroed by the
 * call and accumulated with atomic adds, so their last bits may differ from
 * run to run.  d in {64, 128}.
 * --------------------------------------------------------------------- */
int bsa_attn_bwd(const void *q, const void *k, const void *v, const void *out, const void *dout,
                 const float *lse, int B, int H, int Nq, int Nk, int d, int q_block, int kv_block,
                 const int32_t *idx, const float *bias, const int32_t *count, int max_blocks,
                 float softmax_scale, float *dq, float *dk, float *dv, void *stream);

/* ------------------------------------------------------------------------
 * The same gradients as bsa_attn_bwd (same definition, arguments and
 * outputs), with no atomic adds.  Query blocks 2m and 2m + 1 of a (b, h)
 * run together over the union of their lists: a block both list is one
 * entry whose keys meet all 256 queries (each block's queries under its
 * own entry's shift), and each union entry's dK and dV rows go into one
 * slot of the caller's workspace.  When the two lists are not both valid
 * and strictly ascending below their counts (the plans of bsa_sip_plan
 * are), or hold more than 4,096 entries, the union is simply the first
 * list followed by the second.  One pass per KV block then sums the slots
 * of every union entry that lists it and writes dk and dv (every row; zero
 * for a block no query block lists), summing a block's slots in
 * ascending slot order, so dk and dv are the same bits on every run and
 * for any workspace size.
 *
 * bsa_attn_bwd_workspace_bytes (host, no GPU) reports the bytes one
 * (b, h) slab needs, with P = ceil(nQB / 2) pairs, U = 2 * max_blocks +
 * 3 * max(1, 128 / kv_block) union entries per pair:
 *   P * U * kv_block * 2 * d * 4        partial rows (fp32),
 * plus the key-major lists (4 * (2 (M + 1) + 2 P U): block ranges,
 * cursors, and each block's slots as filled and sorted), the union lists
 * (12 * P * U) and 16 * P bytes of class ends, each array padded to 64
 * elements.  The call processes as many slabs at a time as workspace_bytes
 * holds (all B*H when it holds that many) and returns BSA_ERR_WORKSPACE
 * when it holds less than one, or workspace is NULL; workspace must be
 * 256-byte aligned (BSA_ERR_ALIGN) and its contents are undefined after
 * the call.  P * U above 2^31 - 64, U * kv_block above 2^31 - 1, or
 * B * H * M above 2^33 (M = KV blocks of Nk), returns BSA_ERR_SIZE.  Other
 * errors are bsa_attn_bwd's.
 * --------------------------------------------------------------------- */
int bsa_attn_bwd_workspace_bytes(int Nq, int Nk, int d, int q_block, int kv_block,
                                 int max_blocks, size_t *bytes /* host out */);

int bsa_attn_bwd_ws(const void *q, const void *k, const void *v, const void *out,
                    const void *dout, const float *lse, int B, int H, int Nq, int Nk, int d,
                    int q_block, int kv_block, const int32_t *idx, const float *bias,
                    const int32_t *count, int max_blocks, float softmax_scale, float *dq,
                    float *dk, float *dv, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * BASA-structured lists (BASA page, onedev.kr/papers/688).
 *
 * Geometry: a latent grid T x Hg x Wg (token n = (t*Hg + y)*Wg + x) is
 * shifted cyclically by -(dy, dx) and cut into wh x ww spatial windows that
 * keep every frame (a ragged last window row/column keeps its smaller
 * size).  Window w of the shifted grid is laid out window-major: its tokens
 * in (t, shifted row, shifted column) order, padded with zero rows to a
 * multiple of 128, windows in row-major window order.  The pooled memory G
 * (per-frame non-overlapping ph x pw spatial means of K and V on the
 * unshifted grid, T * ceil(Hg/ph) * ceil(Wg/pw) tokens, raster order) is
 * appended after the last window in the key/value buffers (one KV block may
 * straddle the end: the attention kernel masks keys at or past Nk and reads
 * no row there).  Every query
 * window routes to the `topk` other windows with the largest
 * mean(Q_w) . mean(K_w') (fp32, fixed order: window-local token order sums,
 * one IEEE division, ascending-dim dot product without fused multiply-add;
 * ties to the lowest window).  The block list of a query block of window w
 * is: w's KV blocks, then each routed window's KV blocks (ascending window
 * id), then every pooled block; pi = 1 (no bias).
 *
 * bsa_basa_layout (host, no GPU) reports the sizes:
 *   nwin         number of windows;
 *   Nq_pad       padded query rows (= padded window-major rows);
 *   Nk           key/value rows: Nq_pad + pooled tokens;
 *   max_blocks   list stride;
 *   workspace    bytes of device scratch bsa_basa_plan needs.
 * kv_block must divide every window's token count and 128.
 *
 * bsa_basa_plan: q,k,v [B,H,N,d] bf16 -> qp [B,H,Nq_pad,d], kp, vp
 * [B,H,Nk,d] bf16 (caller-allocated), idx [B,H,Nq_pad/128,max_blocks]
 * int32 (unused tail entries -1), count [B,H,Nq_pad/128] int32, routes
 * optional [B,H,nwin,topk] int32 (rank order, best first).  Pad rows of qp,
 * kp and vp are zero.  topk <= min(64, nwin - 1).
 * Then bsa_attn_fwd(qp, kp, vp, B, H, Nq_pad, Nk, d, 128, kv_block,
 * idx, NULL, count, max_blocks, ...) and bsa_window_unpermute() give the
 * output in raster order.
 * --------------------------------------------------------------------- */
int bsa_basa_layout(int T, int Hg, int Wg, int d, int wh, int ww, int ph, int pw, int topk,
                    int kv_block, int B, int H, int *nwin, int *Nq_pad, int *Nk,
                    int *max_blocks, size_t *workspace /* all host out */);

int bsa_basa_plan(const void *q, const void *k, const void *v, int B, int H, int T, int Hg,
                  int Wg, int d, int wh, int ww, int dy, int dx, int ph, int pw, int topk,
                  int kv_block, void *qp, void *kp, void *vp, int32_t *idx, int32_t *count,
                  int32_t *routes, void *workspace, size_t workspace_bytes, void *stream);

int bsa_window_unpermute(const void *out_perm, void *out, int B, int H, int T, int Hg, int Wg,
                         int d, int wh, int ww, int dy, int dx, void *stream);

/* bsa_basa_plan_noalloc: bsa_basa_plan without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Arguments,
 * outputs and results are those of bsa_basa_plan.  Its scratch (the fp32
 * window means and the routes, the bytes bsa_basa_layout reports as
 * `workspace`) lives in a fixed device array of
 * BSA_BASA_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds
 * until the process ends; the call allocates and frees nothing.  A problem
 * whose scratch exceeds that size (B * H * nwin * (2 d + topk) * 4 bytes
 * plus alignment, so about 60 heads of the 66-window 1664x960 layout at
 * d = 128) returns BSA_ERR_SCRATCH before any HIP call.  Every call on a GPU
 * uses the same array: calls that overlap on one GPU (on different streams
 * or threads) race and must be serialised by the caller. */
#define BSA_BASA_NOALLOC_SCRATCH_BYTES (4u << 20)

int bsa_basa_plan_noalloc(const void *q, const void *k, const void *v, int B, int H, int T,
                          int Hg, int Wg, int d, int wh, int ww, int dy, int dx, int ph, int pw,
                          int topk, int kv_block, void *qp, void *kp, void *vp, int32_t *idx,
                          int32_t *count, int32_t *routes, void *stream);

/* ------------------------------------------------------------------------
 * BASA shift schedule (BASA page, section "어떻게 동작하나": the window
 * boundaries move from layer to layer and from denoising step to step).
 * Host helpers, no GPU; every pointer here is a HOST pointer.
 *
 * bsa_basa_offsets: the L per-layer offsets along an axis of window size w.
 *   Candidates a_i = (i * delta) mod w, delta = max(1, floor(w / L)),
 *   i = 0..L-1; the first half (a_0 .. a_{K-1}, K = ceil(L / 2)) and the
 *   second half alternate: offsets = (a_0, a_K, a_1, a_{K+1}, ...).  For
 *   w = 8, L = 4: (0, 2, 4, 6) -> (0, 4, 2, 6).  offsets [L] int.
 *
 * bsa_basa_shifts: the roll of layer l at step s,
 *   Delta_{l,s} = ((b^h_l + c^h_s) mod wh, (b^w_l + c^w_s) mod ww)
 *   with b^h = bsa_basa_offsets(wh, L), b^w = bsa_basa_offsets(ww, L) and
 *   caller-given per-step offsets c_h, c_w [S] (may be negative; NULL =
 *   zero).  dy, dx [L, S] int, row-major; pass (dy[l*S + s], dx[l*S + s])
 *   to bsa_basa_plan / bsa_window_unpermute of layer l at step s.
 * Errors: BSA_ERR_ARG for null outputs or w, wh, ww, L, S < 1.
 * --------------------------------------------------------------------- */
int bsa_basa_offsets(int w, int L, int *offsets /* host out */);

int bsa_basa_shifts(int wh, int ww, int L, int S, const int *c_h, const int *c_w,
                    int *dy, int *dx /* host out */);

/* ------------------------------------------------------------------------
 * Accuracy diagnostics (AB-Attention page, onedev.kr/papers/1521: section
 * "무엇과 다른가" compares the attention mass an oracle top-k keeps at
 * 128-token and 4-token KV blocks; section "어떻게 쓰나" compares SIP's
 * attention error with that of an oracle top-k).
 *
 * bsa_block_mass: true attention mass of every KV block for every query
 * block of (b, h):
 *   mass[b,h,i,j] = (1/n_i) sum_{n in query block i} sum_{t in block j, t < Nk}
 *                   exp(scale q_n . k_t - lse[b,h,n])
 * with n_i the block's query count.  lse [B,H,Nq] fp32 must be the dense
 * natural-log normaliser of each query (the lse output of bsa_attn_fwd with
 * every block listed and no bias); then every row of mass sums to 1.
 * q [B,H,Nq,d], k [B,H,Nk,d] bf16, 16-byte aligned; mass
 * [B,H,ceil(Nq/128),ceil(Nk/kv_block)] fp32.  q_block = 128; kv_block any
 * integer in [1, 1024] (not only powers of two); d in {64, 128};
 * softmax_scale <= 0 selects 1/sqrt(d).  Logits are bf16 products summed
 * in fp32 (matrix cores); exponentials and sums in fp32; the result is
 * deterministic.
 * --------------------------------------------------------------------- */
int bsa_block_mass(const void *q, const void *k, const float *lse, int B, int H, int Nq, int Nk,
                   int d, int q_block, int kv_block, float softmax_scale, float *mass,
                   void *stream);

/* bsa_plan_coverage: retained mass of a plan,
 *   coverage[r] = sum_{e < count[r]} mass[r, idx[r, e]]   (fp64, in list
 * order), for rows r of [rows, M] fp32 mass and [rows, max_blocks] int32
 * idx; count is clamped to [0, max_blocks] and entries outside [0, M) are
 * skipped.  coverage [rows] fp64. */
int bsa_plan_coverage(const float *mass, const int32_t *idx, const int32_t *count, int rows,
                      int M, int max_blocks, double *coverage, void *stream);

/* bsa_output_error: for each of `slabs` consecutive slabs of n bf16 values
 * (one head's [N, d] output: n = N * d), sums[2 s] = sum (out - ref)^2 and
 * sums[2 s + 1] = sum ref^2, fp64 (relative Frobenius error =
 * sqrt(sums[2 s] / sums[2 s + 1])).  n must be a multiple of 8; out and ref
 * 16-byte aligned; sums [slabs, 2] fp64.  Deterministic. */
int bsa_output_error(const void *out, const void *ref, int slabs, long long n, double *sums,
                     void *stream);

/* ------------------------------------------------------------------------
 * Measurement helper: throughput probe of the bf16 matrix instruction the
 * attention kernel uses (v_mfma_f32_32x32x16_bf16).  `workgroups` groups of
 * 4 waves each run `iters` rounds of 8 independent accumulations from
 * registers (no memory traffic); *flops (host out, may be NULL) receives the
 * flops of the call, workgroups * 4 * iters * 8 * 32768.  The rate the
 * matrix units sustain depends on the operand data (the clock drops under
 * the power of toggling operands), so `operands` selects:
 *   BSA_PROBE_RANDOM       random bf16 operands in +-[1/4, 4), four sets that
 *                          consecutive instructions alternate between (the
 *                          practical peak for real data, against which the
 *                          benchmark also states the attention kernel's
 *                          fraction, beside the published 2516.6 TFLOP/s);
 *   BSA_PROBE_LOW_ENTROPY  a few small operands with short mantissas, fixed
 *                          per lane (the most favourable case).
 * sink: one device float the kernel writes (its result keeps the
 * computation live).  Errors: BSA_ERR_ARG for a null sink, workgroups or
 * iters < 1 or an unknown mode.  Not part of the attention path.
 * --------------------------------------------------------------------- */
enum { BSA_PROBE_RANDOM = 0, BSA_PROBE_LOW_ENTROPY = 1 };

int bsa_mfma_peak_probe(int workgroups, int iters, int operands, float *sink,
                        long long *flops /* host out */, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H */
