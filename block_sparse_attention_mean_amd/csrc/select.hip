// IBCS selector kernels for gfx950: KV-block mean pooling, k-means inside
// each 128-query block, and the block-score GEMM with its softmax.
//
// AB-Attention page (onedev.kr/papers/1521), section "무엇과 다른가": queries
// are grouped in 128-token blocks and keys/values in small (4-token) blocks;
// one k-means iteration inside each query block gives 8 centroids and their
// query shares; a KV block's score is the share-weighted softmax mass of the
// centroids over the pooled keys.  The "전제와 한계" section adds that the
// selector scores many query/KV blocks in one batched matrix operation.
//
// Kernels:
//   pool_split  one wave per KV block: fp32 mean of its keys, then a split
//               into two fp16 halves with a per-row power-of-two scale
//               (x 2^e = hi + lo 2^-11, |x 2^e| < 2^11) so the GEMM below is
//               fp32-accurate on fp16 matrix cores;
//   kmeans      one workgroup per query block; fp32 in a fixed operation
//               order (ascending-row member sums, IEEE division, distances
//               summed over ascending dims without fused multiply-add) --
//               its assignments are discrete decisions and must be
//               reproducible bit for bit;
//   score<0>    sweep 1 of centroids x pooled keys (3 fp16 MFMA per product:
//               hi.hi + (hi.lo + lo.hi) 2^-11): per-row running max and sum
//               of 2^(logit log2 e), per column chunk;
//   score<1>    sweep 2: merges the chunk statistics into a per-row offset
//               beta = max + log2(sum) - log2(share), recomputes the same
//               logits bit for bit and writes S_ij = sum_c 2^(t_cj - beta_c)
//               with the cluster sum done in registers.
#include "common.h"

namespace bsa {

namespace {

typedef _Float16 half_t;

struct SelArgs {
  const uint16_t *q, *k;
  int N, M, nqb, C, iters, kv_shift, R, nchunk, chunk_cols, tiles;
  float *scores, *centroids, *weights;
  half_t *kb_hi, *kb_lo;
  float *kb_cs;
  half_t *ce_hi, *ce_lo;
  float *ce_rs, *ce_w;
  float2 *stats;
  float scale_log2;
};

// Split x (one row, this lane's share) at a row scale 2^e.
__device__ __forceinline__ void split_f16(float x, int e, half_t &hi, half_t &lo) {
  const float sc = ldexpf(x, e);
  hi = (half_t)sc;
  lo = (half_t)((sc - (float)hi) * 2048.f);
}

__device__ __forceinline__ int row_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int ex;
  frexpf(amax, &ex);  // amax in [2^(ex-1), 2^ex)
  int e = 11 - ex;    // amax * 2^e in [2^10, 2^11)
  return e < -100 ? -100 : (e > 100 ? 100 : e);
}

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ---------------------------------------------------------------- pooling
template <int D>
__global__ __launch_bounds__(256) void pool_split_kernel(SelArgs a) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int bh = blockIdx.y;
  if (j >= a.M) return;
  const int kvb = 1 << a.kv_shift;
  const int r0 = j * kvb;
  const int rows = min(kvb, a.N - r0);
  const uint16_t *kp = a.k + ((size_t)bh * a.N + r0) * D + lane * PER;
  float acc[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) acc[p] = 0.f;
  for (int t = 0; t < rows; ++t) {
#pragma unroll
    for (int p = 0; p < PER; ++p) acc[p] = __fadd_rn(acc[p], bf16_to_f32(kp[(size_t)t * D + p]));
  }
  float amax = 0.f;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    acc[p] = rows == kvb ? acc[p] * (1.0f / (float)kvb) : __fdiv_rn(acc[p], (float)rows);
    amax = fmaxf(amax, fabsf(acc[p]));
  }
  amax = wave_max_f(amax);
  const int e = row_exponent(amax);
  const size_t o = ((size_t)bh * a.M + j) * D + lane * PER;
#pragma unroll
  for (int p = 0; p < PER; ++p) split_f16(acc[p], e, a.kb_hi[o + p], a.kb_lo[o + p]);
  if (lane == 0) a.kb_cs[(size_t)bh * a.M + j] = ldexpf(1.f, -e);
}

// ---------------------------------------------------------------- k-means
// One workgroup per query block.  Member sums follow the stated order
// exactly: a stable counting sort lists each cluster's rows in ascending
// order, and one thread per (dim, cluster) adds them in that order.
template <int D>
__global__ __launch_bounds__(256) void kmeans_kernel(SelArgs a) {
  constexpr int QS = D + 8;  // padded bf16 row stride (16-byte aligned rows)
  __shared__ __attribute__((aligned(16))) uint16_t qb16[128 * QS];
  __shared__ __attribute__((aligned(16))) float mu[16 * D];
  __shared__ int asg[128];
  __shared__ int order[128];  // rows sorted by cluster, ascending within
  __shared__ int cnt[16], off[16];
  __shared__ int active[16];
  __shared__ unsigned long long masks[2][16];

  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int qb = blockIdx.x, bh = blockIdx.y;
  const int C = a.C;
  const int n = min(128, a.N - qb * 128);
  const uint16_t *qp = a.q + ((size_t)bh * a.N + (size_t)qb * 128) * D;

  // 16-byte loads of the block into padded rows
  for (int e = t; e < n * (D / 8); e += 256) {
    const int r = e / (D / 8), c8 = e % (D / 8);
    st16(&qb16[r * QS + c8 * 8], ld16(qp + (size_t)r * D + c8 * 8));
  }
  for (int e = t; e < 16 * D; e += 256) mu[e] = 0.f;
  if (t < 16) active[t] = (t < C) && (((t + 1) * n) / C > (t * n) / C);
  if (t < n) {
    int c = 0;
    while (c + 1 < C && ((c + 1) * n) / C <= t) ++c;  // segment of row t
    asg[t] = c;
  }
  __syncthreads();

  auto q_at = [&](int r, int k) -> float { return bf16_to_f32(qb16[r * QS + k]); };

  // counts, offsets and the stable order of rows by cluster, then means
  auto update_means = [&]() {
    if (w < 2) {
      const int r = w * 64 + lane;
      const int c = r < n ? asg[r] : -1;
      for (int k = 0; k < C; ++k) {
        const unsigned long long m = __builtin_amdgcn_ballot_w64(c == k);
        if (lane == 0) masks[w][k] = m;
      }
    }
    __syncthreads();
    if (t == 0) {
      int o = 0;
      for (int k = 0; k < C; ++k) {
        const int c0 = __builtin_popcountll(masks[0][k]), c1 = __builtin_popcountll(masks[1][k]);
        cnt[k] = c0 + c1;
        off[k] = o;
        o += c0 + c1;
      }
    }
    __syncthreads();
    if (w < 2) {
      const int r = w * 64 + lane;
      if (r < n) {
        const int c = asg[r];
        const unsigned long long below = lane ? (~0ull >> (64 - lane)) : 0ull;
        int rank = __builtin_popcountll(masks[w][c] & below);
        if (w == 1) rank += __builtin_popcountll(masks[0][c]);
        order[off[c] + rank] = r;
      }
    }
    __syncthreads();
    // thread (dim, cluster group): clusters g, g + G, ... for G = 256 / D
    constexpr int G = 256 / D;
    const int dim = t % D, g = t / D;
    for (int c = g; c < C; c += G) {
      const int m = cnt[c];
      if (m == 0) continue;  // empty cluster keeps its centroid
      float acc = 0.f;
      const int o = off[c];
      for (int i = 0; i < m; ++i) acc = __fadd_rn(acc, q_at(order[o + i], dim));
      mu[c * D + dim] = __fdiv_rn(acc, (float)m);
    }
    __syncthreads();
  };

  update_means();
  for (int it = 0; it < a.iters; ++it) {
    // distances: thread (row r = t >> 1, cluster parity t & 1)
    const int r = t >> 1, par = t & 1;
    float best = __builtin_inff();
    int bc = 1 << 30;
    if (r < n) {
      for (int c = par; c < C; c += 2) {
        if (!active[c]) continue;
        float dd = 0.f;
        for (int k0 = 0; k0 < D; k0 += 8) {
          const u32x4 qv = *(const u32x4 *)&qb16[r * QS + k0];
          const f32x4 m0 = *(const f32x4 *)&mu[c * D + k0];
          const f32x4 m1 = *(const f32x4 *)&mu[c * D + k0 + 4];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const unsigned word = qv[e >> 1];
            const float qx = __builtin_bit_cast(float, (e & 1) ? (word & 0xffff0000u) : (word << 16));
            const float df = __fsub_rn(qx, e < 4 ? m0[e] : m1[e - 4]);
            dd = __fadd_rn(dd, __fmul_rn(df, df));
          }
        }
        if (dd < best) {
          best = dd;
          bc = c;
        }
      }
    }
    const float ob = __shfl_xor(best, 1, 64);
    const int oc = __shfl_xor(bc, 1, 64);
    if (ob < best || (ob == best && oc < bc)) {
      best = ob;
      bc = oc;
    }
    __syncthreads();
    if (r < n && par == 0) asg[r] = bc;
    __syncthreads();
    update_means();
  }

  // outputs: fp32 centroids / shares (optional) and the fp16 split for the GEMM
  const size_t rbase = ((size_t)bh * a.nqb + qb) * C;
  if (a.weights && t < C) a.weights[rbase + t] = __fdiv_rn((float)cnt[t], (float)n);
  if (a.centroids)
    for (int e = t; e < C * D; e += 256) a.centroids[rbase * D + e] = mu[e];
  // one wave per cluster row for the split
  constexpr int PER = D / 64;
  for (int c = w; c < C; c += 4) {
    float amax = 0.f;
#pragma unroll
    for (int p = 0; p < PER; ++p) amax = fmaxf(amax, fabsf(mu[c * D + lane * PER + p]));
    amax = wave_max_f(amax);
    const int e = row_exponent(amax);
    const size_t o = (rbase + c) * D + lane * PER;
#pragma unroll
    for (int p = 0; p < PER; ++p) split_f16(mu[c * D + lane * PER + p], e, a.ce_hi[o + p], a.ce_lo[o + p]);
    if (lane == 0) {
      a.ce_rs[rbase + c] = ldexpf(a.scale_log2, -e);
      a.ce_w[rbase + c] = __fdiv_rn((float)cnt[c], (float)n);
    }
  }
}

// ---------------------------------------------------------------- scores
// MFMA row i of a 32-row sub-tile -> local row so that lane half h,
// register r holds local row 16 h + r.
__device__ __forceinline__ int local_row(int i) {
  return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
}

template <int D, int PASS>
__global__ __launch_bounds__(256) void score_kernel(SelArgs a) {
  constexpr int KS = D / 16;
  constexpr int BSTR = D + 8;  // LDS row stride (halves)
  constexpr int CT = 64;       // columns per step
  __shared__ __attribute__((aligned(16))) half_t bhi[CT * BSTR];
  __shared__ __attribute__((aligned(16))) half_t blo[CT * BSTR];
  __shared__ float bcs[CT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int tile = blockIdx.x / a.nchunk, chunk = blockIdx.x % a.nchunk;
  const int bh = blockIdx.y;
  const int R = a.R, M = a.M, C = a.C;
  const int rho0 = tile * 128 + wave * 32;

  // A operand: centroid rows (hi, lo)
  f16x8 ahi[KS], alo[KS];
  {
    const int rho = rho0 + local_row(l32);
    const bool ok = rho < R;
    const size_t o = ((size_t)bh * R + (ok ? rho : 0)) * D + hh * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 vh = {0u, 0u, 0u, 0u}, vl = {0u, 0u, 0u, 0u};
      if (ok) {
        vh = ld16(a.ce_hi + o + ks * 16);
        vl = ld16(a.ce_lo + o + ks * 16);
      }
      ahi[ks] = as_f16x8(vh);
      alo[ks] = as_f16x8(vl);
    }
  }
  // per-lane rows 16 hh + r
  float rs[16];
  float stA[16], stB[16];  // PASS 0: running max / sum ; PASS 1: beta
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rho = rho0 + 16 * hh + r;
    rs[r] = rho < R ? a.ce_rs[(size_t)bh * R + rho] : 0.f;
    stA[r] = -__builtin_inff();
    stB[r] = 0.f;
  }
  if (PASS == 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rho = rho0 + 16 * hh + r;
      float beta = __builtin_inff();
      if (rho < R) {
        float m = -__builtin_inff();
        for (int c = 0; c < a.nchunk; ++c)
          m = fmaxf(m, a.stats[((size_t)bh * a.nchunk + c) * R + rho].x);
        float z = 0.f;
        for (int c = 0; c < a.nchunk; ++c) {
          const float2 p = a.stats[((size_t)bh * a.nchunk + c) * R + rho];
          if (p.x != -__builtin_inff()) z += p.y * __builtin_amdgcn_exp2f(p.x - m);
        }
        const float w = a.ce_w[(size_t)bh * R + rho];
        if (w > 0.f && z > 0.f) beta = m + __builtin_log2f(z) - __builtin_log2f(w);
      }
      stA[r] = beta;
    }
  }

  const int c0 = chunk * a.chunk_cols;
  const int c1 = min(M, c0 + a.chunk_cols);
  for (int cb = c0; cb < c1; cb += CT) {
    __syncthreads();
    // stage CT columns of the pooled-key split into LDS
    constexpr int CH = D / 8;
    for (int e = tid; e < CT * CH; e += 256) {
      const int col = e / CH, ch = e % CH;
      const int j = cb + col;
      u32x4 vh = {0u, 0u, 0u, 0u}, vl = {0u, 0u, 0u, 0u};
      if (j < c1) {
        const size_t o = ((size_t)bh * M + j) * D + ch * 8;
        vh = ld16(a.kb_hi + o);
        vl = ld16(a.kb_lo + o);
      }
      st16(&bhi[col * BSTR + ch * 8], vh);
      st16(&blo[col * BSTR + ch * 8], vl);
    }
    if (tid < CT) bcs[tid] = (cb + tid < c1) ? a.kb_cs[(size_t)bh * M + cb + tid] : 0.f;
    __syncthreads();

    float tv[2][16];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      f32x16 acc0, acc1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc0[r] = 0.f;
        acc1[r] = 0.f;
      }
      const int col = tt * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const f16x8 bh16 = as_f16x8(ld16(&bhi[col * BSTR + ks * 16 + hh * 8]));
        const f16x8 bl16 = as_f16x8(ld16(&blo[col * BSTR + ks * 16 + hh * 8]));
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[ks], bh16, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[ks], bl16, acc1, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[ks], bh16, acc1, 0, 0, 0);
      }
      const bool valid = cb + col < c1;
      const float cs = bcs[col];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float v = __builtin_fmaf(acc1[r], 0x1p-11f, acc0[r]);
        tv[tt][r] = valid ? (v * rs[r]) * cs : -__builtin_inff();
      }
    }

    if (PASS == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float mt = fmaxf(tv[0][r], tv[1][r]);
        const float mn = fmaxf(stA[r], mt);
        if (mn != -__builtin_inff()) {
          stB[r] = stB[r] * __builtin_amdgcn_exp2f(stA[r] - mn) +
                   __builtin_amdgcn_exp2f(tv[0][r] - mn) + __builtin_amdgcn_exp2f(tv[1][r] - mn);
          stA[r] = mn;
        }
      }
    } else {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int j = cb + tt * 32 + l32;
        const bool valid = j < c1;
#pragma unroll
        for (int g = 0; g < 16; g += 1) {
          if (g % C) continue;  // groups of C registers = one query block
          float sacc = 0.f;
          for (int q2 = 0; q2 < C; ++q2) sacc += __builtin_amdgcn_exp2f(tv[tt][g + q2] - stA[g + q2]);
          const int rho = rho0 + 16 * hh + g;
          const int qbk = rho / C;
          if (valid && rho < R) a.scores[((size_t)bh * a.nqb + qbk) * M + j] = sacc;
        }
      }
    }
  }

  if (PASS == 0) {
    // merge the 32 lanes of each half (same rows, different columns)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float m = stA[r], z = stB[r];
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) {
        const float m2 = __shfl_xor(m, o, 64);
        const float z2 = __shfl_xor(z, o, 64);
        const float mn = fmaxf(m, m2);
        if (mn != -__builtin_inff()) {
          const float za = m == -__builtin_inff() ? 0.f : z * __builtin_amdgcn_exp2f(m - mn);
          const float zb = m2 == -__builtin_inff() ? 0.f : z2 * __builtin_amdgcn_exp2f(m2 - mn);
          z = za + zb;
          m = mn;
        }
      }
      stA[r] = m;
      stB[r] = z;
    }
    if (l32 == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rho = rho0 + 16 * hh + r;
        if (rho < R) a.stats[((size_t)bh * a.nchunk + chunk) * R + rho] = make_float2(stA[r], stB[r]);
      }
    }
  }
}

struct Layout {
  size_t kb_hi, kb_lo, kb_cs, ce_hi, ce_lo, ce_rs, ce_w, stats, total;
  int nqb, M, R, nchunk, chunk_cols, tiles;
};

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

Layout make_layout(int B, int H, int N, int d, int kv_block, int C) {
  Layout L;
  const size_t BH = (size_t)B * H;
  L.nqb = (N + 127) / 128;
  L.M = (N + kv_block - 1) / kv_block;
  L.R = L.nqb * C;
  L.tiles = (L.R + 127) / 128;
  // column chunks: enough workgroups to fill the chip, whole 64-column steps
  const long long wg = (long long)L.tiles * (long long)BH;
  int nchunk = (int)((2048 + wg - 1) / wg);
  const int steps = (L.M + 63) / 64;
  if (nchunk < 1) nchunk = 1;
  if (nchunk > steps) nchunk = steps;
  if (nchunk > 64) nchunk = 64;
  L.chunk_cols = ((steps + nchunk - 1) / nchunk) * 64;
  L.nchunk = (L.M + L.chunk_cols - 1) / L.chunk_cols;
  size_t off = 0;
  L.kb_hi = off; off += al256(BH * L.M * d * 2);
  L.kb_lo = off; off += al256(BH * L.M * d * 2);
  L.kb_cs = off; off += al256(BH * L.M * 4);
  L.ce_hi = off; off += al256(BH * L.R * d * 2);
  L.ce_lo = off; off += al256(BH * L.R * d * 2);
  L.ce_rs = off; off += al256(BH * L.R * 4);
  L.ce_w = off; off += al256(BH * L.R * 4);
  L.stats = off; off += al256(BH * (size_t)L.nchunk * L.R * 8);
  L.total = off;
  return L;
}

}  // namespace

size_t select_workspace_bytes(int B, int H, int N, int d, int kv_block, int n_clusters) {
  return make_layout(B, H, N, d, kv_block, n_clusters).total;
}

int launch_select_scores(const void *q, const void *k, int B, int H, int N, int d, int kv_block,
                         int n_clusters, int kmeans_iters, float *scores, float *centroids,
                         float *weights, void *workspace, hipStream_t stream) {
  if (n_clusters & (n_clusters - 1)) return BSA_ERR_UNSUPPORTED;  // 1, 2, 4, 8, 16
  const Layout L = make_layout(B, H, N, d, kv_block, n_clusters);
  char *ws = (char *)workspace;
  SelArgs a;
  a.q = (const uint16_t *)q;
  a.k = (const uint16_t *)k;
  a.N = N;
  a.M = L.M;
  a.nqb = L.nqb;
  a.C = n_clusters;
  a.iters = kmeans_iters;
  a.kv_shift = __builtin_ctz((unsigned)kv_block);
  a.R = L.R;
  a.nchunk = L.nchunk;
  a.chunk_cols = L.chunk_cols;
  a.tiles = L.tiles;
  a.scores = scores;
  a.centroids = centroids;
  a.weights = weights;
  a.kb_hi = (half_t *)(ws + L.kb_hi);
  a.kb_lo = (half_t *)(ws + L.kb_lo);
  a.kb_cs = (float *)(ws + L.kb_cs);
  a.ce_hi = (half_t *)(ws + L.ce_hi);
  a.ce_lo = (half_t *)(ws + L.ce_lo);
  a.ce_rs = (float *)(ws + L.ce_rs);
  a.ce_w = (float *)(ws + L.ce_w);
  a.stats = (float2 *)(ws + L.stats);
  a.scale_log2 = kLog2e / sqrtf((float)d);
  const unsigned BH = (unsigned)(B * H);
  const dim3 gpool((L.M + 3) / 4, BH), gkm(L.nqb, BH), gsc(L.tiles * L.nchunk, BH);
  if (d == 128) {
    hipLaunchKernelGGL(pool_split_kernel<128>, gpool, dim3(256), 0, stream, a);
    hipLaunchKernelGGL(kmeans_kernel<128>, gkm, dim3(256), 0, stream, a);
    hipLaunchKernelGGL((score_kernel<128, 0>), gsc, dim3(256), 0, stream, a);
    hipLaunchKernelGGL((score_kernel<128, 1>), gsc, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(pool_split_kernel<64>, gpool, dim3(256), 0, stream, a);
    hipLaunchKernelGGL(kmeans_kernel<64>, gkm, dim3(256), 0, stream, a);
    hipLaunchKernelGGL((score_kernel<64, 0>), gsc, dim3(256), 0, stream, a);
    hipLaunchKernelGGL((score_kernel<64, 1>), gsc, dim3(256), 0, stream, a);
  }
  return status_of(hipGetLastError());
}

}  // namespace bsa
