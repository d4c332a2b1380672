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
//   pool_split  one workgroup per 32 KV blocks (one key tile of the GEMM):
//               fp32 mean of each block's keys, then a split into two fp16
//               halves at one power-of-two scale per tile
//               (x 2^e = hi + lo, |x 2^e| < 2^11, lo the fp16 rounding of
//               the remainder) so the GEMM below is fp32-accurate on fp16
//               matrix cores;
//   kmeans      one workgroup per query block; fp32 in a fixed operation
//               order (ascending-row member sums, IEEE division, distances
//               summed over ascending dims without fused multiply-add) --
//               its assignments are discrete decisions and must be
//               reproducible bit for bit;
//   score<0>    sweep 1 of pooled keys x centroids (3 fp16 MFMA per product,
//               hi.lo + hi.hi + lo.hi, into one fp32 accumulator): per-row
//               running max and sum of 2^(logit log2 e), per column chunk;
//   score<1>    sweep 2: merges the chunk statistics into a per-row offset
//               beta = max + log2(sum) - log2(share), recomputes the same
//               logits bit for bit and writes S_ij = sum_c 2^(t_cj - beta_c)
//               with the cluster sum done across lanes.
#include <type_traits>

#include "common.h"

namespace bsa {

namespace {

typedef _Float16 half_t;

struct SelArgs {
  const uint16_t *q, *k;
  int N, M, nqb, C, iters, kv_shift, R, nchunk, chunk_cols, tiles, ktiles;
  float *scores, *centroids, *weights;
  half_t *kb_hi, *kb_lo;
  float *kb_cs;
  float *ce_f, *ce_w;
  float2 *stats;
  float scale_log2;
};

// Split x (one row, this lane's share) at a row scale 2^e: x 2^e = hi + r
// exactly in fp32, and lo = fp16(r).  With |x 2^e| < 2^11, |r| <= 1/2 ulp
// of hi keeps 11 bits in lo down to |x 2^e| ~ 2^-3 (2^-13 of the row's
// largest value); below that r is an fp16 subnormal, with an absolute error
// under 2^-25 that the dot products cannot see.
__device__ __forceinline__ void split_f16(float x, int e, half_t &hi, half_t &lo) {
  const float sc = ldexpf(x, e);
  hi = (half_t)sc;
  lo = (half_t)(sc - (float)hi);
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
// One workgroup per key tile of 32 KV blocks; wave w pools blocks 8 w .. 8 w + 7
// of the tile, lane l holding dims l PER .. l PER + PER - 1.
template <int D>
__global__ __launch_bounds__(256) void pool_split_kernel(SelArgs a) {
  constexpr int PER = D / 64;
  __shared__ float wmax[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int tile = blockIdx.x, bh = blockIdx.y;
  const int kvb = 1 << a.kv_shift;
  float acc[8][PER];
  int rows[8];
  const uint16_t *kp[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = tile * 32 + w * 8 + i;
    const int r0 = j * kvb;
    rows[i] = j < a.M ? min(kvb, a.N - r0) : 0;
    kp[i] = a.k + ((size_t)bh * a.N + (j < a.M ? r0 : 0)) * D + lane * PER;
#pragma unroll
    for (int p = 0; p < PER; ++p) acc[i][p] = 0.f;
  }
  // rows t0 .. t0 + 3 of all 8 blocks are loaded before any is added, so
  // a wave waits for memory once per batch; the sums keep ascending row
  // order.  Loads past a block's rows re-read its row 0 (always present)
  // and are not added.
  for (int t0 = 0; t0 < kvb; t0 += 4) {
    uint16_t v[8][4][PER];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int tt = t0 + u < rows[i] ? t0 + u : 0;
#pragma unroll
        for (int p = 0; p < PER; ++p) v[i][u][p] = kp[i][(size_t)tt * D + p];
      }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (t0 + u < rows[i]) {
#pragma unroll
          for (int p = 0; p < PER; ++p) acc[i][p] = __fadd_rn(acc[i][p], bf16_to_f32(v[i][u][p]));
        }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (rows[i] > 0) {
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        acc[i][p] = rows[i] == kvb ? acc[i][p] * (1.0f / (float)kvb) : __fdiv_rn(acc[i][p], (float)rows[i]);
        amax = fmaxf(amax, fabsf(acc[i][p]));
      }
    }
  }
  amax = wave_max_f(amax);
  if (lane == 0) wmax[w] = amax;
  __syncthreads();
  const int e = row_exponent(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3])));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = tile * 32 + w * 8 + i;
    if (j < a.M) {
      const size_t o = ((size_t)bh * a.M + j) * D + lane * PER;
#pragma unroll
      for (int p = 0; p < PER; ++p) split_f16(acc[i][p], e, a.kb_hi[o + p], a.kb_lo[o + p]);
    }
  }
  if (threadIdx.x == 0) a.kb_cs[(size_t)bh * a.ktiles + tile] = ldexpf(1.f, -e);
}

// ---------------------------------------------------------------- k-means
// One workgroup per query block.  Member sums follow the stated order
// exactly: a stable counting sort lists each cluster's rows in ascending
// order, and one thread per (dim, cluster) adds them in that order.
// CMAX bounds the cluster count: with CMAX = 8 the workgroup's LDS stays
// under 40 KB, so four workgroups share a CU instead of three.
template <int D, int CMAX>
__global__ __launch_bounds__(256) void kmeans_kernel(SelArgs a) {
  constexpr int QS = D + 8;  // padded bf16 row stride (16-byte aligned rows)
  __shared__ __attribute__((aligned(16))) uint16_t qb16[128 * QS];
  __shared__ __attribute__((aligned(16))) float mu[CMAX * D];
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

  // 16-byte loads of the block into padded rows, all issued before the
  // first LDS store
  {
    constexpr int PER = 128 * (D / 8) / 256;  // chunks per thread
    u32x4 v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {  // rows past n re-read row n - 1 and are not stored
      const int e = t + i * 256, r = min(e / (D / 8), n - 1), c8 = e % (D / 8);
      v[i] = ld16(qp + (size_t)r * D + c8 * 8);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = t + i * 256, r = e / (D / 8), c8 = e % (D / 8);
      if (r < n) st16(&qb16[r * QS + c8 * 8], v[i]);
    }
  }
  for (int e = t; e < CMAX * D; e += 256) mu[e] = 0.f;
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
      // members fetched 8 at a time (their row indices, then their values),
      // so the chain waits for LDS twice per 8 adds; the adds keep the
      // ascending member order
      int i = 0;
      for (; i + 8 <= m; i += 8) {
        int rr[8];
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) rr[u] = order[o + i + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = q_at(rr[u], dim);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc = __fadd_rn(acc, x[u]);
      }
      for (; i < m; ++i) acc = __fadd_rn(acc, q_at(order[o + i], dim));
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
      // this thread's clusters c = par, par + 2, .. side by side: one
      // independent chain each (dims ascending), sharing the query loads
      constexpr int NJ = CMAX / 2;
      float dd[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) dd[j] = 0.f;
      for (int k0 = 0; k0 < D; k0 += 8) {
        const u32x4 qv = *(const u32x4 *)&qb16[r * QS + k0];
        float qx[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const unsigned word = qv[e >> 1];
          qx[e] = __builtin_bit_cast(float, (e & 1) ? (word & 0xffff0000u) : (word << 16));
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int c = par + 2 * j;
          if (c >= C) break;  // uniform
          const f32x4 m0 = *(const f32x4 *)&mu[c * D + k0];
          const f32x4 m1 = *(const f32x4 *)&mu[c * D + k0 + 4];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float df = __fsub_rn(qx[e], e < 4 ? m0[e] : m1[e - 4]);
            dd[j] = __fadd_rn(dd[j], __fmul_rn(df, df));
          }
        }
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int c = par + 2 * j;
        if (c < C && active[c] && dd[j] < best) {
          best = dd[j];
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

  // outputs: fp32 centroids and shares for the score GEMM (and the caller)
  const size_t rbase = ((size_t)bh * a.nqb + qb) * C;
  if (t < C) {
    const float share = __fdiv_rn((float)cnt[t], (float)n);
    a.ce_w[rbase + t] = share;
    if (a.weights) a.weights[rbase + t] = share;
  }
  for (int e = t; e < C * D; e += 256) {
    a.ce_f[rbase * D + e] = mu[e];
    if (a.centroids) a.centroids[rbase * D + e] = mu[e];
  }
}

// ---------------------------------------------------------------- scores
typedef __attribute__((address_space(3))) void lds_void_t;

// 16-byte-chunk XOR swizzle of the pooled-key tiles: the operand read
// (32 rows x one chunk per half-wave) is bank-conflict free.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}

template <int N>
__device__ __forceinline__ void sc_ring_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// x + (x of the lane n below, inside each row of 16 lanes)
template <int N>
__device__ __forceinline__ float add_shr(float x) {
  const int y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xf, 0xf, false);
  return x + __builtin_bit_cast(float, y);
}

// The lane's index, recomputed where it is used (two ALU instructions):
// values derived from it and kept live through the key loop would take
// registers the products need, or be spilled and reloaded behind a wait on
// every outstanding load.
__device__ __forceinline__ int fresh_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Workgroups are dealt to the 8 XCDs round-robin; renumber them so that a
// contiguous range of logical ids (the row tiles sharing one key chunk) runs
// on one XCD and its L2.
__device__ __forceinline__ int xcd_order(int L, int total) {
  const int q = total >> 3, rem = total & 7, x = L & 7;
  return x * q + min(x, rem) + (L >> 3);
}

// One workgroup = 256 centroid rows (4 waves x 64) x one column chunk.  The
// product is taken transposed, D[key][centroid] = K_tile . C^T: the pooled-key
// split tiles (32 keys, hi and lo) stream through a four-slot LDS ring filled
// by direct global->LDS loads and feed the A operand, while each wave keeps
// its 64 centroid rows (two 32-row sub-tiles) split in registers as the B
// operand.  Lane l then owns centroid row l % 32 of each sub-tile and 16 of
// the 32 keys of a step, so the row statistics are two registers.  Sweep 2
// at 8 clusters swaps the two operands (D[centroid][key], see TR below) so
// that a query block's clusters share a lane.  PASS is the sweep; CL =
// log2 of the clusters per query block, the levels of sweep 2's cross-lane
// cluster sum at other cluster counts (0 in sweep 1).
template <int D, int PASS, int CL>
__global__ __launch_bounds__(256, 2) void score_kernel(SelArgs a) {
  constexpr int KS = D / 16;
  constexpr int CT = 32;               // keys per step
  constexpr int NB = 4;                // ring slots
  constexpr int ROWB = D * 2;          // bytes of one fp16 row
  constexpr int TB = CT * ROWB;        // bytes of one hi (or lo) tile
  constexpr int NCH = D / 8;           // 16-byte chunks per row
  constexpr int RPI = 64 / NCH;        // rows per 1 KB wave load
  constexpr int LOADS = 2 * CT / RPI;  // wave loads per step (hi + lo)
  constexpr int LPW = LOADS / 4;       // per wave
  static_assert(LPW >= 1 && LOADS % 4 == 0, "step shape");
  // the ring, one array: slot S holds the hi tile at 2 S TB and the lo tile
  // at (2 S + 1) TB, so both offsets fold into the LDS instructions
  __shared__ __attribute__((aligned(16))) unsigned char ring[2 * NB * TB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int id = xcd_order(blockIdx.x, gridDim.x);
  const int tile = id % a.tiles;
  const int rest = id / a.tiles;
  const int chunk = rest % a.nchunk, bh = rest / a.nchunk;
  const int R = a.R, M = a.M, C = a.C;
  const int rho0 = tile * 256 + wave * 64;
  const int cbeg = chunk * a.chunk_cols;
  const int cend = min(M, cbeg + a.chunk_cols);
  const int nsteps = (cend - cbeg + CT - 1) / CT;
  const unsigned char *khi = (const unsigned char *)(a.kb_hi + (size_t)bh * M * D);
  const unsigned char *klo = (const unsigned char *)(a.kb_lo + (size_t)bh * M * D);
  // key-tile scales, read through the constant address space so that the
  // uniform per-step read is a scalar load: a vector load here would have to
  // wait for the ring's outstanding tile loads
  typedef const __attribute__((address_space(4))) float cfloat_t;
  cfloat_t *kcs = (cfloat_t *)(a.kb_cs + (size_t)bh * a.ktiles + cbeg / CT);

  auto hslot = [&](auto c) -> unsigned char * { return ring + 2 * decltype(c)::value * TB; };
  auto lslot = [&](auto c) -> unsigned char * { return ring + (2 * decltype(c)::value + 1) * TB; };

  // gather of step k into slot S: wave loads u = wave * LPW + j, each lane
  // one 16-byte chunk at a fixed offset inside the 32-key tile.  Keys past
  // the chunk end (ragged last step) read the next rows or the 32-row pad
  // after the split arrays and are masked in the epilogue.
  const unsigned rd_base = (unsigned)(l32 * ROWB + ((hh ^ swz_k<D>(l32)) << 4));
  unsigned koff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int u = wave * LPW + j;
    const int r = (u % (LOADS / 2)) * RPI + lane / NCH;  // tile row
    koff[j] = (unsigned)(r * ROWB + (((lane % NCH) ^ swz_k<D>(r)) << 4));
  }
  auto issue = [&](auto slot_c, int k) {
    unsigned char *ht = hslot(slot_c);
    unsigned char *lt = lslot(slot_c);
    const size_t tile_off = (size_t)(cbeg + k * CT) * ROWB;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int u = wave * LPW + j;
      const bool hi = u < LOADS / 2;
      const int dst = (u % (LOADS / 2)) * RPI * ROWB;  // wave-uniform
      // the empty asm keeps the lane offset a 32-bit register added to a
      // scalar base at each load, instead of a 64-bit address per load
      // hoisted out of the loop (registers the products need)
      unsigned o = koff[j];
      asm volatile("" : "+v"(o));
      __builtin_amdgcn_global_load_lds((const void *)((hi ? khi : klo) + tile_off + o),
                                       (lds_void_t *)((hi ? ht : lt) + dst), 16, 0, 0);
    }
  };

  // B operand: centroid rows rho0 + 32 u + l32, dims 16 ks + 8 hh + e, split
  // into fp16 halves at one power-of-two scale per 32-row sub-tile (its
  // largest magnitude lands in [2^10, 2^11))
  f16x8 chi[2][KS], clo[2][KS];
  float rs[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int rho = rho0 + 32 * u + l32;
    const bool ok = rho < R;
    const float *src = a.ce_f + ((size_t)bh * R + (ok ? rho : 0)) * D + hh * 8;
    f32x4 x[KS][2];
    float amax = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        x[ks][hf] = ok ? *(const f32x4 *)(src + ks * 16 + hf * 4) : (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(x[ks][hf][e]));
      }
    }
    const int ex = row_exponent(wave_max_f(amax));
    rs[u] = ldexpf(a.scale_log2, -ex);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        half_t hi, lo;
        split_f16(x[ks][e >> 2][e & 3], ex, hi, lo);
        chi[u][ks][e] = hi;
        clo[u][ks][e] = lo;
      }
    }
  }

  // row statistics of this lane's two centroid rows; a finite floor for the
  // running maximum keeps 2^(t - m) free of inf - inf
  constexpr float kFloor = -0x1p100f;
  float st_m[2] = {kFloor, kFloor}, st_z[2] = {0.f, 0.f};
  if (PASS == 1) {
    // merge the chunk statistics: beta = max + log2(sum) - log2(share)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int rho = rho0 + 32 * u + l32;
      float beta = __builtin_inff();
      if (rho < R) {
        float m = kFloor;
        for (int c = 0; c < a.nchunk; ++c) m = fmaxf(m, a.stats[((size_t)bh * a.nchunk + c) * R + rho].x);
        float z = 0.f;
        for (int c = 0; c < a.nchunk; ++c) {
          const float2 p = a.stats[((size_t)bh * a.nchunk + c) * R + rho];
          z += p.y * __builtin_amdgcn_exp2f(p.x - m);
        }
        const float w = a.ce_w[(size_t)bh * R + rho];
        if (w > 0.f && z > 0.f) beta = m + __builtin_log2f(z) - __builtin_log2f(w);
      }
      st_m[u] = beta;
    }
  }

  // Sweep 2 with 8 clusters per query block takes the product the other way
  // round, D[centroid][key] = C . K_tile^T (the same register fragments as
  // operands A and B swapped): lane l then owns key l % 32 of the step and
  // register r centroid row 8 (r / 4) + 4 hh + r % 4 of a sub-tile, so a
  // query block's 8 cluster rows are 4 registers in each lane half, its sum
  // two in-lane adds and one exchange between the halves (the same pairing
  // as the prefix sum over 8 lanes, so the same bits), and its 32 keys of a
  // step store as one 128-byte line.  The rows' normalisers come from LDS.
  constexpr bool TR = PASS == 1 && CL == 3;
  __shared__ __attribute__((aligned(16))) float beta_s[TR ? 4 : 1][2][32];
  if constexpr (TR) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (hh == 0) beta_s[wave][u][l32] = st_m[u];
    __syncthreads();
  }

  // Consecutive steps are software-pipelined: the products of step k + 1
  // run while the epilogue of step k (its statistics or scores) runs in the
  // same wave, slice by slice, so that the vector work issues under the
  // matrix work.  The two steps' accumulators alternate between acc[0] and
  // acc[1].  Every value keeps the operation order of an unpipelined step,
  // so the results do not depend on this schedule.
  f32x16 acc[2][2];                            // [step parity][sub-tile]
  float *const sc_bh = a.scores + (size_t)bh * a.nqb * M;
  float ep_mx[2], ep_mn[2], ep_z[2];           // sweep-1 epilogue in flight

  // Epilogue slice j (of KS) of the step k held in acc[P] (key-tile scale
  // cs), in place.  Register r holds key 8 (r / 4) + 4 hh + r % 4 of the
  // step; sub-tile u holds centroid rows rho0 + 32 u + l32.
  auto epi = [&](auto p_c, int k, int j, float cs) {
    constexpr int P = decltype(p_c)::value;
    if constexpr (TR) {
      // slice j: (sub-tile, query block) groups j GPS .. j GPS + GPS - 1
      constexpr int GPS = 8 / KS;
      const int ln = fresh_lane(), lw = ln & 31, hf = ln >> 5;
      const int col = cbeg + k * CT + lw;
#pragma unroll
      for (int gi = 0; gi < GPS; ++gi) {
        const int grp = j * GPS + gi, u = grp >> 2, q = grp & 3;
        const float f = rs[u] * cs;
        const f32x4 b = *(const f32x4 *)&beta_s[wave][u][8 * q + 4 * hf];
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          x[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[P][u][4 * q + i], f, -b[i]));
        const float p = (x[2] + x[3]) + (x[0] + x[1]);
        const float t = p + xor32(p);
        const int qbi = ((rho0 + 32 * u) >> 3) + q;
        if (hf == 0 && qbi < a.nqb && col < cend) sc_bh[(unsigned)qbi * (unsigned)M + (unsigned)col] = t;
      }
      return;
    }
    const bool ragged = cbeg + k * CT + CT > cend;
    if (j == 0 && ragged) {
      // the last step of the row's last chunk: keys at or past cend (the
      // next head's rows or the pad) get logit -inf.  The empty asm keeps
      // this a branch: flattened, it would cost every step two selects per
      // value.
      const int lim = cend - (cbeg + k * CT + 4 * (fresh_lane() >> 5));
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[P][u][r] = 8 * (r >> 2) + (r & 3) < lim ? acc[P][u][r] : -__builtin_inff();
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float f = rs[u] * cs;  // > 0
      if (PASS == 0) {
        // slices 0 .. KS/2 - 1: the maximum; the rest: the sum
        constexpr int HS = KS / 2, PE = 16 / HS;
        if (j < HS) {
#pragma unroll
          for (int e = 0; e < PE; ++e) {
            const int r = j * PE + e;
            ep_mx[u] = r == 0 ? acc[P][u][r] : fmaxf(ep_mx[u], acc[P][u][r]);
          }
          if (j == HS - 1) {
            ep_mn[u] = fmaxf(st_m[u], ep_mx[u] * f);
            ep_z[u] = st_z[u] * __builtin_amdgcn_exp2f(st_m[u] - ep_mn[u]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < PE; ++e) {
            const int r = (j - HS) * PE + e;
            ep_z[u] += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[P][u][r], f, -ep_mn[u]));
          }
          if (j == KS - 1) {
            st_m[u] = ep_mn[u];
            st_z[u] = ep_z[u];
          }
        }
      } else {
        constexpr int PE = 16 / KS;
#pragma unroll
        for (int e = 0; e < PE; ++e) {
          const int r = j * PE + e;
          float x = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[P][u][r], f, -st_m[u]));
          // a query block's C clusters are C consecutive lanes: prefix sums
          // inside rows of 16 lanes leave each block's total in its last lane
          if (CL >= 1) x = add_shr<1>(x);
          if (CL >= 2) x = add_shr<2>(x);
          if (CL >= 3) x = add_shr<4>(x);
          if (CL >= 4) x = add_shr<8>(x);
          acc[P][u][r] = x;
        }
        if (j == KS - 1) {
          // the lane's row, its store offset and the condition are formed
          // here from the lane index; the head's scores come from a scalar
          // base plus a 32-bit element offset (a head holds fewer than 2^32
          // scores)
          const int ln = fresh_lane(), lw = ln & 31;
          const int rho = rho0 + 32 * u + lw;
          const int c0 = cbeg + k * CT + 4 * (ln >> 5);  // key of register 0
          if ((lw & (C - 1)) == C - 1 && rho < R) {
            const unsigned off = (unsigned)(rho >> CL) * (unsigned)M + (unsigned)c0;
            float *dst = sc_bh + off;
            if (!ragged && (M & 3) == 0) {
#pragma unroll
              for (int g = 0; g < 4; ++g)
                *(f32x4 *)(dst + 8 * g) = (f32x4){acc[P][u][4 * g], acc[P][u][4 * g + 1],
                                                  acc[P][u][4 * g + 2], acc[P][u][4 * g + 3]};
            } else {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int col = c0 + 8 * (r >> 2) + (r & 3);
                if (col < cend) dst[8 * (r >> 2) + (r & 3)] = acc[P][u][r];
              }
            }
          }
        }
      }
    }
  };

  // Products of the step in slot S into acc[P] (both sub-tiles), with
  // epilogue slice ks of the previous step (ep) after each k-step's products.
  auto products = [&](auto slot_c, auto p_c, auto &&ep) {
    constexpr int P = decltype(p_c)::value;
    const unsigned char *ht = hslot(slot_c);
    const unsigned char *lt = lslot(slot_c);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[P][u][r] = 0.f;
    // chunk (2 ks + hh) ^ swz of row l32 = (2 ks) ^ (hh ^ swz), and 2 ks
    // only touches bits the row offset l32 ROWB leaves clear: the offset is
    // the lane's base XOR a constant, one instruction from one register
    auto rd = [&](const unsigned char *t, int ks) {
      unsigned b = rd_base;
      asm volatile("" : "+v"(b));
      return as_f16x8(*(const u32x4 *)(t + (b ^ (unsigned)((2 * ks) << 4))));
    };
    f16x8 kh[KS], kl[KS];
    kh[0] = rd(ht, 0);
    kl[0] = rd(lt, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) {  // next k-step's key fragments
        kh[ks + 1] = rd(ht, ks + 1);
        kl[ks + 1] = rd(lt, ks + 1);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
        acc[P][u] = TR ? __builtin_amdgcn_mfma_f32_32x32x16_f16(clo[u][ks], kh[ks], acc[P][u], 0, 0, 0)
                       : __builtin_amdgcn_mfma_f32_32x32x16_f16(kh[ks], clo[u][ks], acc[P][u], 0, 0, 0);
#pragma unroll
      for (int u = 0; u < 2; ++u)
        acc[P][u] = TR ? __builtin_amdgcn_mfma_f32_32x32x16_f16(chi[u][ks], kh[ks], acc[P][u], 0, 0, 0)
                       : __builtin_amdgcn_mfma_f32_32x32x16_f16(kh[ks], chi[u][ks], acc[P][u], 0, 0, 0);
#pragma unroll
      for (int u = 0; u < 2; ++u)
        acc[P][u] = TR ? __builtin_amdgcn_mfma_f32_32x32x16_f16(chi[u][ks], kl[ks], acc[P][u], 0, 0, 0)
                       : __builtin_amdgcn_mfma_f32_32x32x16_f16(kl[ks], chi[u][ks], acc[P][u], 0, 0, 0);
      ep(ks);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Step k's tile is in its slot, and every wave is done with step k - 1's
  // slot (the next prefetch overwrites it).
  auto wait_step = [&](int k) {
    const int ahead = min(NB - 2, nsteps - 1 - k);  // steps after k already requested
    if (ahead >= 2) sc_ring_barrier<2 * LPW>();
    else if (ahead == 1) sc_ring_barrier<LPW>();
    else sc_ring_barrier<0>();
  };

  // The key-tile scale of a step is loaded before the ring barrier that
  // waits for the step's tile, whose wait covers it: a scalar load in flight
  // during the products would force every LDS wait there to drain all
  // outstanding reads (scalar loads return out of order).
  float cs_cur = 0.f;
  // iteration k (slot S = k mod NB): products of step k + 1 beside the
  // epilogue of step k
  auto step = [&](auto slot_c, int k) {
    constexpr int S = decltype(slot_c)::value;
    using SN = std::integral_constant<int, (S + 1) % NB>;
    using PK = std::integral_constant<int, S & 1>;
    using PN = std::integral_constant<int, (S + 1) & 1>;
    const float cs = cs_cur;
    if (k + 1 < nsteps) {
      cs_cur = kcs[k + 1];
      wait_step(k + 1);
      if (k + NB < nsteps) issue(slot_c, k + NB);
      products(SN(), PN(), [&](int j) { epi(PK(), k, j, cs); });
    } else {
#pragma unroll
      for (int j = 0; j < KS; ++j) epi(PK(), k, j, cs);
    }
  };

  for (int k = 0; k < NB - 1 && k < nsteps; ++k) {
    switch (k) {
      case 0: issue(std::integral_constant<int, 0>(), 0); break;
      case 1: issue(std::integral_constant<int, 1>(), 1); break;
      default: issue(std::integral_constant<int, 2>(), 2); break;
    }
  }
  if (nsteps > 0) {
    cs_cur = kcs[0];
    wait_step(0);
    if (NB - 1 < nsteps) issue(std::integral_constant<int, NB - 1>(), NB - 1);
    products(std::integral_constant<int, 0>(), std::integral_constant<int, 0>(), [](int) {});
  }
  static_assert(NB % 2 == 0, "step parity follows the slot");
  for (int k = 0; k < nsteps; k += NB) {
    step(std::integral_constant<int, 0>(), k);
    if (k + 1 < nsteps) step(std::integral_constant<int, 1>(), k + 1);
    if (k + 2 < nsteps) step(std::integral_constant<int, 2>(), k + 2);
    if (k + 3 < nsteps) step(std::integral_constant<int, 3>(), k + 3);
  }

  if (PASS == 0) {
    // lanes l and l + 32 hold the same rows (different keys): merge, store
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float m = st_m[u], z = st_z[u];
      const float m2 = xor32(m), z2 = xor32(z);
      const float mn = fmaxf(m, m2);
      const float zz = z * __builtin_amdgcn_exp2f(m - mn) + z2 * __builtin_amdgcn_exp2f(m2 - mn);
      const int rho = rho0 + 32 * u + l32;
      if (hh == 0 && rho < R) a.stats[((size_t)bh * a.nchunk + chunk) * R + rho] = make_float2(mn, zz);
    }
  }
}

struct Layout {
  size_t kb_hi, kb_lo, kb_cs, ce_f, ce_w, stats, total;
  int nqb, M, R, nchunk, chunk_cols, tiles, ktiles;
};

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

Layout make_layout(int B, int H, int N, int d, int kv_block, int C) {
  Layout L;
  const size_t BH = (size_t)B * H;
  L.nqb = (N + 127) / 128;
  L.M = (N + kv_block - 1) / kv_block;
  L.R = L.nqb * C;
  L.tiles = (L.R + 255) / 256;
  L.ktiles = (L.M + 31) / 32;
  // column chunks of whole 32-key steps: at least two rounds of the 512
  // resident workgroups (2 per CU), preferring a nearly full last round
  const long long wg = (long long)L.tiles * (long long)BH;
  const int steps = L.ktiles;
  int nchunk = 1;
  for (int n = 1; n <= 64 && n <= steps; ++n) {
    nchunk = n;
    const long long tot = wg * n;
    if (tot < 1024) continue;
    const long long rounds = (tot + 511) / 512;
    if (tot * 10 >= rounds * 512 * 9) break;  // rounds at least 90 % occupied
  }
  L.chunk_cols = ((steps + nchunk - 1) / nchunk) * 32;
  L.nchunk = (L.M + L.chunk_cols - 1) / L.chunk_cols;
  size_t off = 0;
  // split keys, each array padded by one 32-key tile (ragged-step reads)
  L.kb_hi = off; off += al256((BH * L.M + 32) * d * 2);
  L.kb_lo = off; off += al256((BH * L.M + 32) * d * 2);
  L.kb_cs = off; off += al256(BH * L.ktiles * 4);
  L.ce_f = off; off += al256(BH * L.R * d * 4);
  L.ce_w = off; off += al256(BH * L.R * 4);
  L.stats = off; off += al256(BH * (size_t)L.nchunk * L.R * 8);
  L.total = off;
  return L;
}

// Sweep 2 with the cluster sum's lane levels fixed at compile time
// (C = 2^CL clusters per query block).
template <int D>
void launch_sweep2(dim3 grid, const SelArgs &a, hipStream_t stream) {
  switch (a.C) {
    case 1: hipLaunchKernelGGL((score_kernel<D, 1, 0>), grid, dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((score_kernel<D, 1, 1>), grid, dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((score_kernel<D, 1, 2>), grid, dim3(256), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((score_kernel<D, 1, 3>), grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL((score_kernel<D, 1, 4>), grid, dim3(256), 0, stream, a); break;
  }
}

}  // namespace

size_t select_workspace_bytes(int B, int H, int N, int d, int kv_block, int n_clusters) {
  return make_layout(B, H, N, d, kv_block, n_clusters).total;
}

int launch_select_scores(const void *q, const void *k, int B, int H, int N, int d, int kv_block,
                         int n_clusters, int kmeans_iters, float *scores, float *centroids,
                         float *weights, void *workspace, hipStream_t stream) {
  clear_pending_error();
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
  a.ktiles = L.ktiles;
  a.scores = scores;
  a.centroids = centroids;
  a.weights = weights;
  a.kb_hi = (half_t *)(ws + L.kb_hi);
  a.kb_lo = (half_t *)(ws + L.kb_lo);
  a.kb_cs = (float *)(ws + L.kb_cs);
  a.ce_f = (float *)(ws + L.ce_f);
  a.ce_w = (float *)(ws + L.ce_w);
  a.stats = (float2 *)(ws + L.stats);
  a.scale_log2 = kLog2e / sqrtf((float)d);
  const unsigned BH = (unsigned)(B * H);
  const long long nsc = (long long)L.tiles * L.nchunk * BH;
  if (nsc > 0x7fffffffLL) return BSA_ERR_UNSUPPORTED;
  const dim3 gpool(L.ktiles, BH), gkm(L.nqb, BH), gsc((unsigned)nsc);
  if (d == 128) {
    hipLaunchKernelGGL(pool_split_kernel<128>, gpool, dim3(256), 0, stream, a);
    if (n_clusters <= 8) hipLaunchKernelGGL((kmeans_kernel<128, 8>), gkm, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((kmeans_kernel<128, 16>), gkm, dim3(256), 0, stream, a);
    hipLaunchKernelGGL((score_kernel<128, 0, 0>), gsc, dim3(256), 0, stream, a);
    launch_sweep2<128>(gsc, a, stream);
  } else {
    hipLaunchKernelGGL(pool_split_kernel<64>, gpool, dim3(256), 0, stream, a);
    if (n_clusters <= 8) hipLaunchKernelGGL((kmeans_kernel<64, 8>), gkm, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((kmeans_kernel<64, 16>), gkm, dim3(256), 0, stream, a);
    hipLaunchKernelGGL((score_kernel<64, 0, 0>), gsc, dim3(256), 0, stream, a);
    launch_sweep2<64>(gsc, a, stream);
  }
  return status_of(hipGetLastError());
}

}  // namespace bsa
