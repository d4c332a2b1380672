// BASA-structured block lists for the sparse attention kernel (gfx950).
//
// BASA page (onedev.kr/papers/688):
//   section "어떻게 동작하나" -- the latent grid is rolled by -Delta and cut into
//     non-overlapping spatial windows that keep every frame; attention runs
//     inside each window and the result is rolled back;
//   section "무엇과 다른가" -- keys and values are mean-pooled per frame into a
//     global memory G that every window also attends to; each window routes
//     to the top-K other windows by mean-query . mean-key relevance and
//     attends to their raw keys and values as well.
//
// Here the whole structure becomes block lists of the one sparse attention
// kernel: Q, K and V are permuted window-major (each window padded with zero
// rows to a multiple of 128 so that a 128-row query block lies in one
// window), G is appended after the last window in the key/value buffers, and
// every query block lists its own window's KV blocks, its routed windows'
// blocks and all pooled blocks (pi = 1, no bias).
//
// Kernels:
//   desc      one workgroup per (window, Q or K, head): fp32 window means in
//             the stated order (window-local token order, one rounding per
//             add, one IEEE division) -- routing is a discrete decision and
//             must match the oracle bit for bit;
//   route     one thread per (head, window): top-K by the fp32 dot product
//             (ascending dims, rounded multiply then rounded add), ties to
//             the lowest window, taken one rank at a time;
//   permute   16-byte chunks of Q/K/V rows into window-major order, zero pad;
//   pool      per-frame ph x pw cell means of K and V (fp32 sum, one
//             division, bf16 round to nearest even), appended after the
//             windows;
//   lists     one workgroup per query block: own, routed (ascending), pooled;
//   unpermute output rows back to raster token order.
#include <type_traits>

#include "common.h"

namespace bsa {

namespace {

// Geometry of the rolled window grid, shared by every kernel.
struct Geo {
  int T, Hg, Wg, wh, ww, dy, dx;  // dy, dx normalised to [0, Hg), [0, Wg)
  int nwy, nwx, hr, wr;           // window rows/cols; last row height, last col width
  int pad_full, pad_fr;           // padded rows of a full window / last-column window (full rows)
  int pad_lr, pad_lrr;            // same two for the last window row
  int prow;                       // padded rows of one full window row
  int nwin, Nq_pad;
  int ph, pw, pyc, pxc, npool;    // pooling cells and pooled tokens
  int kv_shift;
};

inline int pad128(long long n) { return (int)((n + 127) / 128 * 128); }

bool make_geo(int T, int Hg, int Wg, int wh, int ww, int dy, int dx, int ph, int pw, int kv_block,
              Geo &g) {
  g.T = T;
  g.Hg = Hg;
  g.Wg = Wg;
  g.wh = wh;
  g.ww = ww;
  g.dy = ((dy % Hg) + Hg) % Hg;
  g.dx = ((dx % Wg) + Wg) % Wg;
  g.nwy = (Hg + wh - 1) / wh;
  g.nwx = (Wg + ww - 1) / ww;
  g.hr = Hg - (g.nwy - 1) * wh;
  g.wr = Wg - (g.nwx - 1) * ww;
  const long long full = (long long)T * wh * ww, fr = (long long)T * wh * g.wr;
  const long long lr = (long long)T * g.hr * ww, lrr = (long long)T * g.hr * g.wr;
  for (long long n : {full, fr, lr, lrr})
    if (n % kv_block) return false;  // a KV block must not straddle windows
  g.pad_full = pad128(full);
  g.pad_fr = pad128(fr);
  g.pad_lr = pad128(lr);
  g.pad_lrr = pad128(lrr);
  const long long prow = (long long)(g.nwx - 1) * g.pad_full + g.pad_fr;
  const long long nq = (long long)(g.nwy - 1) * prow + (long long)(g.nwx - 1) * g.pad_lr + g.pad_lrr;
  g.nwin = g.nwy * g.nwx;
  g.ph = ph;
  g.pw = pw;
  g.pyc = (Hg + ph - 1) / ph;
  g.pxc = (Wg + pw - 1) / pw;
  const long long npool = (long long)T * g.pyc * g.pxc;
  if (nq + npool + kv_block > 0x7fffffffLL) return false;
  g.prow = (int)prow;
  g.Nq_pad = (int)nq;
  g.npool = (int)npool;
  g.kv_shift = __builtin_ctz((unsigned)kv_block);
  return true;
}

struct Win {
  int a, b, h, w, off, n;  // window row/col, height, width, first padded row, tokens
};

__host__ __device__ inline Win window_at(const Geo &g, int a, int b) {
  Win w;
  w.a = a;
  w.b = b;
  w.h = a == g.nwy - 1 ? g.hr : g.wh;
  w.w = b == g.nwx - 1 ? g.wr : g.ww;
  w.off = a * g.prow + b * (a == g.nwy - 1 ? g.pad_lr : g.pad_full);
  w.n = g.T * w.h * w.w;
  return w;
}

// Raster token of window-local index r (frame, rolled row, rolled column).
__host__ __device__ inline int token_of(const Geo &g, const Win &w, int r) {
  const int hw = w.h * w.w;
  const int t = r / hw, rem = r - t * hw;
  const int yy = rem / w.w, xx = rem - yy * w.w;
  int y = w.a * g.wh + yy + g.dy;
  if (y >= g.Hg) y -= g.Hg;
  int x = w.b * g.ww + xx + g.dx;
  if (x >= g.Wg) x -= g.Wg;
  return (t * g.Hg + y) * g.Wg + x;
}

// Window and local index of padded row R (local >= n: a pad row).
__device__ inline Win window_of_row(const Geo &g, int R, int &local) {
  const int a = min(R / g.prow, g.nwy - 1);
  const int R1 = R - a * g.prow;
  const int pa = a == g.nwy - 1 ? g.pad_lr : g.pad_full;
  const int b = min(R1 / pa, g.nwx - 1);
  local = R1 - b * pa;
  return window_at(g, a, b);
}

struct BasaArgs {
  Geo g;
  const uint16_t *q, *k, *v;
  uint16_t *qp, *kp, *vp;
  int32_t *idx, *count, *routes;
  float *desc;       // [BH][2][nwin][d] window means (Q then K)
  int32_t *rank;     // [BH][nwin][topk] routed windows, rank order
  int B, H, N, d, topk, max_blocks, Nk;
};

// ---------------------------------------------------------------- descriptors
// One thread per dim; the window's tokens in window-local order (frame,
// rolled row, rolled column), their raster index stepped incrementally.
// The adds stay in that order; loads run up to UN tokens ahead of them.
__global__ __launch_bounds__(128) void desc_kernel(BasaArgs a) {
  constexpr int UN = 64;
  const Geo &g = a.g;
  const int wid = blockIdx.x, which = blockIdx.y, bh = blockIdx.z;
  const int dim = threadIdx.x;
  if (dim >= a.d) return;
  const Win w = window_at(g, wid / g.nwx, wid % g.nwx);
  const uint16_t *x = (which ? a.k : a.q) + (size_t)bh * a.N * a.d + dim;
  // cursor: frame t, local row yy, local column xx -> raster token
  int t = 0, yy = 0, xx = 0;
  int y = w.a * g.wh + g.dy;
  if (y >= g.Hg) y -= g.Hg;
  const int x0 = w.b * g.ww + g.dx;
  auto next_token = [&]() -> int {
    int xc = x0 + xx;
    if (xc >= g.Wg) xc -= g.Wg;
    const int tok = (t * g.Hg + y) * g.Wg + xc;
    if (++xx == w.w) {
      xx = 0;
      if (++yy == w.h) {
        yy = 0;
        ++t;
        y = w.a * g.wh + g.dy;
      } else {
        ++y;
      }
      if (y >= g.Hg) y -= g.Hg;
    }
    return tok;
  };
  float acc = 0.f;
  int r = 0;
  auto batch = [&](auto n_c) {
    constexpr int n = decltype(n_c)::value;
    float vu[n];
#pragma unroll
    for (int u = 0; u < n; ++u) vu[u] = bf16_to_f32(x[(size_t)next_token() * a.d]);
#pragma unroll
    for (int u = 0; u < n; ++u) acc = __fadd_rn(acc, vu[u]);
  };
  for (; r + UN <= w.n; r += UN) batch(std::integral_constant<int, UN>());
  for (; r + 8 <= w.n; r += 8) batch(std::integral_constant<int, 8>());
  for (; r < w.n; ++r) acc = __fadd_rn(acc, bf16_to_f32(x[(size_t)next_token() * a.d]));
  a.desc[(((size_t)bh * 2 + which) * g.nwin + wid) * a.d + dim] = __fdiv_rn(acc, (float)w.n);
}

// ---------------------------------------------------------------- routing
__device__ inline float desc_dot(const float *qd, const float *kd, int d) {
  float acc = 0.f;
  for (int c = 0; c < d; ++c) acc = __fadd_rn(acc, __fmul_rn(qd[c], kd[c]));
  return acc;
}

// One wave per (head, query window i): lane l scores candidate windows
// l, l + 64, .. (each dot product in the stated order); the top-k are then
// taken one rank at a time by a wave-wide (score desc, id asc) maximum.
__device__ __forceinline__ bool ranks_before(float s1, int j1, float s2, int j2) {
  return s1 > s2 || (s1 == s2 && j1 < j2);
}

__global__ __launch_bounds__(64) void route_kernel(BasaArgs a) {
  const Geo &g = a.g;
  const int i = blockIdx.x, bh = blockIdx.y, lane = threadIdx.x;
  const float *qd = a.desc + (((size_t)bh * 2 + 0) * g.nwin + i) * a.d;
  const float *kd0 = a.desc + ((size_t)bh * 2 + 1) * g.nwin * a.d;
  // rank p: the best window ranked after pick p-1
  float ps = __builtin_inff();
  int pj = -1;
  for (int p = 0; p < a.topk; ++p) {
    float bs = -__builtin_inff();
    int bj = 0x7fffffff;
    for (int j = lane; j < g.nwin; j += 64) {
      if (j == i) continue;
      const float s = desc_dot(qd, kd0 + (size_t)j * a.d, a.d);
      const bool after = ranks_before(ps, pj, s, j);
      if (after && (bj == 0x7fffffff || ranks_before(s, j, bs, bj))) {
        bs = s;
        bj = j;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float s2 = __shfl_xor(bs, o, 64);
      const int j2 = __shfl_xor(bj, o, 64);
      if (j2 != 0x7fffffff && (bj == 0x7fffffff || ranks_before(s2, j2, bs, bj))) {
        bs = s2;
        bj = j2;
      }
    }
    if (lane == 0) {
      a.rank[((size_t)bh * g.nwin + i) * a.topk + p] = bj;
      if (a.routes) a.routes[((size_t)bh * g.nwin + i) * a.topk + p] = bj;
    }
    ps = bs;
    pj = bj;
  }
}

// ---------------------------------------------------------------- permute
// 16 lanes (d = 128) or 8 lanes (d = 64) per padded row, 16 bytes each.
__global__ __launch_bounds__(256) void permute_kernel(BasaArgs a) {
  const Geo &g = a.g;
  const int cpr = a.d / 8;  // 16-byte chunks per row
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  const int bh = blockIdx.y;
  const long long R = e / cpr;
  const int c = (int)(e - R * cpr);
  if (R >= g.Nq_pad) return;
  int local;
  const Win w = window_of_row(g, (int)R, local);
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 vq = zero, vk = zero, vv = zero;
  if (local < w.n) {
    const size_t src = ((size_t)bh * a.N + token_of(g, w, local)) * a.d + c * 8;
    vq = ld16(a.q + src);
    vk = ld16(a.k + src);
    vv = ld16(a.v + src);
  }
  st16(a.qp + ((size_t)bh * g.Nq_pad + R) * a.d + c * 8, vq);
  st16(a.kp + ((size_t)bh * a.Nk + R) * a.d + c * 8, vk);
  st16(a.vp + ((size_t)bh * a.Nk + R) * a.d + c * 8, vv);
}

// ---------------------------------------------------------------- pooling
// One thread per (pooled token, dim): rows [Nq_pad, Nk) of kp and vp.
__global__ __launch_bounds__(256) void pool_kernel(BasaArgs a) {
  const Geo &g = a.g;
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  const int bh = blockIdx.y;
  const long long gi = e / a.d;
  const int dim = (int)(e - gi * a.d);
  if (gi >= g.npool) return;
  const int cells = g.pyc * g.pxc;
  const int t = (int)gi / cells, rem = (int)gi - t * cells;
  const int cy = rem / g.pxc, cx = rem - cy * g.pxc;
  const int y0 = cy * g.ph, x0 = cx * g.pw;
  const int y1 = min(g.Hg, y0 + g.ph), x1 = min(g.Wg, x0 + g.pw);
  const int wx = x1 - x0, cnt = (y1 - y0) * wx;
  const size_t base = ((size_t)bh * a.N + (size_t)t * g.Hg * g.Wg) * a.d + dim;
  float sk = 0.f, sv = 0.f;
  // the cells in row-major order, UP loads in flight before their adds
  // (cells past the patch re-read its first cell and are not added)
  constexpr int UP = 16;
  for (int c0 = 0; c0 < cnt; c0 += UP) {
    uint16_t kk[UP], vv[UP];
#pragma unroll
    for (int u = 0; u < UP; ++u) {
      const int c = c0 + u < cnt ? c0 + u : 0;
      const int y = y0 + c / wx, x = x0 + c % wx;
      const size_t o = base + ((size_t)y * g.Wg + x) * a.d;
      kk[u] = a.k[o];
      vv[u] = a.v[o];
    }
#pragma unroll
    for (int u = 0; u < UP; ++u)
      if (c0 + u < cnt) {
        sk = __fadd_rn(sk, bf16_to_f32(kk[u]));
        sv = __fadd_rn(sv, bf16_to_f32(vv[u]));
      }
  }
  const size_t o = ((size_t)bh * a.Nk + g.Nq_pad + gi) * a.d + dim;
  a.kp[o] = (unsigned short)bf16_bits(__fdiv_rn(sk, (float)cnt));
  a.vp[o] = (unsigned short)bf16_bits(__fdiv_rn(sv, (float)cnt));
}

// ---------------------------------------------------------------- lists
__global__ __launch_bounds__(256) void list_kernel(BasaArgs a) {
  const Geo &g = a.g;
  const int qb = blockIdx.x, bh = blockIdx.y;
  __shared__ int seg_first[66], seg_len[66];  // own + up to 64 routed + pooled
  __shared__ int ids[64];
  __shared__ int nseg_s, total_s;
  if (threadIdx.x == 0) {
    int local;
    const Win w = window_of_row(g, qb * 128, local);
    const int wid = w.a * g.nwx + w.b;
    const int kvs = g.kv_shift;
    int ns = 0;
    seg_first[ns] = w.off >> kvs;
    seg_len[ns++] = w.n >> kvs;
    // routed windows in ascending id (insertion into the segment table)
    const int32_t *rk = a.rank + ((size_t)bh * g.nwin + wid) * a.topk;
    int nr = 0;
    for (int p = 0; p < a.topk; ++p) {
      const int j = rk[p];
      int pos = nr++;
      while (pos > 0 && ids[pos - 1] > j) {
        ids[pos] = ids[pos - 1];
        --pos;
      }
      ids[pos] = j;
    }
    for (int p = 0; p < nr; ++p) {
      const Win r = window_at(g, ids[p] / g.nwx, ids[p] % g.nwx);
      seg_first[ns] = r.off >> kvs;
      seg_len[ns++] = r.n >> kvs;
    }
    seg_first[ns] = g.Nq_pad >> kvs;
    seg_len[ns++] = (g.npool + (1 << kvs) - 1) >> kvs;
    int tot = 0;
    for (int s = 0; s < ns; ++s) tot += seg_len[s];
    nseg_s = ns;
    total_s = tot;
    a.count[(size_t)bh * (g.Nq_pad / 128) + qb] = tot;
  }
  __syncthreads();
  const int ns = nseg_s, tot = total_s;
  int32_t *row = a.idx + ((size_t)bh * (g.Nq_pad / 128) + qb) * a.max_blocks;
  for (int e = threadIdx.x; e < a.max_blocks; e += 256) {
    int val = -1;
    if (e < tot) {
      int s = 0, base = 0;
      while (s < ns - 1 && e >= base + seg_len[s]) base += seg_len[s++];
      val = seg_first[s] + (e - base);
    }
    row[e] = val;
  }
}

// ---------------------------------------------------------------- unpermute
__global__ __launch_bounds__(256) void unpermute_kernel(Geo g, const uint16_t *op, uint16_t *out,
                                                        int N, int d) {
  const int cpr = d / 8;
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  const int bh = blockIdx.y;
  const long long n = e / cpr;
  const int c = (int)(e - n * cpr);
  if (n >= N) return;
  const int x = (int)(n % g.Wg), y = (int)((n / g.Wg) % g.Hg), t = (int)(n / ((long long)g.Wg * g.Hg));
  int sy = y - g.dy;
  if (sy < 0) sy += g.Hg;
  int sx = x - g.dx;
  if (sx < 0) sx += g.Wg;
  const int wa = sy / g.wh, wb = sx / g.ww;
  const Win w = window_at(g, wa, wb);
  const int local = (t * w.h + (sy - wa * g.wh)) * w.w + (sx - wb * g.ww);
  st16(out + ((size_t)bh * N + n) * d + c * 8, ld16(op + ((size_t)bh * g.Nq_pad + w.off + local) * d + c * 8));
}

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

int basa_layout(int T, int Hg, int Wg, int d, int wh, int ww, int ph, int pw, int topk,
                int kv_block, int B, int H, int *nwin, int *Nq_pad, int *Nk, int *max_blocks,
                size_t *workspace) {
  Geo g;
  if (!make_geo(T, Hg, Wg, wh, ww, 0, 0, ph, pw, kv_block, g)) return BSA_ERR_UNSUPPORTED;
  if (topk > 64) return BSA_ERR_UNSUPPORTED;
  const long long wmax = (long long)T * wh * ww / kv_block;  // blocks of the largest window
  const long long pool_blocks = (g.npool + kv_block - 1) / kv_block;
  const long long mb = (1 + (long long)topk) * wmax + pool_blocks;
  const long long nk = (long long)g.Nq_pad + g.npool;
  if (mb > 0x7fffffffLL || nk > 0x7fffffffLL) return BSA_ERR_SIZE;
  const size_t BH = (size_t)B * H;
  *nwin = g.nwin;
  *Nq_pad = g.Nq_pad;
  *Nk = (int)nk;
  *max_blocks = (int)mb;
  *workspace = al256(BH * 2 * g.nwin * (size_t)d * 4) + al256(BH * g.nwin * (size_t)(topk > 0 ? topk : 1) * 4);
  return BSA_OK;
}

int launch_basa_plan(const void *q, const void *k, const void *v, int B, int H, int T, int Hg,
                     int Wg, int d, int wh, int ww, int dy, int dx, int ph, int pw, int topk,
                     int kv_block, void *qp, void *kp, void *vp, int32_t *idx, int32_t *count,
                     int32_t *routes, void *workspace, hipStream_t stream) {
  clear_pending_error();
  int nwin, nqp, nk, mb;
  size_t ws;
  int st = basa_layout(T, Hg, Wg, d, wh, ww, ph, pw, topk, kv_block, B, H, &nwin, &nqp, &nk, &mb,
                       &ws);
  if (st != BSA_OK) return st;
  BasaArgs a;
  make_geo(T, Hg, Wg, wh, ww, dy, dx, ph, pw, kv_block, a.g);
  a.q = (const uint16_t *)q;
  a.k = (const uint16_t *)k;
  a.v = (const uint16_t *)v;
  a.qp = (uint16_t *)qp;
  a.kp = (uint16_t *)kp;
  a.vp = (uint16_t *)vp;
  a.idx = idx;
  a.count = count;
  a.routes = routes;
  const size_t BH = (size_t)B * H;
  a.desc = (float *)workspace;
  a.rank = (int32_t *)((char *)workspace + al256(BH * 2 * nwin * (size_t)d * 4));
  a.B = B;
  a.H = H;
  a.N = T * Hg * Wg;
  a.d = d;
  a.topk = topk;
  a.max_blocks = mb;
  a.Nk = nk;
  const unsigned bh = (unsigned)BH;
  if (topk > 0) {
    hipLaunchKernelGGL(desc_kernel, dim3(nwin, 2, bh), dim3(128), 0, stream, a);
    hipLaunchKernelGGL(route_kernel, dim3(nwin, bh), dim3(64), 0, stream, a);
  }
  const long long pe = (long long)nqp * (d / 8);
  hipLaunchKernelGGL(permute_kernel, dim3((unsigned)((pe + 255) / 256), bh), dim3(256), 0, stream, a);
  const long long pl = (long long)(nk - nqp) * d;
  hipLaunchKernelGGL(pool_kernel, dim3((unsigned)((pl + 255) / 256), bh), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(list_kernel, dim3(nqp / 128, bh), dim3(256), 0, stream, a);
  return status_of(hipGetLastError());
}

int launch_window_unpermute(const void *out_perm, void *out, int B, int H, int T, int Hg, int Wg,
                            int d, int wh, int ww, int dy, int dx, hipStream_t stream) {
  clear_pending_error();
  Geo g;
  if (!make_geo(T, Hg, Wg, wh, ww, dy, dx, 1, 1, 1, g)) return BSA_ERR_UNSUPPORTED;
  const int N = T * Hg * Wg;
  const long long e = (long long)N * (d / 8);
  hipLaunchKernelGGL(unpermute_kernel, dim3((unsigned)((e + 255) / 256), (unsigned)(B * H)),
                     dim3(256), 0, stream, g, (const uint16_t *)out_perm, (uint16_t *)out, N, d);
  return status_of(hipGetLastError());
}

// Per-layer window offsets (BASA page, section "어떻게 동작하나"): candidates
// a_i = (i delta) mod w with delta = max(1, floor(w / L)), laid out with the
// first half and the second half alternating, so position l holds a_{l/2}
// for even l and a_{K + (l-1)/2} for odd l, K = ceil(L / 2).
static int offset_at(int w, int L, int l) {
  const long long delta = w / L > 1 ? w / L : 1;
  const long long i = (l & 1) ? (L + 1) / 2 + (l >> 1) : (l >> 1);
  return (int)((i * delta) % w);
}

void basa_offsets(int w, int L, int *b) {
  for (int l = 0; l < L; ++l) b[l] = offset_at(w, L, l);
}

// Delta_{l,s} = ((b^h_l + c^h_s) mod w_h, (b^w_l + c^w_s) mod w_w), for every
// layer l < L and step s < S (row-major [L][S]); step offsets may be
// negative or absent (zero).
void basa_shifts(int wh, int ww, int L, int S, const int *c_h, const int *c_w, int *dy, int *dx) {
  auto mod = [](long long x, int m) { return (int)(((x % m) + m) % m); };
  for (int l = 0; l < L; ++l) {
    const int bh = offset_at(wh, L, l), bw = offset_at(ww, L, l);
    for (int s = 0; s < S; ++s) {
      dy[(size_t)l * S + s] = mod((long long)bh + (c_h ? c_h[s] : 0), wh);
      dx[(size_t)l * S + s] = mod((long long)bw + (c_w ? c_w[s] : 0), ww);
    }
  }
}

}  // namespace bsa
