// Sampling plan kernel (SIP or top-k) for gfx950.
//
// AB-Attention page (onedev.kr/papers/1521), section "어떻게 쓰나": per query
// block i, pi_ij = min(1, lambda_i S_ij) with sum_j pi_ij = s; blocks with
// pi = 1 are always kept; a systematic sample draws exactly s distinct
// blocks shared by the whole query block.  Top-k at the same budget is the
// "SIP without pi weighting" level of the ablation paragraph in "전제와 한계".
//
// One workgroup (512 threads) per row; the row sits in LDS when it fits,
// else it is re-read from global memory on every pass.
//
// SIP, exactly as the C ABI documents it:
//   * the number r of saturated blocks is the smallest r with
//     (s - r) S_(r+1) <= T_r.  Over the row values v this reads
//     cond(v): (s - #{S >= v}) v <= sum_{S < v} S, which is monotone in v;
//     the largest x with cond(x) is bracketed by secant steps down from
//     T / s, then either (at most 64 row values inside the bracket) those
//     values are collected in one pass and cond is taken at each, or a
//     bisection over fp32 bit patterns runs until no row value lies inside
//     the bracket; then r = #{S > x}, T_r = sum_{S <= x} S;
//   * each search step decides cond from an fp64 sum whose rounding error
//     is bounded; inside that bound the sum is retaken as a double-double
//     (error below 2^-90 of the sum), and only when even that cannot
//     decide, exactly (integer digits, 352 bits in units of 2^-149, which
//     hold every fp32 value and 2^20 of them);
//   * T_r is the correctly rounded (nearest even) fp64 value of the exact
//     sum: read off the double-double when its error interval lies inside
//     one rounding interval, else from the exact digits; lambda =
//     (s - r) / T_r is one IEEE division and pi_j = min(1, lambda S_j) one
//     IEEE multiply;
//   * Pi_j = floor(pi_j 2^44) and their prefix sums are exact 64-bit
//     integers; points U + k 2^44 (k < s) pick the blocks, in index order.
#include "common.h"

namespace bsa {

__host__ __device__ inline uint64_t splitmix64_at(uint64_t seed, uint64_t i) {
  uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__host__ __device__ inline uint64_t offset_of_row(uint64_t seed, uint64_t row) {
  const uint64_t x = splitmix64_at(seed, row) >> 20;  // 44 bits
  // floor(x * (2^44 - 2^16) / 2^44) = x - ceil(x / 2^28)
  return x - ((x + (1ull << 28) - 1) >> 28);
}

uint64_t sampling_offset(uint64_t seed, uint64_t row) { return offset_of_row(seed, row); }

namespace {

constexpr int PT = 512;               // threads per row
constexpr int NW = PT / 64;           // waves
constexpr int NDIG = 10;              // exact sums use 32-bit digits 0..NDIG (units 2^-149)
constexpr uint64_t UNIT = 1ull << 44;  // fixed-point 1.0 of pi
constexpr int MCAP = 64;              // bracket values resolved without bisection

struct PlanArgs {
  const float *scores;
  int rows, M, budget, mode;
  uint64_t seed;
  const uint64_t *offsets;
  int32_t *idx;
  float *bias;
  int32_t *count;
  double *lambda;
  int32_t *status;  // optional: BSA_ERR_NONFINITE when a row is invalid
};

// Workgroup scratch of a row, for NWV waves.  Small on purpose: with the
// row (M floats) beside it this stays under half of a CU's LDS, so two rows
// of the LDS-resident kernel run per CU.
template <int NWV>
struct SharedT {
  static constexpr int NW = NWV;
  uint64_t wdig[NWV][NDIG + 1];  // per-wave digit sums of an exact sum
  uint64_t total[NDIG + 1];      // normalised digits of the last exact sum
  double red_d[NWV];
  long long red_l[NWV];
  unsigned red_u[NWV];
  unsigned red_u2[NWV];
  long long cl[2][NWV];          // alternating buffers of the one-barrier reductions
  double chi[2][NWV], clo[2][NWV];
  double bcast_d;
  float col[MCAP];  // row values inside the final search bracket
  int cstat[MCAP];  // the condition at each: 1 holds, 0 fails, 2 undecided
  int ncol;
};
typedef SharedT<NW> Shared;

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ long long wave_sum_l(long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ unsigned wave_max_u(unsigned v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (unsigned)__shfl_xor((int)v, o, 64));
  return v;
}
__device__ __forceinline__ unsigned wave_min_u(unsigned v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (unsigned)__shfl_xor((int)v, o, 64));
  return v;
}

// Block-wide sums: every thread gets the total (fixed reduction order).
template <class SH>
__device__ __forceinline__ double block_sum_d(SH &sh, double v) {
  v = wave_sum_d(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.red_d[w] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < SH::NW; ++i) t += sh.red_d[i];
  return t;
}
template <class SH>
__device__ __forceinline__ long long block_sum_l(SH &sh, long long v) {
  v = wave_sum_l(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.red_l[w] = v;
  __syncthreads();
  long long t = 0;
#pragma unroll
  for (int i = 0; i < SH::NW; ++i) t += sh.red_l[i];
  return t;
}
template <class SH>
__device__ __forceinline__ void block_minmax_u(SH &sh, unsigned &mn, unsigned &mx) {
  mn = wave_min_u(mn);
  mx = wave_max_u(mx);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    sh.red_u[w] = mn;
    sh.red_u2[w] = mx;
  }
  __syncthreads();
  mn = sh.red_u[0];
  mx = sh.red_u2[0];
#pragma unroll
  for (int i = 1; i < SH::NW; ++i) {
    mn = min(mn, sh.red_u[i]);
    mx = max(mx, sh.red_u2[i]);
  }
}
// The row's first reductions in one: a packed count, a sum, a minimum and a
// maximum, each combined in the order block_sum_l / block_sum_d /
// block_minmax_u use (so the results are theirs), with one barrier.  Only
// for the first reduction of a kernel: nothing has read the buffers before.
template <class SH>
__device__ __forceinline__ void block_reduce_first(SH &sh, long long &pk, double &tot, unsigned &mn,
                                                   unsigned &mx) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    pk += __shfl_xor(pk, o, 64);
    tot += __shfl_xor(tot, o, 64);
    mn = min(mn, (unsigned)__shfl_xor((int)mn, o, 64));
    mx = max(mx, (unsigned)__shfl_xor((int)mx, o, 64));
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sh.red_l[w] = pk;
    sh.red_d[w] = tot;
    sh.red_u[w] = mn;
    sh.red_u2[w] = mx;
  }
  __syncthreads();
  pk = sh.red_l[0];
  tot = 0.0 + sh.red_d[0];
  mn = sh.red_u[0];
  mx = sh.red_u2[0];
#pragma unroll
  for (int i = 1; i < SH::NW; ++i) {
    pk += sh.red_l[i];
    tot += sh.red_d[i];
    mn = min(mn, sh.red_u[i]);
    mx = max(mx, sh.red_u2[i]);
  }
}

// Exclusive prefix over threads (thread order) of a 64-bit count.
template <class SH>
__device__ __forceinline__ uint64_t block_exscan_u64(SH &sh, uint64_t v, uint64_t &total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint64_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  __syncthreads();
  if (lane == 63) sh.red_l[w] = (long long)inc;
  __syncthreads();
  uint64_t base = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < SH::NW; ++i) {
    const uint64_t t = (uint64_t)sh.red_l[i];
    if (i < w) base += t;
    total += t;
  }
  return base + inc - v;
}

// One-barrier block reduction of a packed count and a double-double (hi,
// lo); every thread gets the same result (symmetric butterflies, then the
// waves in order).  The two buffers alternate with `ph`, so a reduction may
// write before the barrier: the previous reader of that buffer has passed
// the barrier of the reduction in between.
__device__ __forceinline__ void two_sum(double a, double b, double &s, double &e) {
  s = a + b;
  const double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}
// (hi, lo) += (bhi, blo) for non-negative double-doubles (symmetric in the
// two operands, relative error below 6 u^2 per call).
__device__ __forceinline__ void dd_add(double &hi, double &lo, double bhi, double blo) {
  double s, e;
  two_sum(hi, bhi, s, e);
  e += lo + blo;
  hi = s + e;
  lo = e - (hi - s);
}
// The same for a packed count and a plain fp64 sum.
template <class SH>
__device__ __forceinline__ void block_reduce(SH &sh, long long &cnt, double &sum, int &ph) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    cnt += __shfl_xor(cnt, o, 64);
    sum += __shfl_xor(sum, o, 64);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sh.cl[ph][w] = cnt;
    sh.chi[ph][w] = sum;
  }
  __syncthreads();
  cnt = sh.cl[ph][0];
  sum = sh.chi[ph][0];
#pragma unroll
  for (int i = 1; i < SH::NW; ++i) {
    cnt += sh.cl[ph][i];
    sum += sh.chi[ph][i];
  }
  ph ^= 1;
}
template <class SH>
__device__ __forceinline__ void block_reduce(SH &sh, long long &cnt, double &hi, double &lo, int &ph) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const long long c2 = __shfl_xor(cnt, o, 64);
    const double h2 = __shfl_xor(hi, o, 64), l2 = __shfl_xor(lo, o, 64);
    cnt += c2;
    dd_add(hi, lo, h2, l2);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sh.cl[ph][w] = cnt;
    sh.chi[ph][w] = hi;
    sh.clo[ph][w] = lo;
  }
  __syncthreads();
  cnt = sh.cl[ph][0];
  hi = sh.chi[ph][0];
  lo = sh.clo[ph][0];
#pragma unroll
  for (int i = 1; i < SH::NW; ++i) {
    cnt += sh.cl[ph][i];
    dd_add(hi, lo, sh.chi[ph][i], sh.clo[ph][i]);
  }
  ph ^= 1;
}

// Row access: thread t owns the contiguous chunk [lo, hi) (a multiple of
// 4 long, so LDS reads are 16 bytes wide); the row sits in LDS when it
// fits, else it is re-read from global memory on every pass.
template <bool IN_LDS>
struct RowView {
  const float *p;  // LDS copy or global row
  int lo, hi;
  __device__ __forceinline__ void init(const float *grow, float *srow, int M) {
    const int chunk = ((M + PT - 1) / PT + 3) & ~3;
    lo = min(M, (int)threadIdx.x * chunk);
    hi = min(M, lo + chunk);
    if (IN_LDS) {
      // batches of U independent loads per thread, so the copy waits for
      // memory once per batch rather than once per value
      constexpr int U = 16;
      for (int j0 = threadIdx.x; j0 < M; j0 += U * PT) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (j0 + u * PT < M) v[u] = grow[j0 + u * PT];
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (j0 + u * PT < M) srow[j0 + u * PT] = v[u];
      }
      __syncthreads();
      p = srow;
    } else {
      p = grow;
    }
  }
  // f(j, value) over this thread's chunk, ascending j; each_mem is the same
  // here (the register-resident row below reads memory in it instead)
  template <typename F>
  __device__ __forceinline__ void each_mem(F f) const { each(f); }
  template <int G, typename F>
  __device__ __forceinline__ void each_seq(F f) const { each(f); }
  template <typename F>
  __device__ __forceinline__ void each(F f) const {
    int j = lo;
    if (IN_LDS) {
      for (; j + 4 <= hi; j += 4) {
        const float4 q = *(const float4 *)(p + j);
        f(j, q.x);
        f(j + 1, q.y);
        f(j + 2, q.z);
        f(j + 3, q.w);
      }
    }
    for (; j < hi; ++j) f(j, p[j]);
  }
};

// Row held in registers (the SIP kernel for rows of at most 256 CH - 3
// values): thread t owns the CH consecutive positions j0 = t CH - a ..
// j0 + CH - 1, where a (0..3) is the row start's distance in floats from a
// 16-byte boundary, so that every group of four is one aligned 16-byte
// load.  Positions outside [0, M) hold 0, which a SIP plan never counts,
// sums into anything but zero, or draws.  each() runs over the registers
// (fully unrolled); each_mem() re-reads the thread's positions from memory
// in a rolled loop, for the rarely taken double-double and exact
// evaluations and a collection of more than two bracket values per thread,
// whose unrolled code would be large.
template <int CH>
struct RegRow {
  static_assert(CH % 4 == 0, "whole 16-byte groups");
  mutable float v[CH];
  int lo, M;
  const float *g;
  __device__ __forceinline__ void init(const float *grow, int m) {
    const int a = (int)(((uintptr_t)grow >> 2) & 3);
    lo = (int)threadIdx.x * CH - a;
    M = m;
    g = grow;
    // A buffer over positions [-a, M): every group of four is one 16-byte
    // load with no branch, and buffer loads are range-checked per dword, so
    // positions at or past M read as zero (a group wholly past M, or the
    // tail of the one group that straddles M).  Thread 0 zeroes the a
    // positions before the row, which belong to the previous row.
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(grow - a), 0, (M + a) * 4, 0x00020000);
    const int b0 = (int)threadIdx.x * CH * 4;
#pragma unroll
    for (int i = 0; i < CH; i += 4) {
      const f32x4 q = __builtin_amdgcn_raw_buffer_load_b128(rs, b0 + i * 4, 0, 0);
      v[i] = q[0];
      v[i + 1] = q[1];
      v[i + 2] = q[2];
      v[i + 3] = q[3];
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) v[k] = lo + k < 0 ? 0.f : v[k];
  }
  //
  // Passes run in groups of 8 values with a scheduling barrier between
  // groups: unbounded, the compiler computes every value's terms (and keeps
  // every comparison's lane mask) ahead of the accumulations, which takes as
  // many more registers as the row itself.
  template <typename F>
  __device__ __forceinline__ void each(F f) const { each_seq<8>(f); }
  template <int G, typename F>
  __device__ __forceinline__ void each_seq(F f) const {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      asm volatile("" : "+v"(v[i]));
      f(lo + i, v[i]);
      if ((i + 1) % G == 0) __builtin_amdgcn_sched_barrier(0);
    }
  }
  template <typename F>
  __device__ __forceinline__ void each_mem(F f) const {
    const int j1 = min(lo + CH, M);
    for (int j = max(lo, 0); j < j1; ++j) f(j, g[j]);
  }
};

// Double-double sum of {S_j < x} (strict) or {S_j <= x} (!strict), with
// the count of S_j > x.  Per thread: exact two-sums into (hi, lo); then the
// block reduction.  The result's error is below (chunk^2 + 64) 2^-104 of the
// sum (chunk = values per thread).
template <class SH, typename Row>
__device__ __forceinline__ void dd_sum(SH &sh, const Row &row, float x, bool strict, double &hi, double &lo,
                       long long &ngt, int &ph) {
  double h = 0.0, l = 0.0;
  long long c = 0;
  row.each_mem([&](int, float v) {
    const bool in = strict ? v < x : v <= x;
    c += v > x ? 1 : 0;
    double s2, e;
    two_sum(h, in ? (double)v : 0.0, s2, e);
    h = s2;
    l += e;
  });
  const double n = h + l;  // normalise: |l| <= ulp(h) / 2
  l = l - (n - h);
  h = n;
  block_reduce(sh, c, h, l, ph);
  hi = h;
  lo = l;
  ngt = c;
}

// Double-double sum of {S_j <= lo_x} (as dd_sum, same error bound) that also
// collects the row values in (lo_x, hi_x) into sh.col; the caller knows
// there are at most MCAP of them and has cleared sh.ncol.
template <class SH, typename Row>
__device__ __forceinline__ void dd_sum_collect(SH &sh, const Row &row, float lo_x, float hi_x, double &hi,
                               double &lo, int &ph) {
  double h = 0.0, l = 0.0;
  long long c = 0;
  int nin = 0;  // this thread's values inside the bracket (rare)
  // their smallest and largest (positive values): with at most two of them
  // these are the values themselves; only a thread holding more re-reads
  // its part of the row from memory
  float cmin = 3.40282347e38f, cmax = 0.f;
  row.each([&](int, float v) {
    const bool in = v <= lo_x;
    double s2, e;
    two_sum(h, in ? (double)v : 0.0, s2, e);
    h = s2;
    l += e;
    const bool cand = !in && v < hi_x;
    cmin = fminf(cmin, cand ? v : 3.40282347e38f);
    cmax = fmaxf(cmax, cand ? v : 0.f);
    nin += cand ? 1 : 0;
  });
  if (nin > 2) {
    row.each_mem([&](int, float v) {
      if (v > lo_x && v < hi_x) {
        const int slot = atomicAdd(&sh.ncol, 1);
        if (slot < MCAP) sh.col[slot] = v;
      }
    });
  } else if (nin > 0) {
    const int slot = atomicAdd(&sh.ncol, nin);
    if (slot < MCAP) sh.col[slot] = cmin;
    if (nin == 2 && slot + 1 < MCAP) sh.col[slot + 1] = cmax;
  }
  const double n = h + l;
  l = l - (n - h);
  h = n;
  block_reduce(sh, c, h, l, ph);  // its barrier also publishes sh.col
  hi = h;
  lo = l;
}

// Exact sum of {S_j < x} (strict) or {S_j <= x} (!strict) into sh.total as
// 11 normalised 32-bit digits (units of 2^-149).  Only digits dlo..dhi can
// receive a value (the row's exponent range); each thread accumulates them
// in registers, then waves and workgroup add them up.
template <class SH, typename Row>
__device__ __forceinline__ void exact_sum(SH &sh, const Row &row, float x, bool strict, int dlo, int dhi) {
  uint64_t acc[NDIG + 1];
#pragma unroll
  for (int i = 0; i <= NDIG; ++i) acc[i] = 0ull;
  row.each_mem([&](int, float v) {
    const bool in = strict ? v < x : v <= x;
    const unsigned b = in ? __builtin_bit_cast(unsigned, v) : 0u;
    const unsigned e = b >> 23;
    const uint64_t mant = e ? ((b & 0x7fffffu) | 0x800000u) : (b & 0x7fffffu);
    const unsigned shift = e ? e - 1 : 0;
    const uint64_t w = mant << (shift & 31);
    const int d = (int)(shift >> 5);
    const uint64_t wlo = w & 0xffffffffull, whi = w >> 32;
#pragma unroll
    for (int i = 0; i <= NDIG; ++i) {
      if (i < dlo || i > dhi) continue;  // uniform
      acc[i] += (d == i ? wlo : 0ull) + (d + 1 == i ? whi : 0ull);
    }
  });
  const int wv = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i <= NDIG; ++i) {
    if (i < dlo || i > dhi) continue;
    long long a = (long long)acc[i];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o, 64);
    if ((threadIdx.x & 63) == 0) sh.wdig[wv][i] = (uint64_t)a;
  }
  __syncthreads();
  if (threadIdx.x == 0) {  // carry propagation
    uint64_t carry = 0;
    for (int i = 0; i <= NDIG; ++i) {
      uint64_t a = carry;
      if (i >= dlo && i <= dhi)
        for (int k = 0; k < SH::NW; ++k) a += sh.wdig[k][i];
      sh.total[i] = a & 0xffffffffull;
      carry = a >> 32;
    }
  }
  __syncthreads();
}

// Digit index (32-bit digits, units 2^-149) of the low word of an fp32 value.
__device__ __forceinline__ int digit_of(unsigned b) {
  const unsigned e = b >> 23;
  return (int)((e ? e - 1 : 0) >> 5);
}

// Correct rounding (nearest even) of the integer held in `dig` (units 2^-149).
__device__ double digits_to_double(const uint64_t *dig) {
  int top = -1;
  for (int i = NDIG; i >= 0; --i)
    if (dig[i]) {
      top = i;
      break;
    }
  if (top < 0) return 0.0;
  // 128-bit window of the four highest digits; its lowest bit has weight 2^base
  unsigned __int128 w = 0;
  for (int i = top; i >= top - 3; --i) w = (w << 32) | (unsigned __int128)(i >= 0 ? dig[i] : 0u);
  const int base = 32 * (top - 3);
  bool low_nz = false;  // any set bit below the window
  for (int i = top - 4; i >= 0; --i) low_nz |= dig[i] != 0;
  const int p = 32 * top + 31 - __builtin_clz((unsigned)dig[top]);  // highest set bit
  const int sh_m = p - 52 - base;  // window bit of the mantissa's lowest bit (>= 43)
  uint64_t m = (uint64_t)(w >> sh_m) & ((1ull << 53) - 1);
  if (p <= 52) return ldexp((double)m, base + sh_m - 149);  // exact (never below 53 bits here)
  const bool rnd = (w >> (sh_m - 1)) & 1;
  const bool sticky = low_nz || (w & (((unsigned __int128)1 << (sh_m - 1)) - 1)) != 0;
  int ex = p - 52;
  if (rnd && (sticky || (m & 1ull))) {
    ++m;
    if (m == (1ull << 53)) {
      m >>= 1;
      ++ex;
    }
  }
  return ldexp((double)m, ex - 149);
}

// (mult * x) as digits (units 2^-149), x a positive finite fp32 value.
__device__ void scaled_to_digits(unsigned long long mult, float x, uint64_t *dig) {
  for (int i = 0; i <= NDIG; ++i) dig[i] = 0;
  const unsigned b = __builtin_bit_cast(unsigned, x);
  const unsigned e = b >> 23;
  const uint64_t mant = e ? ((b & 0x7fffffu) | 0x800000u) : (b & 0x7fffffu);
  const unsigned shift = e ? e - 1 : 0;
  // mult < 2^21, mant < 2^24: product < 2^45 fits 64 bits
  const unsigned __int128 v = (unsigned __int128)(mult * mant) << (shift & 31);
  const unsigned d = shift >> 5;
  dig[d] = (uint64_t)(v & 0xffffffffu);
  dig[d + 1] = (uint64_t)((v >> 32) & 0xffffffffu);
  if (d + 2 <= (unsigned)NDIG) dig[d + 2] = (uint64_t)(v >> 64);
}

// a >= b for normalised digit arrays.
__device__ bool digits_ge(const uint64_t *a, const uint64_t *b) {
  for (int i = NDIG; i >= 0; --i)
    if (a[i] != b[i]) return a[i] > b[i];
  return true;
}

// The saturation threshold of a SIP row with more than s positive scores,
// by the decision procedure of the file header: nsat = r = #{S > x*} and
// Tr = sum_{S <= x*} S correctly rounded to fp64.  PTH threads; every
// thread's fp32 partial sums cover at most `chunk` row values; npos, mx,
// mnpos (bit patterns of the largest and the smallest positive value) and
// the approximate total tot come from the row's first pass.  Both plan
// kernels take their decisions here, so they agree bit for bit.
template <int PTH, class SH, typename Row>
__device__ __forceinline__ void sip_threshold(SH &sh, const Row &row, int M, int s, long long npos, unsigned mx,
                              unsigned mnpos, double tot, int chunk, long long &nsat,
                              double &Tr) {
  const int t = threadIdx.x;
  // cond(x): (s - #{S >= x}) x <= sum_{S < x} S, decided with a certified
  // fp64 margin or, inside the margin, from a double-double sum and, if
  // even that cannot decide, exactly.  The search visits one point per
  // iteration (a single evaluation site keeps the register footprint of
  // the unrolled row passes small):
  //   stage 0  x = max S           (true: no saturated block); needed only
  //            when max S <= T / s, since cond(x) fails for every x > T / s
  //   stage 1  secant steps down from T / s towards the threshold
  //   stage 2  bisection of [blo, bhi) until no row value lies inside
  // per-thread fp32 partial sums (chunk terms) then an fp64 reduction
  const double err_bound =
      (ldexp((double)(chunk + 2), -23) + ldexp((double)(M + 2 * PTH), -50)) * tot;
  const double dd_rel = ldexp((double)chunk * (double)chunk + 64.0, -104) * 2.0;  // safety x2
  const int dlo = digit_of(mnpos), dhi = digit_of(mx) + 1;
  const float fmx = __builtin_bit_cast(float, mx);
  // nge_lo = #{S >= blo} bounds the values left in (blo, bhi) from above
  unsigned blo = mnpos, bhi = mx;
  long long nge_lo = npos, nge_hi = 0;
  float x = fmx;
  int stage = 0, secant_left = 12, ph = 0;
  float xstar = fmx;
  {
    const float x0 = (float)(tot / (double)s * (1.0 + 0x1p-20));  // above T / s
    if (x0 < fmx && __builtin_bit_cast(unsigned, x0) > blo) {
      x = x0;
      stage = 1;
    }
  }
  bool collect = false;
  while (stage != 3) {
    // ---- one pass at x
    bool holds = true;
    long long cnt = 0;
    double slt = 0.0;
    {
      int cge = 0;
      float sf = 0.f;
      row.each([&](int, float v) {
        const bool ge = v >= x;
        cge += ge ? 1 : 0;
        sf += ge ? 0.f : v;
      });
      cnt = cge;
      slt = (double)sf;
      block_reduce(sh, cnt, slt, ph);
    }
    const long long nge = cnt;
    const long long mult = (long long)s - nge;
    if (mult > 0) {
      const double lhs = (double)mult * (double)x;  // exact: < 2^21 times a 24-bit value
      const double diff = lhs - slt;
      if (diff > err_bound) {
        holds = false;
      } else if (!(diff < -err_bound)) {
        // inside the fp32 margin (common at high budgets): the sum again in
        // fp64, from the row's own copy (registers or LDS), whose error is
        // below (chunk - 1 + 6 + NW) u per term of the total (sequential sum,
        // then the butterfly and the waves); bounded here with room to spare
        double s64 = 0.0;
        row.each([&](int, float v) { s64 += v < x ? (double)v : 0.0; });
        long long none = 0;
        block_reduce(sh, none, s64, ph);
        const double d64 = lhs - s64;
        const double err64 = ldexp((double)(chunk + 16), -52) * tot * (1.0 + 0x1p-30);
        if (d64 > err64) {
          holds = false;
        } else if (!(d64 < -err64)) {
        // inside that margin too: double-double sum of {S < x}
        double thi, tlo;
        long long unused;
        dd_sum(sh, row, x, true, thi, tlo, unused, ph);
        double p, q;
        two_sum(lhs, -thi, p, q);  // lhs - thi = p + q exactly
        const double d = p + (q - tlo);
        const double margin = dd_rel * thi + 0x1p-100 * (lhs + thi);
        if (d > margin) {
          holds = false;
        } else if (!(d < -margin)) {
          exact_sum(sh, row, x, true, dlo, dhi);
          uint64_t ldig[NDIG + 1];
          scaled_to_digits((unsigned long long)mult, x, ldig);
          holds = digits_ge(sh.total, ldig);
        }
        }
      }
    }
    // ---- advance the search
    const unsigned xb = __builtin_bit_cast(unsigned, x);
    if (stage == 0) {
      if (holds) {  // no saturated block: x* = max S
        xstar = x;
        stage = 3;
        continue;
      }
      nge_hi = nge;
      stage = 1;
      x = fminf(fmx, (float)(tot / (double)s * (1.0 + 0x1p-20)));  // x > T/s never holds
      if (!(__builtin_bit_cast(unsigned, x) > blo && __builtin_bit_cast(unsigned, x) < bhi)) stage = 2;
      else continue;
    } else if (stage == 1) {
      if (holds) {
        blo = xb;
        nge_lo = nge;
        stage = 2;
      } else {
        bhi = xb;
        nge_hi = nge;
        // secant step x' = sum_{S<x} / (s - #{S >= x}), aimed 2^-12 low so
        // that the test at x' is decided by the fp64 margin
        const float xn = (float)(slt / (double)mult * (1.0 - 0x1p-12));
        unsigned xnb = xn < x ? __builtin_bit_cast(unsigned, xn) : xb - 1u;
        xnb = max(blo + 1u, xnb);
        if (--secant_left > 0 && xnb > blo && xnb < bhi) {
          x = __builtin_bit_cast(float, xnb);
          continue;
        }
        stage = 2;
      }
    } else {  // stage 2: x was a bisection point
      if (holds) {
        blo = xb;
        nge_lo = nge;
      } else {
        bhi = xb;
        nge_hi = nge;
      }
    }
    // stage 2: few enough values left inside the bracket to resolve them
    // directly (below), else the next bisection point, or done
    if (stage == 2 && nge_lo > nge_hi && nge_lo - nge_hi <= MCAP) {
      collect = true;
      stage = 3;
      continue;
    }
    if (bhi - blo > 1 && nge_lo > nge_hi) {
      x = __builtin_bit_cast(float, blo + (bhi - blo) / 2);
      continue;
    }
    // no row value inside (blo, bhi): x* = blo, and #{S > blo} = #{S >= bhi}
    // = nge_hi (bhi has been tested here: by stage 0, or as a failing secant
    // or bisection point).  The collect pass below (registers only) gives
    // T_r, with nothing to collect.
    xstar = __builtin_bit_cast(float, blo);
    collect = true;
    stage = 3;
  }

  // T_r = sum_{S <= x*} correctly rounded, r = #{S > x*}
  double thi, tlo;
  double E;  // bound on |exact sum - (thi + tlo)|
  if (collect) {
    // The bracket (blo, bhi) holds m <= MCAP row values (at most
    // nge_lo - nge_hi).  One pass sums
    // {S <= blo} and collects them; cond is then taken at each collected
    // value v (nge(v) = nge_hi + #{collected >= v}, slt(v) = sum_{S <= blo}
    // + sum of collected values below v) with the certified double-double
    // margin, and x* is the largest value where it holds (blo if none).
    // cond is monotone, so this is the partition the bisection would find.
    const float flo = __builtin_bit_cast(float, blo), fhi = __builtin_bit_cast(float, bhi);
    if (t == 0) sh.ncol = 0;
    __syncthreads();
    double shi, slo;
    dd_sum_collect(sh, row, flo, fhi, shi, slo, ph);
    // the values actually collected: nge_lo - nge_hi can count more (it
    // counts the values equal to blo too)
    const int m = min(sh.ncol, MCAP);
    const double mrel = dd_rel + 0x1p-90;  // the sum plus up to MCAP exact-rounded terms
    if (t < 64) {
      const float v = t < m ? sh.col[t] : 0.f;
      double bh = 0.0, bl = 0.0;  // collected values below v
      long long ge = 0;           // collected values >= v
      for (int j = 0; j < m; ++j) {
        const float u = sh.col[j];
        if (u < v) {
          double s2, e;
          two_sum(bh, (double)u, s2, e);
          bh = s2;
          bl += e;
        } else {
          ++ge;
        }
      }
      if (t < m) {
        int st = 1;
        const long long mult = (long long)s - nge_hi - ge;
        if (mult > 0) {
          double rh = shi, rl = slo;
          dd_add(rh, rl, bh, bl);
          const double lhs = (double)mult * (double)v;  // exact
          double p, q;
          two_sum(lhs, -rh, p, q);
          const double d = p + (q - rl);
          const double margin = mrel * rh + 0x1p-100 * (lhs + rh);
          st = d > margin ? 0 : (d < -margin ? 1 : 2);
        }
        sh.cstat[t] = st;
      }
    }
    __syncthreads();
    // certain bounds, then any undecided values between them in ascending
    // order, each decided exactly (every thread takes the same steps)
    float vt = flo, vf = fhi;
    for (int j = 0; j < m; ++j) {
      const float u = sh.col[j];
      const int st = sh.cstat[j];
      if (st == 1 && u > vt) vt = u;
      if (st == 0 && u < vf) vf = u;
    }
    for (;;) {
      float nxt = vf;
      for (int j = 0; j < m; ++j) {
        const float u = sh.col[j];
        if (sh.cstat[j] == 2 && u > vt && u < nxt) nxt = u;
      }
      if (!(nxt < vf)) break;
      long long ge = nge_hi;
      for (int j = 0; j < m; ++j) ge += sh.col[j] >= nxt ? 1 : 0;
      const long long mult = (long long)s - ge;
      bool holds = true;
      if (mult > 0) {
        exact_sum(sh, row, nxt, true, dlo, dhi);
        uint64_t ldig[NDIG + 1];
        scaled_to_digits((unsigned long long)mult, nxt, ldig);
        holds = digits_ge(sh.total, ldig);
      }
      if (!holds) break;
      vt = nxt;
    }
    xstar = vt;
    nsat = nge_hi;
    thi = shi;
    tlo = slo;
    for (int j = 0; j < m; ++j) {
      const float u = sh.col[j];
      if (u > xstar) {
        ++nsat;
      } else {
        double s2, e;
        two_sum(thi, (double)u, s2, e);
        thi = s2;
        tlo += e;
      }
    }
    const double n2 = thi + tlo;
    tlo = tlo - (n2 - thi);
    thi = n2;
    E = mrel * thi;
  } else {
    dd_sum(sh, row, xstar, false, thi, tlo, nsat, ph);
    E = dd_rel * thi;
  }
  {
    // thi = RN(thi + tlo); the exact sum lies within E of thi + tlo.  It
    // rounds to thi when that interval stays strictly inside thi's rounding
    // interval (half an ulp above, half the ulp below under it).
    const unsigned long long tb = __builtin_bit_cast(unsigned long long, thi);
    const double up = __builtin_bit_cast(double, tb + 1ull) - thi;
    const double down = thi > 0.0 ? thi - __builtin_bit_cast(double, tb - 1ull) : up;
    if (tlo + E < 0.5 * up && tlo - E > -0.5 * down) {
      Tr = thi;
    } else {
      exact_sum(sh, row, xstar, false, dlo, dhi);
      if (t == 0) sh.bcast_d = digits_to_double(sh.total);
      __syncthreads();
      Tr = sh.bcast_d;
    }
  }
}

template <bool IN_LDS>
__global__ __launch_bounds__(PT) void plan_kernel(PlanArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  Shared &sh = *reinterpret_cast<Shared *>(smem_raw);
  float *srow = reinterpret_cast<float *>(smem_raw + ((sizeof(Shared) + 15) & ~(size_t)15));
  const int t = threadIdx.x;
  const size_t r = blockIdx.x;
  const int M = a.M, s = a.budget;
  int32_t *out_idx = a.idx + r * (size_t)s;
  float *out_bias = a.bias ? a.bias + r * (size_t)s : nullptr;
  RowView<IN_LDS> row;
  row.init(a.scores + r * (size_t)M, srow, M);

  // ---- phase 0: validity, positives, extremes, approximate total
  long long npos = 0, nbad = 0;
  unsigned mx = 0, mnpos = 0x7f800000u;
  double tot = 0.0;
  row.each([&](int, float v) {
    const unsigned b = __builtin_bit_cast(unsigned, v);
    if (!(v >= 0.f) || (b & 0x7fffffffu) >= 0x7f800000u) {
      ++nbad;
    } else if (v > 0.f) {
      ++npos;
      mx = max(mx, b);
      mnpos = min(mnpos, b);
      tot += (double)v;
    }
  });
  nbad = block_sum_l(sh, nbad);
  npos = block_sum_l(sh, npos);
  tot = block_sum_d(sh, tot);
  block_minmax_u(sh, mnpos, mx);

  auto fill_rest = [&](int from) {
    for (int e = from + t; e < s; e += PT) {
      out_idx[e] = -1;
      if (out_bias) out_bias[e] = 0.f;
    }
  };

  if (nbad) {
    fill_rest(0);
    if (t == 0) {
      a.count[r] = -1;
      if (a.lambda) a.lambda[r] = __builtin_nan("");
      if (a.status) *a.status = BSA_ERR_NONFINITE;  // every writer stores the same value
    }
    return;
  }

  if (a.mode == BSA_PLAN_TOPK) {
    // s-th largest value v: largest bit pattern x with #{S >= x} >= s.
    unsigned blo = 0, bhi = mx + 1;  // #{S >= 0} = M >= s ; #{S >= bhi} = 0 < s
    while (bhi - blo > 1) {
      const unsigned mid = blo + (bhi - blo) / 2;
      const float xm = __builtin_bit_cast(float, mid);
      long long c = 0;
      row.each([&](int, float v) { c += v >= xm ? 1 : 0; });
      c = block_sum_l(sh, c);
      if (c >= s) blo = mid; else bhi = mid;
    }
    const float v = __builtin_bit_cast(float, blo);
    long long ngt = 0, ntie = 0;
    row.each([&](int, float x) {
      ngt += x > v ? 1 : 0;
      ntie += x == v ? 1 : 0;
    });
    ngt = block_sum_l(sh, ngt);
    const long long need = s - ngt;
    uint64_t tie_total;
    const uint64_t tie_base = block_exscan_u64(sh, (uint64_t)ntie, tie_total);
    long long nsel = 0;
    {
      uint64_t tr = tie_base;
      row.each([&](int, float x) {
        bool sel = x > v;
        if (x == v) {
          sel = (long long)tr < need;
          ++tr;
        }
        nsel += sel ? 1 : 0;
      });
    }
    uint64_t sel_total;
    uint64_t pos = block_exscan_u64(sh, (uint64_t)nsel, sel_total);
    {
      uint64_t tr = tie_base;
      row.each([&](int j, float x) {
        bool sel = x > v;
        if (x == v) {
          sel = (long long)tr < need;
          ++tr;
        }
        if (sel) {
          out_idx[pos] = j;
          if (out_bias) out_bias[pos] = 0.f;
          ++pos;
        }
      });
    }
    if (t == 0) {
      a.count[r] = s;
      if (a.lambda) a.lambda[r] = 0.0;
    }
    return;
  }

  // ---- SIP
  if (npos <= s) {
    uint64_t total;
    long long mine = 0;
    row.each([&](int, float x) { mine += x > 0.f ? 1 : 0; });
    uint64_t pos = block_exscan_u64(sh, (uint64_t)mine, total);
    row.each([&](int j, float x) {
      if (x > 0.f) {
        out_idx[pos] = j;
        if (out_bias) out_bias[pos] = 0.f;
        ++pos;
      }
    });
    fill_rest((int)npos);
    if (t == 0) {
      a.count[r] = (int)npos;
      if (a.lambda) a.lambda[r] = __builtin_inf();
    }
    return;
  }

  const int chunk = ((M + PT - 1) / PT + 3) & ~3;
  long long nsat;
  double Tr;
  sip_threshold<PT>(sh, row, M, s, npos, mx, mnpos, tot, chunk, nsat, Tr);
  const double lam = (double)(s - nsat) / Tr;

  const uint64_t U = a.offsets ? a.offsets[r] : offset_of_row(a.seed, r);
  // Pi_j = floor(min(1, lam S_j) 2^44) = floor(min(2^44, lam' S_j)) with
  // lam' = lam 2^44 (exact: power-of-two scaling commutes with rounding);
  // floor, then + 2^52 puts the integer in the low mantissa bits.
  const double lam44 = lam * (double)UNIT;
  auto fixed_pi = [&](float v) -> uint64_t {
    const double y = __builtin_floor(fmin((double)UNIT, lam44 * (double)v)) + 0x1p52;
    return __builtin_bit_cast(uint64_t, y) & ((1ull << 52) - 1);
  };
  uint64_t mine = 0;
  row.each([&](int, float v) { mine += fixed_pi(v); });
  uint64_t csum_total;
  const uint64_t C0 = block_exscan_u64(sh, mine, csum_total);
  // With D = C - U, the number of points U + k 2^44 (k >= 0) below C is
  // ((D - 1) >> 44) + 1 (arithmetic shift; 0 while D <= 0).  Block j holds
  // a point exactly when that number grows across it.
  long long qprev = (((long long)C0 - (long long)U) - 1) >> 44;  // points below C, minus 1
  long long D = (long long)C0 - (long long)U;
  row.each([&](int j, float v) {
    const uint64_t Pi = fixed_pi(v);
    D += (long long)Pi;
    const long long q = (D - 1) >> 44;
    if (q > qprev && qprev + 1 < (long long)s) out_idx[qprev + 1] = j;
    qprev = q;
  });
  auto below = [&](uint64_t c) -> uint64_t {  // points U + k 2^44 (k < s) below c
    if (c <= U) return 0;
    const uint64_t n = ((c - U - 1) >> 44) + 1;
    return n < (uint64_t)s ? n : (uint64_t)s;
  };
  const int drawn = (int)below(csum_total);
  if (out_bias) {
    // shifts -ln pi of the drawn blocks, one slot per thread (the indices
    // were written by this workgroup before the barrier)
    __syncthreads();
    constexpr int U = 4;  // independent index loads before the first wait
    for (int e0 = t; e0 < drawn; e0 += U * PT) {
      int jj[U];
#pragma unroll
      for (int u = 0; u < U; ++u) jj[u] = e0 + u * PT < drawn ? out_idx[e0 + u * PT] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (e0 + u * PT < drawn) {
          const double pi = fmin(1.0, lam * (double)row.p[jj[u]]);
          out_bias[e0 + u * PT] = (float)(-log(pi));
        }
    }
  }
  fill_rest(drawn);
  if (t == 0) {
    a.count[r] = drawn;
    if (a.lambda) a.lambda[r] = lam;
  }
}

// SIP plan of rows that fit 256 CH - 3 values, the row in registers (no
// LDS copy, no LDS reads; only the reductions use LDS, so several rows run
// per CU).  The same definition as plan_kernel (the threshold search is the
// same function), with two leaner sampling passes:
//   * sum pass: Pi_j = floor(min(2^44, lambda 2^44 S_j)) summed per thread
//     in fp64, exact (at most 120 terms below 2^44 stay below 2^52);
//   * draw pass: with C0 the exclusive prefix of the thread's chunk and the
//     first sampling point at or above it at C0 + R (R < 2^44 + 2^44,
//     exact in fp64), block j is drawn when R < L_j, the chunk-local prefix
//     after it; then R grows by 2^44 (one point per block at most, since
//     Pi_j <= 2^44), or becomes infinite after the s-th point.
//   * STAGED (budgets to kStageMax): the draw pass puts each drawn block and
//     its score into LDS, and after one barrier a last pass writes the index
//     and shift lists in order, coalesced (the shifts -ln pi computed there);
//     otherwise the draw pass writes the indices and parks the scores in the
//     shift slots, and a last pass turns those into shifts.
// Rows in flight per CU for a chunk of CH values (the register budget).
constexpr int sip_rows_per_cu(int ch) { return ch <= 32 ? 4 : (ch <= 80 ? 3 : 2); }
// Largest budget whose staged draws (8 bytes each) leave LDS for every row
// in flight: 4 rows of 32 KB at the smallest chunk.
constexpr int kStageMax = 4096;

template <int CH, bool STAGED>
__global__ __launch_bounds__(256, sip_rows_per_cu(CH)) void sip_reg_kernel(PlanArgs a) {
  constexpr int PTR = 256;
  __shared__ SharedT<PTR / 64> sh;
  extern __shared__ __attribute__((aligned(16))) unsigned char stage_raw[];
  int32_t *st_idx = (int32_t *)stage_raw;                         // [budget]
  float *st_val = (float *)(stage_raw + 4 * (size_t)a.budget);  // [budget]
  const int t = threadIdx.x;
  const size_t r = blockIdx.x;
  const int M = a.M, s = a.budget;
  int32_t *out_idx = a.idx + r * (size_t)s;
  float *out_bias = a.bias ? a.bias + r * (size_t)s : nullptr;
  const float *grow = a.scores + r * (size_t)M;
  RegRow<CH> row;
  row.init(grow, M);

  // ---- validity (NaN, infinities, negative values), positives, extremes,
  // approximate total
  int mypos = 0, bad = 0;
  float mxf = 0.f, mnf = __builtin_inff();
  double tot = 0.0;
  row.each([&](int, float v) {
    bad |= (v < 0.f || !(v <= 3.40282347e38f)) ? 1 : 0;
    const bool pos = v > 0.f;
    mypos += pos ? 1 : 0;
    mxf = fmaxf(mxf, v);
    mnf = pos ? fminf(mnf, v) : mnf;
    tot += (double)v;
  });
  long long pk = ((long long)bad << 32) | (long long)mypos;
  unsigned mx = __builtin_bit_cast(unsigned, mxf), mnpos = __builtin_bit_cast(unsigned, mnf);
  block_reduce_first(sh, pk, tot, mnpos, mx);
  const long long nbad = pk >> 32;
  long long npos = pk & 0xffffffffll;

  auto fill_rest = [&](int from) {
    for (int e = from + t; e < s; e += PTR) {
      out_idx[e] = -1;
      if (out_bias) out_bias[e] = 0.f;
    }
  };
  if (nbad) {
    fill_rest(0);
    if (t == 0) {
      a.count[r] = -1;
      if (a.lambda) a.lambda[r] = __builtin_nan("");
      if (a.status) *a.status = BSA_ERR_NONFINITE;  // every writer stores the same value
    }
    return;
  }
  if (npos <= s) {  // every positive block, pi = 1
    uint64_t total;
    uint64_t pos = block_exscan_u64(sh, (uint64_t)mypos, total);
    row.each([&](int j, float x) {
      if (x > 0.f) {
        out_idx[pos] = j;
        if (out_bias) out_bias[pos] = 0.f;
        ++pos;
      }
    });
    fill_rest((int)npos);
    if (t == 0) {
      a.count[r] = (int)npos;
      if (a.lambda) a.lambda[r] = __builtin_inf();
    }
    return;
  }

  long long nsat;
  double Tr;
  sip_threshold<PTR>(sh, row, M, s, npos, mx, mnpos, tot, CH, nsat, Tr);
  const double lam = (double)(s - nsat) / Tr;
  const uint64_t U = a.offsets ? a.offsets[r] : offset_of_row(a.seed, r);
  const double lam44 = lam * (double)UNIT;  // exact: a power-of-two scaling
  double mysum = 0.0;
  row.template each_seq<8>([&](int, float v) {
    mysum += __builtin_floor(fmin((double)UNIT, lam44 * (double)v));
  });
  uint64_t total;
  const uint64_t C0 = block_exscan_u64(sh, (uint64_t)mysum, total);
  auto below = [&](uint64_t c) -> uint64_t {  // points U + k 2^44 (k < s) below c
    if (c <= U) return 0;
    const uint64_t n = ((c - U - 1) >> 44) + 1;
    return n < (uint64_t)s ? n : (uint64_t)s;
  };
  const int drawn = (int)below(total);
  int q = (int)below(C0);  // points below the chunk: the next one is number q
  double R = q < s ? (double)((long long)q * (long long)UNIT - ((long long)C0 - (long long)U))
                   : __builtin_inf();
  double L = 0.0;
  row.template each_seq<8>([&](int j, float v) {
    L += __builtin_floor(fmin((double)UNIT, lam44 * (double)v));
    if (R < L) {
      if (STAGED) {
        st_idx[q] = j;
        st_val[q] = v;
      } else {
        out_idx[q] = j;
        if (out_bias) out_bias[q] = v;  // the score, turned into its shift below
      }
      ++q;
      R = q < s ? R + (double)UNIT : __builtin_inf();
    }
  });
  if (STAGED) {
    __syncthreads();
    for (int e = t; e < s; e += PTR) {
      const bool d = e < drawn;
      out_idx[e] = d ? st_idx[e] : -1;
      if (out_bias) out_bias[e] = d ? (float)(-log(fmin(1.0, lam * (double)st_val[e]))) : 0.f;
    }
    if (t == 0) {
      a.count[r] = drawn;
      if (a.lambda) a.lambda[r] = lam;
    }
    return;
  }
  if (out_bias) {
    // shifts -ln pi of the drawn blocks, from the scores parked in their
    // slots (written by this workgroup before the barrier)
    __syncthreads();
    constexpr int UB = 8;  // all of a thread's loads (budgets to 2048) before the first wait
    for (int e0 = t; e0 < drawn; e0 += UB * PTR) {
      float vv[UB];
#pragma unroll
      for (int u = 0; u < UB; ++u) vv[u] = e0 + u * PTR < drawn ? out_bias[e0 + u * PTR] : 1.f;
#pragma unroll
      for (int u = 0; u < UB; ++u)
        if (e0 + u * PTR < drawn) out_bias[e0 + u * PTR] = (float)(-log(fmin(1.0, lam * (double)vv[u])));
    }
  }
  fill_rest(drawn);
  if (t == 0) {
    a.count[r] = drawn;
    if (a.lambda) a.lambda[r] = lam;
  }
}

__global__ void status_init_kernel(int32_t *status) { *status = BSA_OK; }

}  // namespace

int launch_sip_plan(const float *scores, int rows, int nqb, int M, int budget, int mode,
                    uint64_t seed, const uint64_t *offsets, int32_t *idx, float *bias,
                    int32_t *count, double *lambda, int32_t *status, hipStream_t stream) {
  clear_pending_error();
  (void)nqb;
  PlanArgs a{scores, rows, M, budget, mode, seed, offsets, idx, bias, count, lambda, status};
  // the status word is set by a kernel (not a memset) so that the call can
  // be captured into a graph and replayed
  if (status) hipLaunchKernelGGL(status_init_kernel, dim3(1), dim3(1), 0, stream, status);
  int dev = 0, max_lds = 65536;
  if (hipGetDevice(&dev) != hipSuccess) return BSA_ERR_HIP;
  if (hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
      hipSuccess)
    return BSA_ERR_HIP;
  const size_t base = (sizeof(Shared) + 15) & ~(size_t)15;
  const size_t with_row = base + (size_t)(M + 4) * sizeof(float);
  // SIP rows that fit a register-resident instance (the row's start may sit
  // up to 3 floats past a 16-byte boundary)
  const long long span = (long long)M + 3;
  const bool staged = budget <= kStageMax;
  const size_t stage = staged ? (size_t)budget * 8 : 0;
  // Budgets of half the row or more (but below the whole row, which needs no
  // search), past the staged range, go to the 512-thread kernel when the row
  // fits its LDS: there the searches take more passes and the sampling
  // writes most of the row, and twice the threads with the row in LDS
  // measured faster (40 heads of 18,900 blocks: 2.80 against 2.94 ms at
  // half the row, 3.31 against 4.14 at three quarters, 3.91 against 4.93 at
  // 90 %).
  const bool wide = mode == BSA_PLAN_SIP && !staged && 2 * (long long)budget >= M && budget < M &&
                    with_row <= (size_t)max_lds;
  if (wide) {
    hipLaunchKernelGGL(plan_kernel<true>, dim3(rows), dim3(PT), with_row, stream, a);
  } else if (mode == BSA_PLAN_SIP && span <= 256 * 32) {
    if (staged) hipLaunchKernelGGL((sip_reg_kernel<32, true>), dim3(rows), dim3(256), stage, stream, a);
    else hipLaunchKernelGGL((sip_reg_kernel<32, false>), dim3(rows), dim3(256), 0, stream, a);
  } else if (mode == BSA_PLAN_SIP && span <= 256 * 80) {
    if (staged) hipLaunchKernelGGL((sip_reg_kernel<80, true>), dim3(rows), dim3(256), stage, stream, a);
    else hipLaunchKernelGGL((sip_reg_kernel<80, false>), dim3(rows), dim3(256), 0, stream, a);
  } else if (mode == BSA_PLAN_SIP && span <= 256 * 120) {
    if (staged) hipLaunchKernelGGL((sip_reg_kernel<120, true>), dim3(rows), dim3(256), stage, stream, a);
    else hipLaunchKernelGGL((sip_reg_kernel<120, false>), dim3(rows), dim3(256), 0, stream, a);
  } else if (with_row <= (size_t)max_lds)
    hipLaunchKernelGGL(plan_kernel<true>, dim3(rows), dim3(PT), with_row, stream, a);
  else
    hipLaunchKernelGGL(plan_kernel<false>, dim3(rows), dim3(PT), base, stream, a);
  return status_of(hipGetLastError());
}

}  // namespace bsa
