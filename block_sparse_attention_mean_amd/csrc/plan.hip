// Sampling plan kernel (SIP or top-k) for gfx950.
//
// AB-Attention page (onedev.kr/papers/1521), section "어떻게 쓰나": per query
// block i, pi_ij = min(1, lambda_i S_ij) with sum_j pi_ij = s; blocks with
// pi = 1 are always kept; a systematic sample draws exactly s distinct
// blocks shared by the whole query block.  Top-k at the same budget is the
// "SIP without pi weighting" level of the ablation paragraph in "전제와 한계".
//
// One workgroup (256 threads) per row.  The row sits in LDS when it fits.
//
// SIP, exactly as the C ABI documents it:
//   * the number r of saturated blocks is the smallest r with
//     (s - r) S_(r+1) <= T_r.  Over the row values v this reads
//     cond(v): (s - #{S >= v}) v <= sum_{S < v} S, which is monotone in v;
//     a bisection over fp32 bit patterns finds the largest x with cond(x),
//     and then r = #{S > x}, T_r = sum_{S <= x} S;
//   * each bisection step decides cond from an fp64 sum whose rounding
//     error is bounded; only when the margin is inside that bound is the
//     sum recomputed exactly (integer superaccumulator, 320 bits in units
//     of 2^-149, which holds every fp32 value and 2^20 of them);
//   * T_r is always taken from the superaccumulator and rounded once to
//     fp64 (round to nearest even); lambda = (s - r) / T_r is one IEEE
//     division and pi_j = min(1, lambda S_j) one IEEE multiply;
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

constexpr int PT = 256;               // threads per row
constexpr int NW = PT / 64;           // waves
constexpr int NDIG = 10;              // 32-bit digits of the superaccumulator
constexpr uint64_t UNIT = 1ull << 44;  // fixed-point 1.0 of pi

struct PlanArgs {
  const float *scores;
  int rows, M, budget, mode;
  uint64_t seed;
  const uint64_t *offsets;
  int32_t *idx;
  float *bias;
  int32_t *count;
  double *lambda;
};

struct Shared {
  uint64_t digits[NDIG * PT];   // per-thread carry-save digits [digit][thread]
  uint64_t total[NDIG + 1];     // normalised digits of the last exact sum
  double red_d[NW];
  long long red_l[NW];
  unsigned red_u[NW];
  unsigned red_u2[NW];
  int flag;
  double bcast_d;
};

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
__device__ double block_sum_d(Shared &sh, double v) {
  v = wave_sum_d(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.red_d[w] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < NW; ++i) t += sh.red_d[i];
  return t;
}
__device__ long long block_sum_l(Shared &sh, long long v) {
  v = wave_sum_l(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.red_l[w] = v;
  __syncthreads();
  long long t = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) t += sh.red_l[i];
  return t;
}
__device__ void block_minmax_u(Shared &sh, unsigned &mn, unsigned &mx) {
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
  for (int i = 1; i < NW; ++i) {
    mn = min(mn, sh.red_u[i]);
    mx = max(mx, sh.red_u2[i]);
  }
}
// Exclusive prefix over threads (thread order) of a 64-bit count.
__device__ uint64_t block_exscan_u64(Shared &sh, uint64_t v, uint64_t &total) {
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
  for (int i = 0; i < NW; ++i) {
    const uint64_t t = (uint64_t)sh.red_l[i];
    if (i < w) base += t;
    total += t;
  }
  return base + inc - v;
}

// Exact sum of {S_j : S_j < x} (strict) or {S_j <= x} (!strict) into
// sh.total as 11 normalised 32-bit digits (units of 2^-149).
template <typename RowT>
__device__ void exact_sum(Shared &sh, RowT row, int lo, int hi, float x, bool strict) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < NDIG; ++i) sh.digits[i * PT + t] = 0ull;
  for (int j = lo; j < hi; ++j) {
    const float s = row[j];
    if (strict ? !(s < x) : !(s <= x)) continue;
    const unsigned b = __builtin_bit_cast(unsigned, s);
    const unsigned e = b >> 23;
    const uint64_t mant = e ? ((b & 0x7fffffu) | 0x800000u) : (b & 0x7fffffu);
    const unsigned shift = e ? e - 1 : 0;
    const uint64_t v = mant << (shift & 31);
    const unsigned d = shift >> 5;
    atomicAdd((unsigned long long *)&sh.digits[d * PT + t], (unsigned long long)(v & 0xffffffffull));
    atomicAdd((unsigned long long *)&sh.digits[(d + 1) * PT + t], (unsigned long long)(v >> 32));
  }
  __syncthreads();
  if (t < NDIG) {
    uint64_t acc = 0;
    for (int i = 0; i < PT; ++i) acc += sh.digits[t * PT + i];
    sh.digits[t * PT] = acc;  // column total parked in slot 0
  }
  __syncthreads();
  if (t == 0) {
    uint64_t carry = 0;
    for (int i = 0; i < NDIG; ++i) {
      const uint64_t x2 = sh.digits[i * PT] + carry;
      sh.total[i] = x2 & 0xffffffffull;
      carry = x2 >> 32;
    }
    sh.total[NDIG] = carry;
  }
  __syncthreads();
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
  const int p = 32 * top + 31 - __builtin_clz((unsigned)dig[top]);  // highest set bit
  auto bit = [&](int k) -> uint64_t { return k < 0 ? 0ull : ((dig[k >> 5] >> (k & 31)) & 1ull); };
  if (p <= 52) {
    uint64_t m = 0;
    for (int k = p; k >= 0; --k) m = (m << 1) | bit(k);
    return ldexp((double)m, -149);
  }
  uint64_t m = 0;
  for (int k = p; k >= p - 52; --k) m = (m << 1) | bit(k);
  const uint64_t rnd = bit(p - 53);
  bool sticky = false;
  for (int k = p - 54; k >= 0 && !sticky; --k) sticky = bit(k) != 0;
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

template <bool IN_LDS>
__global__ __launch_bounds__(PT) void plan_kernel(PlanArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  Shared &sh = *reinterpret_cast<Shared *>(smem_raw);
  float *srow = reinterpret_cast<float *>(smem_raw + ((sizeof(Shared) + 15) & ~(size_t)15));

  const int t = threadIdx.x;
  const size_t r = blockIdx.x;
  const int M = a.M, s = a.budget;
  const float *grow = a.scores + r * (size_t)M;
  const float *row = IN_LDS ? srow : grow;
  int32_t *out_idx = a.idx + r * (size_t)s;
  float *out_bias = a.bias ? a.bias + r * (size_t)s : nullptr;

  if (IN_LDS) {
    for (int j = t; j < M; j += PT) srow[j] = grow[j];
    __syncthreads();
  }
  const int chunk = (M + PT - 1) / PT;
  const int lo = min(M, t * chunk), hi = min(M, lo + chunk);

  // ---- phase 0: validity, positives, extremes, approximate total
  long long npos = 0, nbad = 0;
  unsigned mx = 0, mnpos = 0x7f800000u;
  double tot = 0.0;
  for (int j = lo; j < hi; ++j) {
    const float v = row[j];
    const unsigned b = __builtin_bit_cast(unsigned, v);
    if (!(v >= 0.f) || b >= 0x7f800000u) {
      ++nbad;
      continue;
    }
    if (b != 0u) {  // +0 only (-0 has the sign bit and is >= 0 but b != 0)
      if (b & 0x80000000u) continue;
      ++npos;
      mx = max(mx, b);
      mnpos = min(mnpos, b);
      tot += (double)v;
    }
  }
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
      for (int j = lo; j < hi; ++j) c += row[j] >= xm ? 1 : 0;
      c = block_sum_l(sh, c);
      if (c >= s) blo = mid; else bhi = mid;
    }
    const float v = __builtin_bit_cast(float, blo);
    // values are >= 0 here; -0 equals +0 and is treated as 0
    long long ngt = 0, ntie = 0;
    for (int j = lo; j < hi; ++j) {
      ngt += row[j] > v ? 1 : 0;
      ntie += row[j] == v ? 1 : 0;
    }
    ngt = block_sum_l(sh, ngt);
    const long long need = s - ngt;
    uint64_t tie_total;
    const uint64_t tie_base = block_exscan_u64(sh, (uint64_t)ntie, tie_total);
    long long nsel = 0;
    {
      uint64_t tr = tie_base;
      for (int j = lo; j < hi; ++j) {
        const float x = row[j];
        bool sel = x > v;
        if (x == v) {
          sel = (long long)tr < need;
          ++tr;
        }
        nsel += sel ? 1 : 0;
      }
    }
    uint64_t sel_total;
    uint64_t pos = block_exscan_u64(sh, (uint64_t)nsel, sel_total);
    {
      uint64_t tr = tie_base;
      for (int j = lo; j < hi; ++j) {
        const float x = row[j];
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
      }
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
    for (int j = lo; j < hi; ++j) mine += row[j] > 0.f ? 1 : 0;
    uint64_t pos = block_exscan_u64(sh, (uint64_t)mine, total);
    for (int j = lo; j < hi; ++j)
      if (row[j] > 0.f) {
        out_idx[pos] = j;
        if (out_bias) out_bias[pos] = 0.f;
        ++pos;
      }
    fill_rest((int)npos);
    if (t == 0) {
      a.count[r] = (int)npos;
      if (a.lambda) a.lambda[r] = __builtin_inf();
    }
    return;
  }

  // cond(x): (s - #{S >= x}) x <= sum_{S < x} S, decided with a certified
  // fp64 margin or, inside the margin, exactly.
  const double err_bound = ldexp((double)(M + 2 * PT), -50) * tot;
  auto cond = [&](float x) -> bool {
    long long nge = 0;
    double slt = 0.0;
    for (int j = lo; j < hi; ++j) {
      const float v = row[j];
      if (v >= x) ++nge;
      else slt += (double)v;
    }
    nge = block_sum_l(sh, nge);
    slt = block_sum_d(sh, slt);
    const long long mult = (long long)s - nge;
    if (mult <= 0) return true;
    const double lhs = (double)mult * (double)x;  // exact: < 2^21 times a 24-bit value
    const double diff = lhs - slt;
    if (diff > err_bound) return false;
    if (diff < -err_bound) return true;
    exact_sum(sh, row, lo, hi, x, true);
    uint64_t ldig[NDIG + 1];
    scaled_to_digits((unsigned long long)mult, x, ldig);
    return digits_ge(sh.total, ldig);
  };

  unsigned blo = mnpos, bhi = mx;
  float xstar;
  if (cond(__builtin_bit_cast(float, mx))) {
    xstar = __builtin_bit_cast(float, mx);  // no saturated block
  } else {
    // x > T/s can never satisfy cond: tighten the upper end when possible.
    const double up = tot / (double)s * (1.0 + 0x1p-20);
    const float upf = (float)up;
    if (upf < __builtin_bit_cast(float, mx)) {
      const unsigned ub = __builtin_bit_cast(unsigned, upf) + 1u;
      if (ub > blo && ub < bhi && !cond(__builtin_bit_cast(float, ub))) bhi = ub;
    }
    while (bhi - blo > 1) {
      const unsigned mid = blo + (bhi - blo) / 2;
      if (cond(__builtin_bit_cast(float, mid))) blo = mid; else bhi = mid;
    }
    xstar = __builtin_bit_cast(float, blo);
  }

  long long nsat = 0;
  for (int j = lo; j < hi; ++j) nsat += row[j] > xstar ? 1 : 0;
  nsat = block_sum_l(sh, nsat);
  exact_sum(sh, row, lo, hi, xstar, false);
  if (t == 0) sh.bcast_d = digits_to_double(sh.total);
  __syncthreads();
  const double Tr = sh.bcast_d;
  const double lam = (double)(s - nsat) / Tr;

  const uint64_t U = a.offsets ? a.offsets[r] : offset_of_row(a.seed, r);
  uint64_t mine = 0;
  for (int j = lo; j < hi; ++j) {
    const double pi = fmin(1.0, lam * (double)row[j]);
    mine += (uint64_t)(pi * (double)UNIT);
  }
  uint64_t csum_total;
  uint64_t C = block_exscan_u64(sh, mine, csum_total);
  auto below = [&](uint64_t c) -> uint64_t {  // points U + k 2^44 (k < s) below c
    if (c <= U) return 0;
    const uint64_t n = ((c - U - 1) >> 44) + 1;
    return n < (uint64_t)s ? n : (uint64_t)s;
  };
  for (int j = lo; j < hi; ++j) {
    const double pi = fmin(1.0, lam * (double)row[j]);
    const uint64_t Pi = (uint64_t)(pi * (double)UNIT);
    const uint64_t p0 = below(C), p1 = below(C + Pi);
    if (p1 > p0) {
      out_idx[p0] = j;
      if (out_bias) out_bias[p0] = (float)(-log(pi));
    }
    C += Pi;
  }
  const int drawn = (int)below(csum_total);
  fill_rest(drawn);
  if (t == 0) {
    a.count[r] = drawn;
    if (a.lambda) a.lambda[r] = lam;
  }
}

}  // namespace

int launch_sip_plan(const float *scores, int rows, int nqb, int M, int budget, int mode,
                    uint64_t seed, const uint64_t *offsets, int32_t *idx, float *bias,
                    int32_t *count, double *lambda, hipStream_t stream) {
  (void)nqb;
  PlanArgs a{scores, rows, M, budget, mode, seed, offsets, idx, bias, count, lambda};
  int dev = 0, max_lds = 65536;
  if (hipGetDevice(&dev) != hipSuccess) return BSA_ERR_HIP;
  if (hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
      hipSuccess)
    return BSA_ERR_HIP;
  const size_t base = (sizeof(Shared) + 15) & ~(size_t)15;
  const size_t with_row = base + (size_t)M * sizeof(float);
  if (with_row <= (size_t)max_lds) {
    hipLaunchKernelGGL(plan_kernel<true>, dim3(rows), dim3(PT), with_row, stream, a);
  } else {
    hipLaunchKernelGGL(plan_kernel<false>, dim3(rows), dim3(PT), base, stream, a);
  }
  return status_of(hipGetLastError());
}

}  // namespace bsa
