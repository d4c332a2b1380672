// Accuracy diagnostics of a sampling plan, for gfx950.
//
// AB-Attention page (onedev.kr/papers/1521): section "무엇과 다른가" compares
// the attention mass an oracle top-k keeps at different KV block sizes,
// section "어떻게 쓰나" compares SIP's attention error with an oracle
// top-k's.  These kernels measure both quantities on given activations:
//
//   * block_mass: the true attention mass of every KV block for every query
//     block, A_ij = mean over the block's queries n of
//     sum_{t in block j} exp(scale q_n . k_t - lse_n), with lse the dense
//     log-normaliser (the LSE output of a dense attention call).  One
//     workgroup covers one 128-query block and a chunk of at most 3584 keys
//     that starts on a KV-block boundary; wave w holds queries 32 w .. +32
//     as the A operand of S = Q K^T (bf16 MFMA 32x32x16) and every wave
//     reads the same 32-key K tiles from a three-slot LDS ring filled by
//     direct global->LDS loads (16-byte-chunk XOR swizzle, bank-conflict
//     free operand reads).  Each lane's accumulators hold one key of 16
//     queries, so a key's column sum over the wave's 32 queries is 15
//     in-lane adds and one swap with the other lane half.  The four waves'
//     sums of a tile are added per key (in wave order) one step later, into
//     the chunk's key sums in LDS, which are summed into blocks in key order
//     at the end: deterministic for any block size.
//   * plan_coverage: sum of A over the blocks a plan lists (fp64, list
//     order).
//   * output_error: sum (O - R)^2 and sum R^2 per head (fp64).
#include <type_traits>

#include "common.h"

namespace bsa {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kMassChunk = 3584;  // keys per workgroup, at most (LDS under 40 KB: 4 workgroups per CU)

// This wave's global->LDS loads older than the newest N vector-memory ops
// and its LDS accesses are complete, then a workgroup barrier.
template <int N>
__device__ __forceinline__ void ring_wait_barrier() {
  static_assert(N >= 0 && N < 16, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(N | (7 << 4) | (0 << 8));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Chunk swizzle of row r of a row-major K tile: 16 consecutive rows read at
// one chunk column land on 16 different chunks (256-byte rows), or 8 rows
// pair up (128-byte rows).
template <int D>
__device__ __forceinline__ int swz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}

struct MassArgs {
  const uint16_t *q, *k;
  const float *lse;
  float *mass;
  int Nq, Nk, nqb, M, kv_block, ck, nchunk, total_wg;
  float scale_log2;
};

template <int D>
__global__ __launch_bounds__(256, 2) void block_mass_kernel(MassArgs a) {
  constexpr int NW = 4;             // waves: one 32-query quarter each
  constexpr int KT = 32;            // keys per tile
  constexpr int NCH = D / 8;        // 16-byte chunks per row
  constexpr int ROWB = D * 2;       // row bytes
  constexpr int TILEB = KT * ROWB;  // bytes of one K tile
  constexpr int RPI = 64 / NCH;     // rows per 1 KB wave load
  constexpr int RPW = KT / NW;      // tile rows loaded by one wave
  constexpr int LPW = RPW / RPI;    // wave loads per tile
  constexpr int DS = D / 16;        // k-steps
  static_assert(LPW >= 1 && RPW % RPI == 0, "tile split");

  __shared__ __attribute__((aligned(16))) unsigned char k0[TILEB], k1[TILEB], k2[TILEB];
  __shared__ float colw[2][NW][KT];       // per-wave key sums of the last two tiles
  __shared__ float keysum[kMassChunk];    // key sums of the chunk

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  // XCD-aware order: each XCD gets a contiguous run of workgroups, i.e. of
  // query blocks of one key chunk, which then share its K tiles in L2.
  int wg = blockIdx.x;
  {
    const int per = 8 * 64;
    const int full = (a.total_wg / per) * per;
    if (wg < full) {
      const int r = wg / per, u = wg % per;
      wg = r * per + (u & 7) * 64 + (u >> 3);
    }
  }
  const int qb = wg % a.nqb;
  const int rest = wg / a.nqb;
  const int chunk = rest % a.nchunk;
  const int bh = rest / a.nchunk;
  const int key0 = chunk * a.ck;
  const int nk = min(a.ck, a.Nk - key0);
  const int ntiles = (nk + KT - 1) / KT;
  const int nrow = min(128, a.Nq - qb * 128);
  const uint16_t *qbase = a.q + (size_t)bh * a.Nq * D;
  const unsigned char *kbase = (const unsigned char *)(a.k + (size_t)bh * a.Nk * D);

  // Q fragments (A operand): query row 32 wave + l32, dims 16 ds + 8 hh ..
  const int qrow = qb * 128 + wave * 32 + l32;
  bf16x8 qf[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (qrow < a.Nq) v = ld16(qbase + (size_t)qrow * D + ds * 16 + hh * 8);
    qf[ds] = as_bf16x8(v);
  }
  // Base-2 normalisers of the queries of this lane's accumulator registers:
  // register r holds query 8 (r >> 2) + 4 hh + (r & 3) of the wave; rows
  // past Nq get +inf (probability 0).
  float nl[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = qb * 128 + wave * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
    nl[r] = row < a.Nq ? a.lse[(size_t)bh * a.Nq + row] * kLog2e : __builtin_inff();
  }

  // Loads: tile row r = RPW wave + RPI j + lane / NCH, stored chunk
  // lane % NCH holds source chunk (lane % NCH) ^ swz(r).  Rows past Nk
  // re-read row Nk - 1 (their sums are never stored).
  int g_off[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int r = wave * RPW + j * RPI + lane / NCH;
    g_off[j] = ((lane % NCH) ^ swz<D>(r)) << 4;
  }
  auto kslot = [&](auto c) -> unsigned char * {
    constexpr int S = decltype(c)::value;
    return S == 0 ? k0 : (S == 1 ? k1 : k2);
  };
  auto issue = [&](auto slot_c, int t) {
    unsigned char *kt = kslot(slot_c);
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int r = wave * RPW + j * RPI + lane / NCH;
      const int key = min(key0 + t * KT + r, a.Nk - 1);
      __builtin_amdgcn_global_load_lds((const void *)(kbase + (size_t)key * ROWB + g_off[j]),
                                       (lds_void *)(kt + (wave * RPW + j * RPI) * ROWB), 16, 0, 0);
    }
  };

  int koff[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) koff[ds] = l32 * ROWB + (((2 * ds + hh) ^ swz<D>(l32)) << 4);

  auto compute = [&](auto slot_c, int t) {
    const unsigned char *kt = kslot(slot_c);
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const bf16x8 kf = as_bf16x8(*(const u32x4 *)(kt + koff[ds]));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ds], kf, s, 0, 0, 0);
    }
    float col = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) col += __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.scale_log2, -nl[r]));
    col += xor32(col);  // both halves add the same two values
    if (hh == 0) colw[t & 1][wave][l32] = col;
  };
  // key sums of tile t (its four wave sums complete: called after a
  // barrier that every wave passed after computing tile t)
  auto fold = [&](int t) {
    const int key = t * KT + l32;
    if (wave == (t & 3) && hh == 0 && key < nk)
      keysum[key] = ((colw[t & 1][0][l32] + colw[t & 1][1][l32]) + colw[t & 1][2][l32]) + colw[t & 1][3][l32];
  };

  auto step = [&](auto slot_c, int t) {
    constexpr int S = decltype(slot_c)::value;
    if (t + 1 < ntiles) ring_wait_barrier<LPW>();
    else ring_wait_barrier<0>();
    if (t + 2 < ntiles) issue(std::integral_constant<int, (S + 2) % 3>(), t + 2);
    if (t > 0) fold(t - 1);
    compute(slot_c, t);
  };

  if (ntiles > 0) issue(std::integral_constant<int, 0>(), 0);
  if (ntiles > 1) issue(std::integral_constant<int, 1>(), 1);
  for (int t = 0; t < ntiles; t += 3) {
    step(std::integral_constant<int, 0>(), t);
    if (t + 1 < ntiles) step(std::integral_constant<int, 1>(), t + 1);
    if (t + 2 < ntiles) step(std::integral_constant<int, 2>(), t + 2);
  }
  __syncthreads();
  if (ntiles > 0) fold(ntiles - 1);
  __syncthreads();

  // Block sums in key order, each key's four wave sums in wave order; one
  // IEEE division by the query count.
  const int nb = (nk + a.kv_block - 1) / a.kv_block;
  float *orow = a.mass + ((size_t)bh * a.nqb + qb) * a.M + chunk * (a.ck / a.kv_block);
  for (int b = tid; b < nb; b += NW * 64) {
    const int t0 = b * a.kv_block, t1 = min(nk, t0 + a.kv_block);
    float acc = 0.f;
    for (int t = t0; t < t1; ++t) acc += keysum[t];
    orow[b] = acc / (float)nrow;
  }
}

__global__ __launch_bounds__(256) void plan_coverage_kernel(const float *mass, const int32_t *idx,
                                                            const int32_t *count, int rows, int M,
                                                            int L, double *cov) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  int c = count[r];
  c = c < 0 ? 0 : (c > L ? L : c);
  const int32_t *ir = idx + (size_t)r * L;
  const float *mr = mass + (size_t)r * M;
  double acc = 0.0;
  for (int e = 0; e < c; ++e) {
    const int j = ir[e];
    if (j >= 0 && j < M) acc += (double)mr[j];
  }
  cov[r] = acc;
}

// One workgroup per head: 16-byte loads of both tensors, fp64 sums per
// thread, then a fixed-order tree over the workgroup.
__global__ __launch_bounds__(1024) void output_error_kernel(const uint16_t *o, const uint16_t *ref,
                                                            long long n, double *sums) {
  __shared__ double sd[1024], sr[1024];
  const int tid = threadIdx.x;
  const uint16_t *ob = o + (size_t)blockIdx.x * n;
  const uint16_t *rb = ref + (size_t)blockIdx.x * n;
  double d2 = 0.0, r2 = 0.0;
  for (long long i = (long long)tid * 8; i < n; i += 1024 * 8) {
    const u32x4 x = ld16(ob + i), y = ld16(rb + i);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const double a = (double)__builtin_bit_cast(float, (x[w] >> (16 * h)) << 16);
        const double b = (double)__builtin_bit_cast(float, (y[w] >> (16 * h)) << 16);
        const double e = a - b;
        d2 += e * e;
        r2 += b * b;
      }
    }
  }
  sd[tid] = d2;
  sr[tid] = r2;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if (tid < s) {
      sd[tid] += sd[tid + s];
      sr[tid] += sr[tid + s];
    }
    __syncthreads();
  }
  if (tid == 0) {
    sums[2 * blockIdx.x] = sd[0];
    sums[2 * blockIdx.x + 1] = sr[0];
  }
}

}  // namespace

int mass_chunk_keys(int kv_block) { return kv_block * (kMassChunk / kv_block); }

int launch_block_mass(const void *q, const void *k, const float *lse, int B, int H, int Nq, int Nk,
                      int d, int kv_block, float scale, float *mass, hipStream_t stream) {
  clear_pending_error();
  MassArgs a;
  a.q = (const uint16_t *)q;
  a.k = (const uint16_t *)k;
  a.lse = lse;
  a.mass = mass;
  a.Nq = Nq;
  a.Nk = Nk;
  a.nqb = (Nq + 127) / 128;
  a.M = (Nk + kv_block - 1) / kv_block;
  a.kv_block = kv_block;
  a.ck = mass_chunk_keys(kv_block);
  a.nchunk = (Nk + a.ck - 1) / a.ck;
  a.scale_log2 = scale * kLog2e;
  const long long total = (long long)B * H * a.nqb * a.nchunk;
  a.total_wg = (int)total;
  dim3 grid((unsigned)total), block(256);
  if (d == 128) hipLaunchKernelGGL((block_mass_kernel<128>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((block_mass_kernel<64>), grid, block, 0, stream, a);
  return status_of(hipGetLastError());
}

int launch_plan_coverage(const float *mass, const int32_t *idx, const int32_t *count, int rows,
                         int M, int max_blocks, double *cov, hipStream_t stream) {
  clear_pending_error();
  dim3 grid((unsigned)((rows + 255) / 256)), block(256);
  hipLaunchKernelGGL(plan_coverage_kernel, grid, block, 0, stream, mass, idx, count, rows, M,
                     max_blocks, cov);
  return status_of(hipGetLastError());
}

int launch_output_error(const void *out, const void *ref, int slabs, long long n, double *sums,
                        hipStream_t stream) {
  clear_pending_error();
  dim3 grid((unsigned)slabs), block(1024);
  hipLaunchKernelGGL(output_error_kernel, grid, block, 0, stream, (const uint16_t *)out,
                     (const uint16_t *)ref, n, sums);
  return status_of(hipGetLastError());
}

}  // namespace bsa
