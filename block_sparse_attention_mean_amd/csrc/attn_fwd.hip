// Fused block-sparse attention forward for gfx950.
//
// AB-Attention page (onedev.kr/papers/1521), section "전제와 한계", first
// paragraph: the kernel gathers the sampled small KV blocks by index into
// full matrix-core tiles and performs the -log pi logit shift, the online
// softmax and the value accumulation in one pass, with no token reordering
// and no reordered copy of the sequence in memory.  The shift itself is the
// 1/pi weighting of section "어떻게 쓰나".
//
// Design (one workgroup = one 128-query block of one (b, h); 2 waves of 64
// queries each):
//   * Q stays in registers as the B operand of S^T = K Q^T (bf16 MFMA
//     32x32x16), so every lane owns one query column and the row max / row
//     sum need a single cross-half exchange;
//   * per 64-key tile the workgroup gathers the listed blocks into LDS:
//     K row-major [key][dim] and V transposed [dim][key], so both MFMA
//     operands are 16-byte LDS reads; the next tile's global loads are in
//     flight while the current tile computes;
//   * the K rows are fed to the MFMA in a permuted order chosen so that the
//     S^T accumulator registers of a lane hold 8 consecutive keys, which is
//     exactly the B-operand layout of O^T = V^T P^T -- P never leaves
//     registers;
//   * logits are moved to base 2 once (scale * log2 e, bias * log2 e) so
//     the softmax uses v_exp_f32 directly.
#include "common.h"

namespace bsa {

struct AttnArgs {
  const uint16_t *q, *k, *v;
  const int32_t *idx;
  const float *bias;
  const int32_t *count;
  uint16_t *out;
  float *lse;
  int Nq, Nk, nqb, max_blocks, kv_shift, M;
  int total_wg;
  float scale_log2;
};

// MFMA A-row -> key within a 32-key sub-tile (see the file comment).
__device__ __forceinline__ int key_of_row(int i) {
  return ((i >> 4) << 4) | (((i >> 2) & 1) << 3) | (((i >> 3) & 1) << 2) | (i & 3);
}

template <int D>
__global__ __launch_bounds__(128) void attn_fwd_kernel(AttnArgs a) {
  constexpr int KT = 64;            // keys per tile
  constexpr int NCH = D / 8;        // 16-byte chunks per row
  constexpr int KSTR = D + 8;       // K row stride (bf16 elements)
  constexpr int VSTR = KT + 8;      // V^T row stride
  constexpr int ITEMS = (KT / 4) * NCH;
  constexpr int IPT = ITEMS / 128;  // gather items per thread
  constexpr int DS = D / 16;        // k-steps of QK^T
  constexpr int DT = D / 32;        // dim tiles of O^T

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[KT * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D * VSTR];
  __shared__ __attribute__((aligned(16))) float bias_lds[KT];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  const int wg = blockIdx.x;
  const int qb = wg % a.nqb;
  const int bh = wg / a.nqb;
  const size_t row_id = (size_t)bh * a.nqb + qb;
  const uint16_t *qbase = a.q + (size_t)bh * a.Nq * D;
  const uint16_t *kbase = a.k + (size_t)bh * a.Nk * D;
  const uint16_t *vbase = a.v + (size_t)bh * a.Nk * D;
  const int32_t *idx_row = a.idx + row_id * a.max_blocks;
  const float *bias_row = a.bias ? a.bias + row_id * a.max_blocks : nullptr;
  int cnt = a.count[row_id];
  cnt = cnt < 0 ? 0 : (cnt > a.max_blocks ? a.max_blocks : cnt);
  const int kvb = 1 << a.kv_shift;
  const int nkeys = cnt << a.kv_shift;
  const int ntiles = (nkeys + KT - 1) / KT;

  // ---- Q fragments (B operand): lane holds query column l32, 8 dims.
  bf16x8 qf[2][DS];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int row = qb * 128 + wave * 64 + qs * 32 + l32;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < a.Nq) v = ld16(qbase + (size_t)row * D + ds * 16 + hh * 8);
      qf[qs][ds] = as_bf16x8(v);
    }
  }

  // ---- gather staging registers
  u32x4 kreg[IPT][4], vreg[IPT][4];
  float breg = 0.f;

  auto resolve = [&](int pos) -> int {
    if (pos >= nkeys) return -1;
    const int e = pos >> a.kv_shift;
    const int blk = idx_row[e];
    if (blk < 0 || blk >= a.M) return -1;
    const int key = (blk << a.kv_shift) + (pos & (kvb - 1));
    return key < a.Nk ? key : -1;
  };

  auto load_tile = [&](int t) {
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int item = tid + 128 * it;
      const int g = item / NCH, c = item % NCH;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int key = resolve(t * KT + 4 * g + kk);
        u32x4 zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
        if (key >= 0) {
          zk = ld16(kbase + (size_t)key * D + c * 8);
          zv = ld16(vbase + (size_t)key * D + c * 8);
        }
        kreg[it][kk] = zk;
        vreg[it][kk] = zv;
      }
    }
    if (tid < KT) {
      const int pos = t * KT + tid;
      const int key = resolve(pos);
      breg = key >= 0 ? (bias_row ? bias_row[pos >> a.kv_shift] * kLog2e : 0.f)
                      : -__builtin_inff();
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int item = tid + 128 * it;
      const int g = item / NCH, c = item % NCH;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) st16(&k_lds[(4 * g + kk) * KSTR + c * 8], kreg[it][kk]);
      // transpose 4 keys x 8 dims into V^T rows (4 consecutive keys per row)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const unsigned a0 = vreg[it][0][w], a1 = vreg[it][1][w];
        const unsigned a2 = vreg[it][2][w], a3 = vreg[it][3][w];
        u32x2 lo = {(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
        u32x2 hi = {(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
        *(u32x2 *)&vt_lds[(c * 8 + 2 * w) * VSTR + 4 * g] = lo;
        *(u32x2 *)&vt_lds[(c * 8 + 2 * w + 1) * VSTR + 4 * g] = hi;
      }
    }
    if (tid < KT) bias_lds[tid] = breg;
  };

  f32x16 oacc[2][DT];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qs][dt][r] = 0.f;
  float m_run[2] = {-__builtin_inff(), -__builtin_inff()};
  float l_run[2] = {0.f, 0.f};

  if (ntiles > 0) load_tile(0);

  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < ntiles) load_tile(t + 1);

    // ---- S^T = K Q^T for 2 key sub-tiles x 2 query sub-tiles
    f32x16 sacc[2][2];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[qs][ks][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int krow = ks * 32 + key_of_row(l32);
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const bf16x8 af = as_bf16x8(ld16(&k_lds[krow * KSTR + ds * 16 + hh * 8]));
        sacc[0][ks] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[0][ds], sacc[0][ks], 0, 0, 0);
        sacc[1][ks] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[1][ds], sacc[1][ks], 0, 0, 0);
      }
    }

    // ---- per-key base-2 shift of this lane's keys: 32 ks + 16 (r>>3) + 8 hh + (r&7)
    float bk[2][16];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2) {
        const f32x4 b0 = *(const f32x4 *)&bias_lds[ks * 32 + m2 * 16 + hh * 8];
        const f32x4 b1 = *(const f32x4 *)&bias_lds[ks * 32 + m2 * 16 + hh * 8 + 4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bk[ks][m2 * 8 + e] = b0[e];
          bk[ks][m2 * 8 + 4 + e] = b1[e];
        }
      }

    // ---- online softmax (base 2); P^T stays in registers
    bf16x8 pf[2][4];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float tv = __builtin_fmaf(sacc[qs][ks][r], a.scale_log2, bk[ks][r]);
          sacc[qs][ks][r] = tv;
          mx = fmaxf(mx, tv);
        }
      mx = fmaxf(mx, xor32(mx));
      const float m_new = fmaxf(m_run[qs], mx);
      const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[qs] - m_use);
      m_run[qs] = m_new;
      float rs = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(sacc[qs][ks][r] - m_use);
          sacc[qs][ks][r] = pv;
          rs += pv;
        }
      l_run[qs] = l_run[qs] * alpha + rs;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[qs][dt][r] *= alpha;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int ks = m >> 1, r0 = 8 * (m & 1);
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = pack_bf16x2(sacc[qs][ks][r0 + 2 * e], sacc[qs][ks][r0 + 2 * e + 1]);
        pf[qs][m] = as_bf16x8(w);
      }
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const bf16x8 af = as_bf16x8(ld16(&vt_lds[(dt * 32 + l32) * VSTR + m * 16 + hh * 8]));
        oacc[0][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, pf[0][m], oacc[0][dt], 0, 0, 0);
        oacc[1][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, pf[1][m], oacc[1][dt], 0, 0, 0);
      }
  }

  // ---- normalise and store
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const float l = l_run[qs] + xor32(l_run[qs]);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int row = qb * 128 + wave * 64 + qs * 32 + l32;
    if (row < a.Nq) {
      uint16_t *orow = a.out + ((size_t)bh * a.Nq + row) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 w = {pack_bf16x2(oacc[qs][dt][4 * g] * inv, oacc[qs][dt][4 * g + 1] * inv),
                     pack_bf16x2(oacc[qs][dt][4 * g + 2] * inv, oacc[qs][dt][4 * g + 3] * inv)};
          *(u32x2 *)&orow[dt * 32 + g * 8 + hh * 4] = w;
        }
      if (a.lse && hh == 0)
        a.lse[(size_t)bh * a.Nq + row] =
            l > 0.f ? (m_run[qs] + __builtin_log2f(l)) * kLn2 : -__builtin_inff();
    }
  }
}

int launch_attn_fwd(const void *q, const void *k, const void *v, int B, int H, int Nq, int Nk,
                    int d, int kv_block, const int32_t *idx, const float *bias,
                    const int32_t *count, int max_blocks, float scale, void *out, float *lse,
                    hipStream_t stream) {
  AttnArgs a;
  a.q = (const uint16_t *)q;
  a.k = (const uint16_t *)k;
  a.v = (const uint16_t *)v;
  a.idx = idx;
  a.bias = bias;
  a.count = count;
  a.out = (uint16_t *)out;
  a.lse = lse;
  a.Nq = Nq;
  a.Nk = Nk;
  a.nqb = (Nq + 127) / 128;
  a.max_blocks = max_blocks;
  a.kv_shift = __builtin_ctz((unsigned)kv_block);
  a.M = (Nk + kv_block - 1) / kv_block;
  a.scale_log2 = scale * kLog2e;
  const long long total = (long long)B * H * a.nqb;
  a.total_wg = (int)total;
  dim3 grid((unsigned)total), block(128);
  if (d == 128)
    hipLaunchKernelGGL(attn_fwd_kernel<128>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<64>, grid, block, 0, stream, a);
  return status_of(hipGetLastError());
}

}  // namespace bsa
