// Backward pass of the fused block-sparse attention, for gfx950.
//
// AB-Attention page (onedev.kr/papers/1521): the forward pass gathers the
// listed small KV blocks and runs softmax attention with each block's
// logits shifted by -log pi (sections "어떻게 쓰나" and "전제와 한계"); the
// page names a trainable version, with a backward pass, as future work in
// its closing paragraph.  With the plan and its shifts held fixed, for
// query n and gathered key t: P = softmax(scale q.k + shift), D_n =
// dO_n . O_n, dS = P (dO_n . v_t - D_n); dQ = scale dS K, dK += scale dS^T Q
// and dV += P^T dO over every listed occurrence.  P comes from the
// forward's log-sum-exp, so no online softmax is needed.
//
// Two kernels, both one workgroup per 128-query block (4 waves):
//   * dq: wave w owns queries 32 w .. +32.  The listed blocks are gathered
//     into a three-slot LDS ring of 32-key K and V tiles as in the forward
//     pass, and per tile S^T = K Q^T, dP^T = V dO^T (Q and dO stay in
//     registers) and dQ^T += K^T dS^T (K^T through the transposing LDS
//     read).  K and V use one 16-byte-chunk swizzle that keeps both the row
//     reads and the transposing reads free of bank conflicts.
//   * dkdv: wave w owns 32 of every 128 gathered keys and all 128 queries,
//     so the keys' dK and dV are complete in its registers after one pass
//     over the query block: S = Q K^T and dP = dO V^T with Q and dO rows
//     from LDS and the wave's K and V rows loaded straight into registers,
//     then dV += P^T dO and dK += dS^T Q with dO and Q through the
//     transposing read.  Each key's rows are then added into fp32 dK and dV
//     in global memory (atomic adds: a key is listed by many query blocks).
// Outputs are fp32: dQ is written, dK and dV are zeroed by the entry point
// first.  Head dims 64 and 128.
#include <type_traits>

#include "common.h"

namespace bsa {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int CAP = 512;       // list entries staged per phase

// Chunk swizzle of row r: 16 consecutive rows read at one chunk, and 4
// consecutive rows (the first a multiple of 4) read at 4 consecutive chunks
// (the first a multiple of 4), both hit 16 different 16-byte bank slots --
// the row-read and the transposing-read patterns.  256-byte rows (d = 128)
// fill the 64 banks; 128-byte rows (d = 64) pair up, so there bit 2 of the
// chunk separates rows 2m and 2m + 2.
template <int D>
__device__ __forceinline__ int swz(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// MFMA A-row -> key within a 32-key tile, chosen so that accumulator
// register r of lane half h holds key 16 (r >> 3) + 8 h + (r & 7): S^T's
// registers are then directly the B operand of products over keys.
__device__ __forceinline__ int key_of_row(int i) {
  return ((i >> 4) << 4) | (((i >> 2) & 1) << 3) | (((i >> 3) & 1) << 2) | (i & 3);
}

// Byte offset, inside a swizzled row-major tile, of this lane's 8-byte part
// of a transposing read that yields, for the lane's dim 32 dt + (lane % 32),
// the four rows base + 0..3 (base depends only on the lane's half): lanes of
// a 16-lane group read row base + (i >> 2) at columns 4 (i & 3) .. +3 of
// their group's 16 columns.
template <int D>
__device__ __forceinline__ int tr_off(int base, int dt, int lane) {
  const int gi = lane & 15, gg = lane >> 4;
  const int r = base + (gi >> 2);
  const int n0 = dt * 32 + 16 * (gg & 1) + 4 * (gi & 3);
  return r * (D * 2) + (((n0 >> 3) ^ swz<D>(r)) << 4) + ((n0 >> 2) & 1) * 8;
}

template <int N>
__device__ __forceinline__ void ring_barrier() {
  static_assert(N >= 0 && N < 16, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(N | (7 << 4) | (0 << 8));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ bf16x8 tr_pair(const unsigned char *base, int off0, int off1) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base + off0));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base + off1));
  const u32x2 w0 = __builtin_bit_cast(u32x2, a), w1 = __builtin_bit_cast(u32x2, b);
  const u32x4 w = {w0[0], w0[1], w1[0], w1[1]};
  return as_bf16x8(w);
}

// fp32 sum of dO . O over this lane's half of the dims of its query row
// (the dims of the B/A operand fragments: 16 ds + 8 hh + 0..7), plus the
// other half.
template <int D>
__device__ __forceinline__ float row_dot(const uint16_t *o_row, const uint16_t *do_row, int hh,
                                         bool valid) {
  float part = 0.f;
  if (valid) {
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      const u32x4 x = ld16(o_row + ds * 16 + hh * 8), y = ld16(do_row + ds * 16 + hh * 8);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        part += __builtin_bit_cast(float, x[w] << 16) * __builtin_bit_cast(float, y[w] << 16);
        part += __builtin_bit_cast(float, x[w] & 0xffff0000u) *
                __builtin_bit_cast(float, y[w] & 0xffff0000u);
      }
    }
  }
  return part + xor32(part);
}

}  // namespace

struct BwdArgs {
  const uint16_t *q, *k, *v, *o, *dout;
  const float *lse;
  const int32_t *idx;
  const float *bias;
  const int32_t *count;
  float *dq, *dk, *dv;
  int Nq, Nk, nqb, max_blocks, kv_shift, M;
  int total_wg;
  float scale, scale_log2;
};

namespace {

__device__ __forceinline__ int xcd_order(int wg, int total) {
  const int per = 8 * 64;
  const int full = (total / per) * per;
  if (wg < full) {
    const int r = wg / per, u = wg % per;
    wg = r * per + (u & 7) * 64 + (u >> 3);
  }
  return wg;
}

// Stage list entries [base, base + n) of the row into LDS: block index
// (invalid -> 0) and base-2 shift (invalid -> -inf); entries past the
// phase up to `padded` are invalid.
__device__ __forceinline__ void stage_list(const BwdArgs &a, const int32_t *idx_row,
                                           const float *bias_row, int base, int pc, int padded,
                                           int32_t *idx_s, float *sh_s, int tid) {
  for (int e = tid; e < padded; e += 256) {
    int blk = e < pc ? idx_row[base + e] : -1;
    float sh = (e < pc && bias_row) ? bias_row[base + e] * kLog2e : 0.f;
    if (blk < 0 || blk >= a.M) {
      blk = 0;
      sh = -__builtin_inff();
    }
    idx_s[e] = blk;
    sh_s[e] = sh;
  }
}

template <int D>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(BwdArgs a) {
  constexpr int ROWB = D * 2;        // row bytes
  constexpr int NCH = D / 8;         // 16-byte chunks per row
  constexpr int DS = D / 16;         // k-steps over the head dim
  constexpr int DT = D / 32;         // 32-wide dim tiles
  constexpr int NW = 4, KT = 32, NBUF = 3;
  constexpr int TILEB = KT * ROWB;
  constexpr int RPI = 64 / NCH;      // rows per 1 KB wave load
  constexpr int RPW = KT / NW;       // tile rows loaded by one wave
  constexpr int LPW = RPW / RPI;     // wave loads per operand per tile
  constexpr int LPT = 2 * LPW;       // vector-memory ops per wave per tile

  __shared__ __attribute__((aligned(16))) unsigned char k0[TILEB], v0[TILEB];
  __shared__ __attribute__((aligned(16))) unsigned char k1[TILEB], v1[TILEB];
  __shared__ __attribute__((aligned(16))) unsigned char k2[TILEB], v2[TILEB];
  __shared__ __attribute__((aligned(16))) int32_t idx_s[CAP];
  __shared__ __attribute__((aligned(16))) float sh_s[CAP];
  __shared__ __attribute__((aligned(16))) float bring[NBUF * KT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int wg = xcd_order(blockIdx.x, a.total_wg);
  const int qb = wg % a.nqb;
  const int bh = wg / a.nqb;
  const size_t row_id = (size_t)bh * a.nqb + qb;
  const unsigned char *kbase = (const unsigned char *)(a.k + (size_t)bh * a.Nk * D);
  const unsigned char *vbase = (const unsigned char *)(a.v + (size_t)bh * a.Nk * D);
  const int32_t *idx_row = a.idx + row_id * a.max_blocks;
  const float *bias_row = a.bias ? a.bias + row_id * a.max_blocks : nullptr;
  int cnt = a.count[row_id];
  cnt = cnt < 0 ? 0 : (cnt > a.max_blocks ? a.max_blocks : cnt);
  const int kvb = 1 << a.kv_shift;

  // Q and dO (B operands, query column l32, dims 16 ds + 8 hh ..), D and
  // the base-2 normaliser of this lane's query.
  const int qrow = qb * 128 + wave * 32 + l32;
  const bool qok = qrow < a.Nq;
  const size_t qoff = ((size_t)bh * a.Nq + (qok ? qrow : 0)) * D;
  bf16x8 qf[DS], df[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (qok) {
      x = ld16(a.q + qoff + ds * 16 + hh * 8);
      y = ld16(a.dout + qoff + ds * 16 + hh * 8);
    }
    qf[ds] = as_bf16x8(x);
    df[ds] = as_bf16x8(y);
  }
  const float Dq = row_dot<D>(a.o + qoff, a.dout + qoff, hh, qok);
  float Lq = __builtin_inff();
  if (qok) {
    const float l = a.lse[(size_t)bh * a.Nq + qrow];
    if (l > -__builtin_inff()) Lq = l * kLog2e;
  }

  f32x16 dqacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[dt][r] = 0.f;

  // gather: tile row r = RPW wave + RPI j + lane / NCH; stored chunk
  // lane % NCH holds source chunk (lane % NCH) ^ swz(r)
  int g_row[LPW], g_off[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int r = wave * RPW + j * RPI + lane / NCH;
    g_row[j] = r;
    g_off[j] = ((lane % NCH) ^ swz<D>(r)) << 4;
  }
  auto kslot = [&](auto c) -> unsigned char * {
    constexpr int S = decltype(c)::value;
    return S == 0 ? k0 : (S == 1 ? k1 : k2);
  };
  auto vslot = [&](auto c) -> unsigned char * {
    constexpr int S = decltype(c)::value;
    return S == 0 ? v0 : (S == 1 ? v1 : v2);
  };
  auto issue = [&](auto slot_c, int t) {
    constexpr int S = decltype(slot_c)::value;
    unsigned char *kt = kslot(slot_c);
    unsigned char *vt = vslot(slot_c);
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int pos = t * KT + g_row[j];
      const int e = pos >> a.kv_shift;
      const int kk = (idx_s[e] << a.kv_shift) + (pos & (kvb - 1));
      const bool ok = kk < a.Nk;
      const size_t src = (size_t)(ok ? kk : 0) * ROWB;
      const int dst = (wave * RPW + j * RPI) * ROWB;
      __builtin_amdgcn_global_load_lds((const void *)(kbase + src + g_off[j]), (lds_void *)(kt + dst), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void *)(vbase + src + g_off[j]), (lds_void *)(vt + dst), 16, 0, 0);
      if (lane % NCH == 0) bring[S * KT + g_row[j]] = ok ? sh_s[e] : -__builtin_inff();
    }
  };

  const int krow = key_of_row(l32);
  int koff[DS], toff[DT][2];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) koff[ds] = krow * ROWB + (((2 * ds + hh) ^ swz<D>(krow)) << 4);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int p = 0; p < 2; ++p) toff[dt][p] = tr_off<D>(8 * hh + 4 * p, dt, lane);

  auto compute = [&](auto slot_c) {
    constexpr int S = decltype(slot_c)::value;
    const unsigned char *kt = kslot(slot_c);
    const unsigned char *vt = vslot(slot_c);
    f32x16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = 0.f;
      dp[r] = 0.f;
    }
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      asm volatile("" : "+v"(koff[ds]));
      const bf16x8 kf = as_bf16x8(*(const u32x4 *)(kt + koff[ds]));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ds], s, 0, 0, 0);
      const bf16x8 vf = as_bf16x8(*(const u32x4 *)(vt + koff[ds]));
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, df[ds], dp, 0, 0, 0);
    }
    // register r of half hh <-> key 16 (r >> 3) + 8 hh + (r & 7)
    const float *bt = bring + S * KT;
    bf16x8 dsf[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const f32x4 b0 = *(const f32x4 *)&bt[m * 16 + hh * 8];
      const f32x4 b1 = *(const f32x4 *)&bt[m * 16 + hh * 8 + 4];
      float g[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * m + e;
        const float sh = e < 4 ? b0[e] : b1[e - 4];
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.scale_log2, sh - Lq));
        g[e] = p * (dp[r] - Dq);
      }
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(g[2 * e], g[2 * e + 1]);
      dsf[m] = as_bf16x8(w);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      asm volatile("" : "+v"(toff[dt][0]), "+v"(toff[dt][1]));
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const bf16x8 kT = tr_pair(kt + 16 * m * ROWB, toff[dt][0], toff[dt][1]);
        dqacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kT, dsf[m], dqacc[dt], 0, 0, 0);
      }
    }
  };

  int ntiles = 0;
  auto step = [&](auto slot_c, int t) {
    constexpr int S = decltype(slot_c)::value;
    if (t + 1 < ntiles) ring_barrier<LPT>();
    else ring_barrier<0>();
    if (t + 2 < ntiles) issue(std::integral_constant<int, (S + 2) % NBUF>(), t + 2);
    compute(slot_c);
  };

  for (int base = 0; base < cnt; base += CAP) {
    const int pc = min(CAP, cnt - base);
    ntiles = ((pc << a.kv_shift) + KT - 1) / KT;
    __syncthreads();
    stage_list(a, idx_row, bias_row, base, pc, min(CAP, ((ntiles * KT) >> a.kv_shift) + 1), idx_s,
               sh_s, tid);
    __syncthreads();
    if (ntiles > 0) issue(std::integral_constant<int, 0>(), 0);
    if (ntiles > 1) issue(std::integral_constant<int, 1>(), 1);
    for (int t = 0; t < ntiles; t += 3) {
      step(std::integral_constant<int, 0>(), t);
      if (t + 1 < ntiles) step(std::integral_constant<int, 1>(), t + 1);
      if (t + 2 < ntiles) step(std::integral_constant<int, 2>(), t + 2);
    }
  }

  // dQ = scale dQ^T: lane holds query l32, dims 32 dt + 8 g + 4 hh + 0..3
  if (qok) {
    float *out = a.dq + ((size_t)bh * a.Nq + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 w = {dqacc[dt][4 * g] * a.scale, dqacc[dt][4 * g + 1] * a.scale,
                   dqacc[dt][4 * g + 2] * a.scale, dqacc[dt][4 * g + 3] * a.scale};
        *(f32x4 *)&out[dt * 32 + g * 8 + hh * 4] = w;
      }
  }
}

template <int D>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv_kernel(BwdArgs a) {
  constexpr int ROWB = D * 2;        // row bytes
  constexpr int NCH = D / 8;         // 16-byte chunks per row
  constexpr int DS = D / 16;         // k-steps over the head dim
  constexpr int DT = D / 32;         // 32-wide dim tiles
  constexpr int NW = 4;
  constexpr int KT = 128;            // gathered keys per pass (32 per wave)
  constexpr int QTB = 128 * ROWB;    // bytes of the Q (or dO) block

  __shared__ __attribute__((aligned(16))) unsigned char q_s[QTB], do_s[QTB];
  __shared__ __attribute__((aligned(16))) int32_t idx_s[CAP];
  __shared__ __attribute__((aligned(16))) float sh_s[CAP];
  __shared__ __attribute__((aligned(16))) float dq_s[128], lq_s[128];
  __shared__ __attribute__((aligned(16))) int32_t keyrow_s[NW][32];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int wg = xcd_order(blockIdx.x, a.total_wg);
  const int qb = wg % a.nqb;
  const int bh = wg / a.nqb;
  const size_t row_id = (size_t)bh * a.nqb + qb;
  const int32_t *idx_row = a.idx + row_id * a.max_blocks;
  const float *bias_row = a.bias ? a.bias + row_id * a.max_blocks : nullptr;
  int cnt = a.count[row_id];
  cnt = cnt < 0 ? 0 : (cnt > a.max_blocks ? a.max_blocks : cnt);
  const int kvb = 1 << a.kv_shift;
  const int nrow = min(128, a.Nq - qb * 128);

  // Q and dO of the block into LDS (swizzled; rows past Nq are zero)
  {
    const uint16_t *qg = a.q + ((size_t)bh * a.Nq + (size_t)qb * 128) * D;
    const uint16_t *dg = a.dout + ((size_t)bh * a.Nq + (size_t)qb * 128) * D;
#pragma unroll
    for (int i = 0; i < 128 * NCH / 256; ++i) {
      const int c = i * 256 + tid;
      const int r = c / NCH, ch = c % NCH;
      u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
      if (r < nrow) {
        x = ld16(qg + (size_t)r * D + ch * 8);
        y = ld16(dg + (size_t)r * D + ch * 8);
      }
      const int off = r * ROWB + ((ch ^ swz<D>(r)) << 4);
      st16(q_s + off, x);
      st16(do_s + off, y);
    }
    // D and the base-2 normaliser per query (two lanes per query)
    const int qr = tid >> 1, half = tid & 1;
    float part = 0.f;
    if (qr < nrow) {
      const size_t off = ((size_t)bh * a.Nq + (size_t)qb * 128 + qr) * D + half * (D / 2);
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const u32x4 x = ld16(a.o + off + c * 8), y = ld16(a.dout + off + c * 8);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          part += __builtin_bit_cast(float, x[w] << 16) * __builtin_bit_cast(float, y[w] << 16);
          part += __builtin_bit_cast(float, x[w] & 0xffff0000u) *
                  __builtin_bit_cast(float, y[w] & 0xffff0000u);
        }
      }
    }
    part += __shfl_xor(part, 1, 64);
    if (half == 0) {
      dq_s[qr] = part;
      float L = __builtin_inff();
      if (qr < nrow) {
        const float l = a.lse[(size_t)bh * a.Nq + (size_t)qb * 128 + qr];
        if (l > -__builtin_inff()) L = l * kLog2e;
      }
      lq_s[qr] = L;
    }
  }

  // per-lane LDS offsets: rows of Q/dO (A operands, query row l32 of
  // sub-tile qs, dims 16 ds + 8 hh ..) and transposing reads (B operands,
  // dim 32 dt + l32, queries 32 qs + 16 ks + 8 p + 4 hh + 0..3)
  int roff[DS], toff[DT][2][2];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) roff[ds] = l32 * ROWB + (((2 * ds + hh) ^ swz<D>(l32)) << 4);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int p = 0; p < 2; ++p) toff[dt][ks][p] = tr_off<D>(16 * ks + 8 * p + 4 * hh, dt, lane);

  const uint16_t *kbase = a.k + (size_t)bh * a.Nk * D;
  const uint16_t *vbase = a.v + (size_t)bh * a.Nk * D;

  for (int base = 0; base < cnt; base += CAP) {
    const int pc = min(CAP, cnt - base);
    const int ntiles = ((pc << a.kv_shift) + KT - 1) / KT;
    __syncthreads();
    stage_list(a, idx_row, bias_row, base, pc, min(CAP, ((ntiles * KT) >> a.kv_shift) + 1), idx_s,
               sh_s, tid);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      // this wave's key (lane column l32) of the pass
      const int pos = t * KT + wave * 32 + l32;
      const int e = pos >> a.kv_shift;
      const int kk = (idx_s[e] << a.kv_shift) + (pos & (kvb - 1));
      const float shv = sh_s[e];
      const bool ok = kk < a.Nk && shv > -__builtin_inff();
      const float sh = ok ? shv : -__builtin_inff();
      if (hh == 0) keyrow_s[wave][l32] = ok ? kk : -1;
      const uint16_t *krp = kbase + (size_t)(ok ? kk : 0) * D;
      const uint16_t *vrp = vbase + (size_t)(ok ? kk : 0) * D;
      bf16x8 kf[DS], vf[DS];
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        kf[ds] = as_bf16x8(ld16(krp + ds * 16 + hh * 8));
        vf[ds] = as_bf16x8(ld16(vrp + ds * 16 + hh * 8));
      }
      f32x16 dkacc[DT], dvacc[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          dkacc[dt][r] = 0.f;
          dvacc[dt][r] = 0.f;
        }
#pragma unroll
      for (int qs = 0; qs < 4; ++qs) {
        const unsigned char *qt = q_s + qs * 32 * ROWB;
        const unsigned char *dt_ = do_s + qs * 32 * ROWB;
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[r] = 0.f;
          dp[r] = 0.f;
        }
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          const bf16x8 qa = as_bf16x8(*(const u32x4 *)(qt + roff[ds]));
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ds], s, 0, 0, 0);
          const bf16x8 da = as_bf16x8(*(const u32x4 *)(dt_ + roff[ds]));
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vf[ds], dp, 0, 0, 0);
        }
        // register r <-> query 32 qs + 8 (r >> 2) + 4 hh + (r & 3)
        bf16x8 pa[2], ga[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          float pv[8], gv[8];
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const int q0 = qs * 32 + 16 * ks + 8 * hf + 4 * hh;
            const f32x4 L = *(const f32x4 *)&lq_s[q0];
            const f32x4 Dv = *(const f32x4 *)&dq_s[q0];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int r = 8 * ks + 4 * hf + j;
              const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.scale_log2, sh - L[j]));
              pv[4 * hf + j] = p;
              gv[4 * hf + j] = p * (dp[r] - Dv[j]);
            }
          }
          u32x4 wp, wg2;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            wp[e2] = pack_bf16x2(pv[2 * e2], pv[2 * e2 + 1]);
            wg2[e2] = pack_bf16x2(gv[2 * e2], gv[2 * e2 + 1]);
          }
          pa[ks] = as_bf16x8(wp);
          ga[ks] = as_bf16x8(wg2);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const bf16x8 dob = tr_pair(dt_, toff[dt][ks][0], toff[dt][ks][1]);
            dvacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[ks], dob, dvacc[dt], 0, 0, 0);
            const bf16x8 qbm = tr_pair(qt, toff[dt][ks][0], toff[dt][ks][1]);
            dkacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[ks], qbm, dkacc[dt], 0, 0, 0);
          }
        }
      }
      // add the 32 keys' rows: register r <-> key 8 (r >> 2) + 4 hh + (r & 3)
      // of the wave, lane <-> dim 32 dt + l32
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int4 kr = *(const int4 *)&keyrow_s[wave][8 * g + 4 * hh];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = j == 0 ? kr.x : (j == 1 ? kr.y : (j == 2 ? kr.z : kr.w));
          if (row >= 0) {
            float *dkp = a.dk + ((size_t)bh * a.Nk + row) * D + l32;
            float *dvp = a.dv + ((size_t)bh * a.Nk + row) * D + l32;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
              unsafeAtomicAdd(dkp + dt * 32, dkacc[dt][4 * g + j] * a.scale);
              unsafeAtomicAdd(dvp + dt * 32, dvacc[dt][4 * g + j]);
            }
          }
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void zero_kernel(f32x4 *p, size_t n4) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) p[i] = z;
}

}  // namespace

int launch_attn_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
                    const float *lse, int B, int H, int Nq, int Nk, int d, int kv_block,
                    const int32_t *idx, const float *bias, const int32_t *count, int max_blocks,
                    float scale, float *dq, float *dk, float *dv, hipStream_t stream) {
  BwdArgs a;
  a.q = (const uint16_t *)q;
  a.k = (const uint16_t *)k;
  a.v = (const uint16_t *)v;
  a.o = (const uint16_t *)o;
  a.dout = (const uint16_t *)dout;
  a.lse = lse;
  a.idx = idx;
  a.bias = bias;
  a.count = count;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.Nq = Nq;
  a.Nk = Nk;
  a.nqb = (Nq + 127) / 128;
  a.max_blocks = max_blocks;
  a.kv_shift = __builtin_ctz((unsigned)kv_block);
  a.M = (Nk + kv_block - 1) / kv_block;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  const long long total = (long long)B * H * a.nqb;
  a.total_wg = (int)total;
  const size_t n4 = (size_t)B * H * Nk * d / 4;
  const unsigned zg = (unsigned)min((size_t)8192, (n4 + 255) / 256);
  hipLaunchKernelGGL(zero_kernel, dim3(zg), dim3(256), 0, stream, (f32x4 *)dk, n4);
  hipLaunchKernelGGL(zero_kernel, dim3(zg), dim3(256), 0, stream, (f32x4 *)dv, n4);
  if (d == 128) {
    hipLaunchKernelGGL((attn_bwd_dq_kernel<128>), dim3((unsigned)total), dim3(256), 0, stream, a);
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<128>), dim3((unsigned)total), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((attn_bwd_dq_kernel<64>), dim3((unsigned)total), dim3(256), 0, stream, a);
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<64>), dim3((unsigned)total), dim3(256), 0, stream, a);
  }
  return status_of(hipGetLastError());
}

}  // namespace bsa
