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
// Two kernels, one workgroup (4 waves) per 128-query block (the dkdv
// kernel of the workspace variant: per pair of query blocks):
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
//     in global memory (atomic adds: a key is listed by many query blocks),
//     or, in the workspace variant, stored as its union entry's partial rows.
// Outputs are fp32: dQ is written; the atomic form zeroes dK and dV first,
// the workspace form writes every row of them.  Head dims 64 and 128.
//
// Workspace variant.  A fp32 atomic add runs at a fixed rate of about one
// dword per clock per L2 channel, whatever the locality, and at the 720p
// shape the adds (one per key value per listing query block) take most of
// the backward's time.  The variant removes them: per chunk of (b, h)
// slabs that fits the caller's workspace,
//   * query blocks 2m and 2m + 1 form a pair, and the union of their lists
//     is built, grouped into blocks both list, the first only and the
//     second only (each padded to whole 128-key passes); neighbouring query
//     blocks share a large part of their lists, so the union is shorter
//     than the two lists;
//   * a key-major copy of the union lists is built: per KV block, the
//     (pair, union entry) slots that list it (count with integer atomics,
//     an exclusive scan per slab, a fill through per-block cursors, then
//     each block's slots sorted);
//   * the dkdv pair kernel runs each union entry's keys against the queries
//     of the blocks that list it and stores its dK (unscaled) and dV rows
//     with plain stores into the entry's own slot, a pass's rows during the
//     next pass (two sets of accumulators), so the stores spread over the
//     products instead of ending each pass in a burst;
//   * one wave per KV block sums its slots' partial rows in fp32 and
//     writes dK (times the softmax scale) and dV, zero for a block no
//     query block lists.
// The fill runs in whatever order its integer atomics take, so each block's
// slots are sorted before the sums: the workspace form gives the same bits
// on every run, for any number of slabs per pass (the atomic form does not).
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
  // workspace variant: slabs bh0 .. bh0 + nslab of this chunk, their
  // partial rows, and the key-major lists (per slab: kstart and kcur of
  // Ms ints, ent of cap ints)
  int bh0, nslab, Ms, cap;
  float *part;
  int32_t *kstart, *kcur, *ent, *ents;  // ents: each block's slots in ascending order
  // pairs of query blocks per slab, union entries per pair, and the union
  // lists: block (-1 = empty), the two base-2 shifts (float2), class ends
  int npairs, ucap;
  int32_t *ublk;
  float *ush;
  int32_t *ucls;
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
  // while tile t + 2 exists: the same step without conditions, under the
  // backend's hint to interleave LDS reads and matrix operations (at the
  // Wan2.1-14B 720p shape, interleaved on one box, the whole workspace
  // backward 110.2 against 110.9 ms, dQ unchanged bit for bit)
  auto step_full = [&](auto slot_c, int t) {
    constexpr int S = decltype(slot_c)::value;
    __builtin_amdgcn_iglp_opt(0);
    ring_barrier<LPT>();
    issue(std::integral_constant<int, (S + 2) % NBUF>(), t + 2);
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
    int t = 0;
    for (; t + 4 < ntiles; t += 3) {
      step_full(std::integral_constant<int, 0>(), t);
      step_full(std::integral_constant<int, 1>(), t + 1);
      step_full(std::integral_constant<int, 2>(), t + 2);
    }
    for (; t < ntiles; t += 3) {
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

// One query sub-step (32 queries) of a dkdv pass: S = Q K^T and dP = dO V^T,
// then P and dS, then dV += P^T dO and dK += dS^T Q.  qt / dt_ point at the
// sub-step's 32 rows of the swizzled Q and dO blocks in LDS, lq / dd at its
// 32 base-2 normalisers and D values; kf / vf hold the lane's key and value
// row (B operands), sh its base-2 shift.  rbo / tbo are the lane's row and
// transposing-read offset bases (see the kernels).
template <int D>
__device__ __forceinline__ void dkdv_substep(const unsigned char *qt, const unsigned char *dt_,
                                             const float *lq, const float *dd, int &rbo, int &tbo,
                                             int hh, const bf16x8 *kf, const bf16x8 *vf, float sh,
                                             float scale_log2, f32x16 *dkacc, f32x16 *dvacc) {
  constexpr int ROWB = D * 2;
  constexpr int DS = D / 16;
  constexpr int DT = D / 32;
  asm volatile("" : "+v"(rbo), "+v"(tbo));
  f32x16 s, dp;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s[r] = 0.f;
    dp[r] = 0.f;
  }
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    const bf16x8 qa = as_bf16x8(*(const u32x4 *)(qt + (rbo ^ (32 * ds))));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ds], s, 0, 0, 0);
    const bf16x8 da = as_bf16x8(*(const u32x4 *)(dt_ + (rbo ^ (32 * ds))));
    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vf[ds], dp, 0, 0, 0);
  }
  bf16x8 pa[2], ga[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    float pv[8], gv[8];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int q0 = 16 * ks + 8 * hf + 4 * hh;
      const f32x4 L = *(const f32x4 *)&lq[q0];
      const f32x4 Dv = *(const f32x4 *)&dd[q0];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 8 * ks + 4 * hf + j;
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], scale_log2, sh - L[j]));
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
      const bf16x8 dob = tr_pair(dt_, (tbo ^ (64 * dt)) + 16 * ks * ROWB,
                                 (tbo ^ (64 * dt + 32)) + (16 * ks + 8) * ROWB);
      dvacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[ks], dob, dvacc[dt], 0, 0, 0);
      const bf16x8 qbm = tr_pair(qt, (tbo ^ (64 * dt)) + 16 * ks * ROWB,
                                 (tbo ^ (64 * dt + 32)) + (16 * ks + 8) * ROWB);
      dkacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[ks], qbm, dkacc[dt], 0, 0, 0);
    }
  }
}

// Q and dO of `nrows` consecutive query rows starting at global row `q0row`
// of the slab into LDS (swizzled; rows at or past Nq are zero), with each
// row's D = dO . O and base-2 normaliser (+inf for rows past Nq or with lse
// = -inf, so that their P vanishes).  nrows is a multiple of 128.
template <int D>
__device__ __forceinline__ void load_query_rows(const BwdArgs &a, int bh, int q0row, int nrows,
                                                unsigned char *q_s, unsigned char *do_s,
                                                float *dq_s, float *lq_s, int tid) {
  constexpr int ROWB = D * 2;
  constexpr int NCH = D / 8;
  const int nrow = min(nrows, a.Nq - q0row);
  const uint16_t *qg = a.q + ((size_t)bh * a.Nq + (size_t)q0row) * D;
  const uint16_t *dg = a.dout + ((size_t)bh * a.Nq + (size_t)q0row) * D;
  for (int c = tid; c < nrows * NCH; c += 256) {
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
  // two lanes per query, each over half the dims
  for (int qr0 = 0; qr0 < nrows; qr0 += 128) {
    const int qr = qr0 + (tid >> 1), half = tid & 1;
    float part = 0.f;
    if (qr < nrow) {
      const size_t off = ((size_t)bh * a.Nq + (size_t)q0row + qr) * D + half * (D / 2);
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
        const float l = a.lse[(size_t)bh * a.Nq + (size_t)q0row + qr];
        if (l > -__builtin_inff()) L = l * kLog2e;
      }
      lq_s[qr] = L;
    }
  }
}

// Atomic form: one workgroup per query block; each pass's 128 keys are
// added into dK and dV at the pass's end.
template <int D>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv_kernel(BwdArgs a) {
  constexpr int ROWB = D * 2;        // row bytes
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
  const int bh = a.bh0 + wg / a.nqb;
  const size_t row_id = (size_t)bh * a.nqb + qb;
  const int32_t *idx_row = a.idx + row_id * a.max_blocks;
  const float *bias_row = a.bias ? a.bias + row_id * a.max_blocks : nullptr;
  int cnt = a.count[row_id];
  cnt = cnt < 0 ? 0 : (cnt > a.max_blocks ? a.max_blocks : cnt);
  const int kvb = 1 << a.kv_shift;

  load_query_rows<D>(a, bh, qb * 128, 128, q_s, do_s, dq_s, lq_s, tid);

  // per-lane LDS offsets: rows of Q/dO (A operands, query row l32 of
  // sub-tile qs, dims 16 ds + 8 hh ..) and transposing reads (B operands,
  // dim 32 dt + l32, queries 32 qs + 16 ks + 8 p + 4 hh + 0..3).  The
  // swizzle XORs the chunk field, which lies below the row bits, so each
  // family is one base register: row offset (ds) = rbo ^ 32 ds, transposing
  // offset (dt, ks, p) = (tbo ^ (64 dt + 32 p)) + (16 ks + 8 p) rows.
  int rbo = l32 * ROWB + ((hh ^ swz<D>(l32)) << 4);
  int tbo = tr_off<D>(4 * hh, 0, lane);

  const uint16_t *kbase = a.k + (size_t)bh * a.Nk * D;
  const uint16_t *vbase = a.v + (size_t)bh * a.Nk * D;
  f32x16 dka[DT], dva[DT];
  for (int base = 0; base < cnt; base += CAP) {
    const int pc = min(CAP, cnt - base);
    const int ntiles = ((pc << a.kv_shift) + KT - 1) / KT;
    __syncthreads();
    stage_list(a, idx_row, bias_row, base, pc, min(CAP, ((ntiles * KT) >> a.kv_shift) + 1), idx_s,
               sh_s, tid);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
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
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          dka[dt][r] = 0.f;
          dva[dt][r] = 0.f;
        }
#pragma unroll
      for (int qs = 0; qs < 4; ++qs)
        dkdv_substep<D>(q_s + qs * 32 * ROWB, do_s + qs * 32 * ROWB, lq_s + qs * 32,
                        dq_s + qs * 32, rbo, tbo, hh, kf, vf, sh, a.scale_log2, dka, dva);
      // the 32 keys' rows: register r <-> key 8 (r >> 2) + 4 hh + (r & 3)
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
              unsafeAtomicAdd(dkp + dt * 32, dka[dt][4 * g + j] * a.scale);
              unsafeAtomicAdd(dvp + dt * 32, dva[dt][4 * g + j]);
            }
          }
        }
      }
    }
  }
}

// Workspace form: one workgroup per pair of query blocks (2m, 2m + 1) of a
// slab, over the pair's union list (built by pair_union_kernel): entries
// both blocks list run their keys against all 256 queries (each half with
// its own entry's shift), the others against their own block's 128, and
// every union entry's dK (unscaled) and dV rows go once into its slot.
// Two neighbouring query blocks share a large part of their lists, so this
// stores fewer partial rows than one slot per list entry.  The union list
// is grouped by class (both, first only, second only), each class padded to
// whole passes, so a pass is of one class.  A pass's rows are stored during
// the next pass (one group of 8 keys after each of its first 4 query
// sub-steps) from a second set of accumulators, so the stores spread over
// the products instead of ending each pass in a burst.
template <int D>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv_pair_kernel(BwdArgs a) {
  constexpr int ROWB = D * 2;        // row bytes
  constexpr int DS = D / 16;         // k-steps over the head dim
  constexpr int DT = D / 32;         // 32-wide dim tiles
  constexpr int NW = 4;
  constexpr int KT = 128;            // gathered keys per pass (32 per wave)
  constexpr int QTB = 256 * ROWB;    // bytes of the pair's Q (or dO) rows

  __shared__ __attribute__((aligned(16))) unsigned char q_s[QTB], do_s[QTB];
  __shared__ __attribute__((aligned(16))) int32_t idx_s[CAP];
  __shared__ __attribute__((aligned(16))) float2 sh_s[CAP];
  __shared__ __attribute__((aligned(16))) float dq_s[256], lq_s[256];
  __shared__ __attribute__((aligned(16))) int32_t keyrow2_s[2][NW][32];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int pl = xcd_order(blockIdx.x, a.total_wg);  // pair of the chunk
  const int m = pl % a.npairs;
  const int bh = a.bh0 + pl / a.npairs;
  const int kvb = 1 << a.kv_shift;
  const int32_t *ub = a.ublk + (size_t)pl * a.ucap;
  const float2 *us = (const float2 *)a.ush + (size_t)pl * a.ucap;
  const int cb0 = a.ucls[(size_t)pl * 4], cb1 = a.ucls[(size_t)pl * 4 + 1];
  const int ulen = a.ucls[(size_t)pl * 4 + 2];
  // key position p of the union list (entry p >> kv_shift, token p &
  // (kvb - 1)) owns 2 D floats of the slot array: dK, then dV
  float *const prow = a.part + ((size_t)pl * a.ucap << a.kv_shift) * (2 * D);

  load_query_rows<D>(a, bh, 2 * m * 128, 256, q_s, do_s, dq_s, lq_s, tid);

  int rbo = l32 * ROWB + ((hh ^ swz<D>(l32)) << 4);
  int tbo = tr_off<D>(4 * hh, 0, lane);

  const uint16_t *kbase = a.k + (size_t)bh * a.Nk * D;
  const uint16_t *vbase = a.v + (size_t)bh * a.Nk * D;
  f32x16 dka[2][DT], dva[2][DT];
  int base = 0;
  // the rows of keys 8 g + 4 hh + j of pass t (register 4 g + j, lane <->
  // dim 32 dt + l32) from accumulator set P, into their entries' slots
  auto store_group = [&](auto P_c, int t, int g) {
    constexpr int P = decltype(P_c)::value;
    const int4 kr = *(const int4 *)&keyrow2_s[P][wave][8 * g + 4 * hh];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = j == 0 ? kr.x : (j == 1 ? kr.y : (j == 2 ? kr.z : kr.w));
      if (row >= 0) {
        const int p = (base << a.kv_shift) + t * KT + wave * 32 + 8 * g + 4 * hh + j;
        float *dst = prow + (size_t)p * (2 * D) + l32;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          __builtin_nontemporal_store(dka[P][dt][4 * g + j], dst + dt * 32);
          __builtin_nontemporal_store(dva[P][dt][4 * g + j], dst + D + dt * 32);
        }
      }
    }
  };
  for (base = 0; base < ulen; base += CAP) {
    const int pc = min(CAP, ulen - base);
    const int ntiles = ((pc << a.kv_shift) + KT - 1) / KT;
    const int nst = min(CAP, ((ntiles * KT) >> a.kv_shift) + 1);
    __syncthreads();
    for (int e = tid; e < nst; e += 256) {
      const int blk = e < pc ? ub[base + e] : -1;
      const float2 sh = e < pc ? us[base + e] : float2{-__builtin_inff(), -__builtin_inff()};
      idx_s[e] = blk;
      sh_s[e] = blk >= 0 ? sh : float2{-__builtin_inff(), -__builtin_inff()};
    }
    __syncthreads();
    // the phase's passes of each class, one run each: both halves (H0 = 0,
    // NH = 2), the first only (0, 1), the second only (1, 1); class ends
    // are whole passes
    auto tiles_below = [&](int cend) {
      return min(ntiles, max(0, ((cend - base) << a.kv_shift) / KT));
    };
    auto run = [&](auto H0_c, auto NH_c, int tb, int te) {
      constexpr int H0 = decltype(H0_c)::value, NH = decltype(NH_c)::value;
      auto tile = [&](auto P_c, int t, bool prev) {
        constexpr int P = decltype(P_c)::value, O = 1 - P;
        const int pos = t * KT + wave * 32 + l32;
        const int e = pos >> a.kv_shift;
        const int blk = idx_s[e];
        const int kk = (max(blk, 0) << a.kv_shift) + (pos & (kvb - 1));
        const bool ok = blk >= 0 && kk < a.Nk;
        const float2 shv = sh_s[e];
        const float sh0 = ok ? shv.x : -__builtin_inff(), sh1 = ok ? shv.y : -__builtin_inff();
        if (hh == 0) keyrow2_s[P][wave][l32] = ok ? kk : -1;
        const uint16_t *krp = kbase + (size_t)(ok ? kk : 0) * D;
        const uint16_t *vrp = vbase + (size_t)(ok ? kk : 0) * D;
        bf16x8 kf[DS], vf[DS];
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          kf[ds] = as_bf16x8(ld16(krp + ds * 16 + hh * 8));
          vf[ds] = as_bf16x8(ld16(vrp + ds * 16 + hh * 8));
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            dka[P][dt][r] = 0.f;
            dva[P][dt][r] = 0.f;
          }
        // the previous pass's rows are stored during the first half, so
        // each stored group's registers are free after it
#pragma unroll
        for (int h = H0; h < H0 + NH; ++h)
#pragma unroll
          for (int qs = 0; qs < 4; ++qs) {
            const int q32 = (4 * h + qs) * 32;
            dkdv_substep<D>(q_s + q32 * ROWB, do_s + q32 * ROWB, lq_s + q32, dq_s + q32, rbo, tbo,
                            hh, kf, vf, h == 0 ? sh0 : sh1, a.scale_log2, dka[P], dva[P]);
            if (h == H0 && prev) store_group(std::integral_constant<int, O>(), t - 1, qs);
          }
      };
      int t = tb;
      for (; t + 1 < te; t += 2) {
        tile(std::integral_constant<int, 0>(), t, t > tb);
        tile(std::integral_constant<int, 1>(), t + 1, true);
      }
      if (t < te) {
        tile(std::integral_constant<int, 0>(), t, t > tb);
#pragma unroll
        for (int g = 0; g < 4; ++g) store_group(std::integral_constant<int, 0>(), t, g);
      } else if (te > tb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) store_group(std::integral_constant<int, 1>(), t - 1, g);
      }
    };
    const int tb0 = tiles_below(cb0), tb1 = tiles_below(cb1);
    run(std::integral_constant<int, 0>(), std::integral_constant<int, 2>(), 0, tb0);
    run(std::integral_constant<int, 0>(), std::integral_constant<int, 1>(), tb0, tb1);
    run(std::integral_constant<int, 1>(), std::integral_constant<int, 1>(), tb1, ntiles);
  }
}

__global__ __launch_bounds__(256) void zero_kernel(f32x4 *p, size_t n4) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) p[i] = z;
}

// Union list of the pair of query blocks (2m, 2m + 1) of a slab (one
// workgroup per pair of the chunk), grouped by class: blocks both list,
// blocks only the first lists, blocks only the second lists, each class
// padded with empty entries (-1) to a whole number of 128-key passes.  An
// entry holds its block and the two lists' base-2 shifts (-inf where a list
// does not hold it).  Classes are formed when both lists are, below their
// counts, valid (block inside [0, M), shift above -inf) and strictly
// ascending, as the plans are; otherwise (or past 4,096 entries) the pair's
// union is the first list, then the second, invalid entries emptied, which
// is correct for any list.  ucls[4 pair + 0, 1, 2] = the ends of the three
// classes in entries.
constexpr int UCAP_LDS = 4096;

__device__ __forceinline__ int find_sorted(const int32_t *l, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (l[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo < n && l[lo] == v ? lo : -1;
}

__global__ __launch_bounds__(256) void pair_union_kernel(BwdArgs a) {
  __shared__ int32_t l0[UCAP_LDS], l1[UCAP_LDS];
  __shared__ int sc[3][256];
  const int tid = threadIdx.x;
  const int pl = blockIdx.x;
  const int m = pl % a.npairs;
  const int bh = a.bh0 + pl / a.npairs;
  const bool has1 = 2 * m + 1 < a.nqb;
  const size_t r0 = (size_t)bh * a.nqb + 2 * m, r1 = r0 + 1;
  const int32_t *i0 = a.idx + r0 * a.max_blocks, *i1 = a.idx + r1 * a.max_blocks;
  const float *b0 = a.bias ? a.bias + r0 * a.max_blocks : nullptr;
  const float *b1 = a.bias ? a.bias + r1 * a.max_blocks : nullptr;
  auto clampc = [&](int c) { return c < 0 ? 0 : (c > a.max_blocks ? a.max_blocks : c); };
  const int c0 = clampc(a.count[r0]), c1 = has1 ? clampc(a.count[r1]) : 0;
  const int bpp = a.kv_shift >= 7 ? 1 : 128 >> a.kv_shift;
  auto up = [&](int n) { return (n + bpp - 1) / bpp * bpp; };
  int32_t *ub = a.ublk + (size_t)pl * a.ucap;
  float2 *us = (float2 *)a.ush + (size_t)pl * a.ucap;
  const float NINF = -__builtin_inff();
  auto shift = [](const float *b, int e) { return b ? b[e] * kLog2e : 0.f; };
  auto valid = [&](int blk, float sh) { return blk >= 0 && blk < a.M && sh > NINF; };

  bool ok = c0 <= UCAP_LDS && c1 <= UCAP_LDS;
  if (ok) {
    for (int e = tid; e < c0; e += 256) {
      const int blk = i0[e];
      ok = ok && valid(blk, shift(b0, e)) && (e == 0 || i0[e - 1] < blk);
      l0[e] = blk;
    }
    for (int e = tid; e < c1; e += 256) {
      const int blk = i1[e];
      ok = ok && valid(blk, shift(b1, e)) && (e == 0 || i1[e - 1] < blk);
      l1[e] = blk;
    }
  }
  if (__syncthreads_and(ok)) {
    // thread t walks entries [lo, hi) of each list
    const int n0 = (c0 + 255) / 256, n1 = (c1 + 255) / 256;
    const int lo0 = min(c0, tid * n0), hi0 = min(c0, lo0 + n0);
    const int lo1 = min(c1, tid * n1), hi1 = min(c1, lo1 + n1);
    int nb = 0, no1 = 0;
    for (int e = lo0; e < hi0; ++e) nb += find_sorted(l1, c1, l0[e]) >= 0;
    for (int e = lo1; e < hi1; ++e) no1 += find_sorted(l0, c0, l1[e]) < 0;
    sc[0][tid] = nb;
    sc[1][tid] = (hi0 - lo0) - nb;
    sc[2][tid] = no1;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {  // inclusive scans
      int v[3];
#pragma unroll
      for (int c = 0; c < 3; ++c) v[c] = tid >= off ? sc[c][tid - off] : 0;
      __syncthreads();
#pragma unroll
      for (int c = 0; c < 3; ++c) sc[c][tid] += v[c];
      __syncthreads();
    }
    const int NB = sc[0][255], NO0 = sc[1][255], NO1 = sc[2][255];
    const int PB = up(NB), PO0 = up(NO0), PO1 = up(NO1);
    int pb = sc[0][tid] - nb, po0 = PB + sc[1][tid] - ((hi0 - lo0) - nb);
    int po1 = PB + PO0 + sc[2][tid] - no1;
    for (int e = lo0; e < hi0; ++e) {
      const int blk = l0[e], j = find_sorted(l1, c1, blk);
      if (j >= 0) {
        ub[pb] = blk;
        us[pb++] = float2{shift(b0, e), shift(b1, j)};
      } else {
        ub[po0] = blk;
        us[po0++] = float2{shift(b0, e), NINF};
      }
    }
    for (int e = lo1; e < hi1; ++e) {
      const int blk = l1[e];
      if (find_sorted(l0, c0, blk) < 0) {
        ub[po1] = blk;
        us[po1++] = float2{NINF, shift(b1, e)};
      }
    }
    auto pad = [&](int from, int to) {
      for (int u = from + tid; u < to; u += 256) {
        ub[u] = -1;
        us[u] = float2{NINF, NINF};
      }
    };
    pad(NB, PB);
    pad(PB + NO0, PB + PO0);
    pad(PB + PO0 + NO1, PB + PO0 + PO1);
    if (tid == 0) {
      a.ucls[(size_t)pl * 4] = PB;
      a.ucls[(size_t)pl * 4 + 1] = PB + PO0;
      a.ucls[(size_t)pl * 4 + 2] = PB + PO0 + PO1;
    }
  } else {
    const int P0 = up(c0), P1 = up(c1);
    for (int u = tid; u < P0 + P1; u += 256) {
      const bool first = u < P0;
      const int e = first ? u : u - P0;
      int blk = -1;
      float sh = NINF;
      if (e < (first ? c0 : c1)) {
        blk = (first ? i0 : i1)[e];
        sh = shift(first ? b0 : b1, e);
        if (!valid(blk, sh)) {
          blk = -1;
          sh = NINF;
        }
      }
      ub[u] = blk;
      us[u] = first ? float2{sh, NINF} : float2{NINF, sh};
    }
    if (tid == 0) {
      a.ucls[(size_t)pl * 4] = 0;
      a.ucls[(size_t)pl * 4 + 1] = P0;
      a.ucls[(size_t)pl * 4 + 2] = P0 + P1;
    }
  }
}

// Key-major lists, pass 1 (FILL = false): count the union entries listing
// each block; pass 2 (FILL = true): write (pair of the chunk) * ucap +
// entry, the entry's slot, at the block's cursor.  One workgroup per pair
// of the chunk.
template <bool FILL>
__global__ __launch_bounds__(256) void csr_pass_kernel(BwdArgs a) {
  const int pl = blockIdx.x;
  const int s = pl / a.npairs;
  const int32_t *ub = a.ublk + (size_t)pl * a.ucap;
  const int n = a.ucls[(size_t)pl * 4 + 2];
  for (int u = threadIdx.x; u < n; u += 256) {
    const int blk = ub[u];
    if (blk < 0) continue;
    if (FILL) {
      const int pos = atomicAdd(&a.kcur[(size_t)s * a.Ms + blk], 1);
      a.ent[(size_t)s * a.cap + pos] = pl * a.ucap + u;
    } else {
      atomicAdd(&a.kstart[(size_t)s * a.Ms + blk], 1);
    }
  }
}

// Exclusive scan of one slab's counts, in place: kstart[b] = entries of
// blocks before b, kstart[M] = all; kcur = kstart.  One workgroup per slab.
__global__ __launch_bounds__(1024) void csr_scan_kernel(BwdArgs a) {
  __shared__ int part[1024];
  int32_t *ks = a.kstart + (size_t)blockIdx.x * a.Ms;
  int32_t *kc = a.kcur + (size_t)blockIdx.x * a.Ms;
  const int t = threadIdx.x;
  const int per = (a.M + 1023) / 1024;
  const int lo = min(a.M, t * per), hi = min(a.M, lo + per);
  int sum = 0;
  for (int b = lo; b < hi; ++b) sum += ks[b];
  part[t] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
    const int v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = part[t] - sum;
  for (int b = lo; b < hi; ++b) {
    const int c = ks[b];
    ks[b] = run;
    kc[b] = run;
    run += c;
  }
  if (t == 1023) ks[a.M] = part[1023];
}

// Each KV block's slot numbers in ascending order (one wave per block):
// the fill above places them in the order its integer atomics ran, which
// varies from run to run; summing them in slot order makes dK and dV the
// same bits on every run and for any number of slabs per pass.  An entry's
// rank is the number of the block's slots below it (slots are distinct).
__global__ __launch_bounds__(256) void csr_sort_kernel(BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const long long gw = (long long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (gw >= (long long)a.nslab * a.M) return;
  const int s = (int)(gw / a.M), b = (int)(gw % a.M);
  const int32_t *ks = a.kstart + (size_t)s * a.Ms;
  const int beg = ks[b], n = ks[b + 1] - beg;
  const int32_t *ent = a.ent + (size_t)s * a.cap + beg;
  int32_t *out = a.ents + (size_t)s * a.cap + beg;
  for (int i0 = 0; i0 < n; i0 += 64) {
    const int own = i0 + lane < n ? ent[i0 + lane] : 0x7fffffff;
    int rank = 0;
    for (int j0 = 0; j0 < n; j0 += 64) {
      const int other = j0 + lane < n ? ent[j0 + lane] : 0x7fffffff;
#pragma unroll 16
      for (int j = 0; j < 64; ++j) rank += __shfl(other, j, 64) < own ? 1 : 0;
    }
    if (i0 + lane < n) out[rank] = own;
  }
}

// dK and dV of one KV block (one wave): the sum, in fp32 and in ascending
// slot order, of the partial rows of every entry that lists it; rows at or
// past Nk are not written.
// Lane l handles the 16-byte pieces c = c0 + l + 64 u of the block's
// kvb * 2D floats (token c / (D/2); dK for the first D/4 pieces of a
// token, dV for the rest).
template <int D>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs a) {
  constexpr int U = 4;
  const int lane = threadIdx.x & 63;
  const long long gw = (long long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (gw >= (long long)a.nslab * a.M) return;
  const int s = (int)(gw / a.M), b = (int)(gw % a.M);
  const int32_t *ks = a.kstart + (size_t)s * a.Ms;
  const int beg = ks[b], end = ks[b + 1];
  const int32_t *ent = a.ents + (size_t)s * a.cap;
  const int kvb = 1 << a.kv_shift;
  const size_t F4 = (size_t)kvb * (D / 2);                // pieces per entry
  const int ntok = min(kvb, a.Nk - b * kvb);
  const int nv = ntok * (D / 2);                          // pieces written
  const f32x4 *part = (const f32x4 *)a.part;
  const size_t key0 = (size_t)(a.bh0 + s) * a.Nk + (size_t)b * kvb;
  for (int c0 = 0; c0 < nv; c0 += 64 * U) {
    f32x4 acc[U];
    bool on[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      on[u] = c0 + lane + 64 * u < nv;
    }
    const size_t cl = (size_t)(c0 + lane);
    int p = beg;
    for (; p + 4 <= end; p += 4) {
      f32x4 x[4][U];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 *src = part + (size_t)ent[p + i] * F4 + cl;
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (on[u]) x[i][u] = src[64 * u];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (on[u]) acc[u] += x[i][u];
    }
    for (; p < end; ++p) {
      const f32x4 *src = part + (size_t)ent[p] * F4 + cl;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (on[u]) acc[u] += src[64 * u];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!on[u]) continue;
      const int c = c0 + lane + 64 * u;
      const int j = c / (D / 2), w = c % (D / 2);
      if (w < D / 4)
        *(f32x4 *)(a.dk + (key0 + j) * D + 4 * w) = acc[u] * a.scale;
      else
        *(f32x4 *)(a.dv + (key0 + j) * D + 4 * (w - D / 4)) = acc[u];
    }
  }
}

}  // namespace

int launch_attn_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
                    const float *lse, int B, int H, int Nq, int Nk, int d, int kv_block,
                    const int32_t *idx, const float *bias, const int32_t *count, int max_blocks,
                    float scale, float *dq, float *dk, float *dv, hipStream_t stream) {
  clear_pending_error();
  BwdArgs a{};
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
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<128>), dim3((unsigned)total), dim3(256), 0,
                       stream, a);
  } else {
    hipLaunchKernelGGL((attn_bwd_dq_kernel<64>), dim3((unsigned)total), dim3(256), 0, stream, a);
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<64>), dim3((unsigned)total), dim3(256), 0,
                       stream, a);
  }
  return status_of(hipGetLastError());
}

namespace {

struct SlabLayout {
  int npairs, ucap;   // pairs of query blocks, union entries per pair
  size_t part_bytes;  // partial rows of one slab
  int Ms, cap;        // ints per slab of kstart / kcur, and of ent (also ents, ublk, ush pairs)
  int ncls;           // ints per slab of ucls
  size_t bytes;       // all of one slab
};

SlabLayout slab_layout(int Nq, int Nk, int d, int kv_block, int max_blocks) {
  SlabLayout L;
  const int nqb = (Nq + 127) / 128;
  const size_t M = ((size_t)Nk + kv_block - 1) / kv_block;
  const int bpp = kv_block >= 128 ? 1 : 128 / kv_block;  // blocks per 128-key pass
  L.npairs = (nqb + 1) / 2;
  L.ucap = 2 * max_blocks + 3 * bpp;  // both lists, three classes padded to whole passes
  L.part_bytes = (size_t)L.npairs * L.ucap * kv_block * 2 * d * sizeof(float);  // multiple of 512
  L.Ms = (int)((M + 1 + 63) / 64 * 64);
  L.cap = (int)(((size_t)L.npairs * L.ucap + 63) / 64 * 64);
  L.ncls = (L.npairs * 4 + 63) / 64 * 64;
  // 256-byte multiples each
  L.bytes = L.part_bytes + 2 * (size_t)L.Ms * 4 + (size_t)L.cap * (4 + 4 + 4 + 8) + (size_t)L.ncls * 4;
  return L;
}

}  // namespace

size_t attn_bwd_slab_bytes(int Nq, int Nk, int d, int kv_block, int max_blocks) {
  return slab_layout(Nq, Nk, d, kv_block, max_blocks).bytes;
}

long long attn_bwd_union_entries(int Nq, int kv_block, int max_blocks) {
  const long long bpp = kv_block >= 128 ? 1 : 128 / kv_block;
  return (long long)((Nq + 127) / 128 + 1) / 2 * (2LL * max_blocks + 3 * bpp);
}

int launch_attn_bwd_ws(const void *q, const void *k, const void *v, const void *o,
                       const void *dout, const float *lse, int B, int H, int Nq, int Nk, int d,
                       int kv_block, const int32_t *idx, const float *bias, const int32_t *count,
                       int max_blocks, float scale, float *dq, float *dk, float *dv,
                       void *workspace, size_t workspace_bytes, hipStream_t stream) {
  clear_pending_error();
  const SlabLayout L = slab_layout(Nq, Nk, d, kv_block, max_blocks);
  const int BH = B * H;
  long long per = (long long)(workspace_bytes / L.bytes);
  per = per < BH ? per : BH;
  const long long by_index = 0x7fffffffLL / L.cap;  // ent values and the fill's positions
  per = per < by_index ? per : by_index;
  if (per < 1) return BSA_ERR_WORKSPACE;
  BwdArgs a{};
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
  a.Ms = L.Ms;
  a.cap = L.cap;
  a.npairs = L.npairs;
  a.ucap = L.ucap;
  a.total_wg = BH * a.nqb;
  if (d == 128)
    hipLaunchKernelGGL((attn_bwd_dq_kernel<128>), dim3((unsigned)a.total_wg), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_bwd_dq_kernel<64>), dim3((unsigned)a.total_wg), dim3(256), 0, stream, a);
  unsigned char *ws = (unsigned char *)workspace;
  for (int bh0 = 0; bh0 < BH; bh0 += (int)per) {
    const int n = (int)(BH - bh0 < per ? BH - bh0 : per);
    a.bh0 = bh0;
    a.nslab = n;
    a.part = (float *)ws;
    a.kstart = (int32_t *)(ws + (size_t)n * L.part_bytes);
    a.kcur = a.kstart + (size_t)n * L.Ms;
    a.ent = a.kcur + (size_t)n * L.Ms;
    a.ents = a.ent + (size_t)n * L.cap;
    a.ublk = a.ents + (size_t)n * L.cap;
    a.ush = (float *)(a.ublk + (size_t)n * L.cap);
    a.ucls = (int32_t *)(a.ush + 2 * (size_t)n * L.cap);
    a.total_wg = n * a.npairs;
    const size_t z4 = (size_t)n * L.Ms / 4;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)min((size_t)8192, (z4 + 255) / 256)), dim3(256),
                       0, stream, (f32x4 *)a.kstart, z4);
    hipLaunchKernelGGL(pair_union_kernel, dim3((unsigned)a.total_wg), dim3(256), 0, stream, a);
    hipLaunchKernelGGL((csr_pass_kernel<false>), dim3((unsigned)a.total_wg), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(csr_scan_kernel, dim3((unsigned)n), dim3(1024), 0, stream, a);
    hipLaunchKernelGGL((csr_pass_kernel<true>), dim3((unsigned)a.total_wg), dim3(256), 0, stream, a);
    const unsigned rg = (unsigned)(((long long)n * a.M + 3) / 4);
    hipLaunchKernelGGL(csr_sort_kernel, dim3(rg), dim3(256), 0, stream, a);
    if (d == 128) {
      hipLaunchKernelGGL((attn_bwd_dkdv_pair_kernel<128>), dim3((unsigned)a.total_wg), dim3(256),
                         0, stream, a);
      hipLaunchKernelGGL((bwd_reduce_kernel<128>), dim3(rg), dim3(256), 0, stream, a);
    } else {
      hipLaunchKernelGGL((attn_bwd_dkdv_pair_kernel<64>), dim3((unsigned)a.total_wg), dim3(256),
                         0, stream, a);
      hipLaunchKernelGGL((bwd_reduce_kernel<64>), dim3(rg), dim3(256), 0, stream, a);
    }
  }
  return status_of(hipGetLastError());
}

}  // namespace bsa
