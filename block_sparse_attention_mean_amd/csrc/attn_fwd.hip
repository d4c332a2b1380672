// Fused block-sparse attention forward for gfx950.
//
// AB-Attention page (onedev.kr/papers/1521), section "전제와 한계", first
// paragraph: the kernel gathers the sampled small KV blocks by index into
// full matrix-core tiles and performs the -log pi logit shift, the online
// softmax and the value accumulation in one pass, with no token reordering
// and no reordered copy of the sequence in memory.  The shift itself is the
// 1/pi weighting of section "어떻게 쓰나".
//
// Design (one workgroup = one 128-query block of one (b, h), 4 waves; three
// workgroups share a CU, so each SIMD interleaves three waves' matrix and
// vector work and a stall at one workgroup's barrier is covered by the
// others):
//   * wave w owns queries 32 w .. +32 and computes every key of every tile;
//   * the block list and shifts of the query block are staged in LDS, so
//     gather addresses never wait on global memory;
//   * listed blocks are gathered with direct global->LDS 16-byte loads into
//     a ring of three 32-key K/V tiles (tile t+2 is requested while tile t
//     is consumed); K and V stay row-major with 16-byte-chunk XOR swizzles
//     (bank-conflict free for their MFMA operand reads) realised by each
//     lane's choice of source address;
//   * S^T = K Q^T (bf16 MFMA 32x32x16; Q stays in registers as the B
//     operand), with the K rows fed in a permuted order so that each lane's
//     accumulators hold 8 consecutive keys of one query -- exactly the
//     B-operand layout of O^T = V^T P^T; the V^T operand comes from the
//     row-major V tile through the gfx950 transposing LDS read
//     (ds_read_b64_tr_b16); P never leaves registers;
//   * base-2 softmax (scale and shift pre-multiplied by log2 e) against a
//     lazy reference maximum folded into the logit fma: O and the row sum
//     are rescaled only when a tile exceeds the reference by more than 8
//     (a wave-uniform test);
//   * group-shift path, taken when each wave load (4 rows at d = 128, 8 at
//     d = 64) lies inside one KV block: every aligned group of 4 keys
//     shares one shift, staged once per phase in the order the softmax
//     reads it, so a lane's 16 logits need 4 shifts (one 16-byte LDS read);
//     the block index of a load is wave-uniform, so it comes from a scalar
//     load and the row address from scalar arithmetic, leaving one vector
//     add per gather.  When Nk is not a whole number of loads, a separate
//     instance also handles the load and the 4-key group crossing Nk: the
//     load's lanes past Nk re-read its last valid row, and the tile's keys
//     past Nk are masked before the exponentials;
//   * half-load variant of that path, for KV blocks of half a wave load
//     (2 tokens at d = 128, 4 at d = 64) and Nk a whole number of blocks:
//     each 32-lane half of a load gathers one block (two scalar list loads
//     per load, one lane select), and at d = 128 the shifts are staged per
//     2-key group (8 per lane and tile, two 16-byte reads);
//   * otherwise (smaller blocks, or a block crossing Nk) the per-key path:
//     the phase's list staged in LDS and one shift per key.
#include <type_traits>

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

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// MFMA A-row -> key within a 32-key sub-tile, chosen so that accumulator
// register r of lane half h holds key 16 (r >> 3) + 8 h + (r & 7).
__device__ __forceinline__ int key_of_row(int i) {
  return ((i >> 4) << 4) | (((i >> 2) & 1) << 3) | (((i >> 3) & 1) << 2) | (i & 3);
}

// Workgroup barrier for the gather ring: this wave's gathers older than the
// newest N vector-memory ops and all its LDS writes are complete, then
// s_barrier.  The compiler-only fences keep LDS accesses from moving across
// it; no release fence is used because that would also wait for the gathers
// still in flight into other ring slots.
template <int N>
__device__ __forceinline__ void ring_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// 16-byte-chunk XOR swizzles of the row-major K and V tiles, chosen so
// that the MFMA operand reads are free of LDS bank conflicts: K is read as
// 16 rows x one chunk per 16 lanes, V (transposing read) as 4 consecutive
// rows x 4 consecutive chunks per 32 lanes.  256-byte rows (d = 128) fill
// the 64 banks; 128-byte rows (d = 64) pair up.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

// Position of 4-key group q (0..7) of a tile in the shift ring when the
// shift is uniform per group: [0 1 4 5 | 2 3 6 7], so that lane half h
// finds its four groups (keys 8h + 0..7 and 16 + 8h + 0..7) in one 16-byte
// read at 4 h.
__device__ __forceinline__ int quad_pos(int q) {
  return (q & 1) | (((q >> 2) & 1) << 1) | (((q >> 1) & 1) << 2);
}
// The same for 2-key groups p (0..15): [0-3 8-11 | 4-7 12-15], so that lane
// half h finds its eight pairs in two 16-byte reads at 8 h.
__device__ __forceinline__ int pair_pos(int p) {
  return (((p >> 2) & 1) << 3) | ((p >> 3) << 2) | (p & 3);
}

// QUAD: group shifts and the scalar gather (KV blocks of at least one wave
// load); PART: with them, loads and 4-key groups crossing Nk may occur (Nk
// not a whole number of wave loads), so their rows past Nk are handled.
// HALF (with QUAD, without PART): KV blocks of exactly half a wave load
// (2 tokens at d = 128, 4 at d = 64) and Nk a whole number of blocks; each
// 32-lane half of a load gathers one block, and at d = 128 the shifts are
// staged per 2-key group.
template <int D, bool QUAD, bool PART, bool HALF = false>
__global__ __launch_bounds__(256, 3) void attn_fwd_kernel(AttnArgs a) {
  constexpr int NW = 4;              // waves: one 32-query quarter each
  constexpr int KT = 32;             // keys per tile
  constexpr int NBUF = 3;            // ring slots
  constexpr int NCH = D / 8;         // 16-byte chunks per row
  constexpr int ROWB = D * 2;        // row bytes
  constexpr int TILEB = KT * ROWB;   // bytes of one K (or V) tile
  constexpr int RPI = 64 / NCH;      // rows per 1 KB wave load
  constexpr int RPW = KT / NW;       // tile rows gathered by one wave
  constexpr int LPW = RPW / RPI;     // wave loads per operand per tile
  constexpr int LPT = 2 * LPW;       // vector-memory ops per wave per tile
  constexpr int DS = D / 16;         // k-steps of QK^T
  constexpr int DT = D / 32;         // dim tiles of O^T
  constexpr int CAP = 512;           // list entries staged per phase (per-key shifts)
  constexpr int CAPG = 1024;         // key groups staged per phase (group shifts)
  constexpr int SG = HALF && D == 128 ? 2 : 4;  // keys per group shift
  static_assert(!HALF || (QUAD && !PART), "HALF is a mode of the group-shift path");
  static_assert(LPW >= 1 && RPW % RPI == 0, "tile too small for the gather split");

  // Ring of K/V tiles.  Separate arrays let the compiler see that a gather
  // into one slot never aliases the reads of another, so it does not wait
  // for in-flight gathers before reading the current slot.
  __shared__ __attribute__((aligned(16))) unsigned char k0[TILEB], v0[TILEB];
  __shared__ __attribute__((aligned(16))) unsigned char k1[TILEB], v1[TILEB];
  __shared__ __attribute__((aligned(16))) unsigned char k2[TILEB], v2[TILEB];
  // Per-key shifts: the phase's list in LDS and a shift ring beside the
  // tiles.  Group shifts: one shift per 4-key group of the phase, stored
  // per tile in the order the softmax reads them.
  __shared__ __attribute__((aligned(16))) int32_t idx_s[QUAD ? 1 : CAP];
  __shared__ __attribute__((aligned(16))) float bias_s[QUAD ? 1 : CAP];
  __shared__ __attribute__((aligned(16))) float bring[QUAD ? 1 : NBUF * KT];
  __shared__ __attribute__((aligned(16))) float gb_s[QUAD ? CAPG : 1];
  // Group shifts with Nk inside a 4-key group (only the block holding key
  // Nk - 1): per tile, the rows past Nk of such groups.
  __shared__ uint32_t pmask_s[QUAD && PART ? CAPG / 8 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  // XCD-aware order: the hardware deals workgroups round-robin over 8
  // XCDs; give each XCD a contiguous run of query blocks.
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
  const int bh = wg / a.nqb;
  const size_t row_id = (size_t)bh * a.nqb + qb;
  const uint16_t *qbase = a.q + (size_t)bh * a.Nq * D;
  const unsigned char *kbase = (const unsigned char *)(a.k + (size_t)bh * a.Nk * D);
  const unsigned char *vbase = (const unsigned char *)(a.v + (size_t)bh * a.Nk * D);
  const int32_t *idx_row = a.idx + row_id * a.max_blocks;
  const float *bias_row = a.bias ? a.bias + row_id * a.max_blocks : nullptr;
  int cnt = a.count[row_id];
  cnt = cnt < 0 ? 0 : (cnt > a.max_blocks ? a.max_blocks : cnt);
  const int kvb = 1 << a.kv_shift;

  // ---- Q fragments (B operand of S^T): query column l32, dims 16 ds + 8 hh ..
  const int qrow = qb * 128 + wave * 32 + l32;
  bf16x8 qf[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (qrow < a.Nq) v = ld16(qbase + (size_t)qrow * D + ds * 16 + hh * 8);
    qf[ds] = as_bf16x8(v);
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_run = 0.f;   // reference maximum (base 2), raised lazily
  float l_run = 0.f;
  bool fresh = true;    // no key of this query seen yet (same in both halves)

  int nkeys = 0, ntiles = 0, pbase = 0, pcnt = 0;

  // Per-lane constants of the gather: tile row of load j and the swizzled
  // source chunk offsets of that row in K and V (with group shifts, the
  // offsets include the row's distance from the first row of the load).
  int g_row[LPW], g_koff[LPW], g_voff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int r = wave * RPW + j * RPI + lane / NCH;
    const int cl = lane % NCH;
    const int rel = QUAD ? ((lane / NCH) % (HALF ? RPI / 2 : RPI)) * ROWB : 0;
    g_row[j] = r;
    g_koff[j] = rel + ((cl ^ swz_k<D>(r)) << 4);
    g_voff[j] = rel + ((cl ^ swz_v<D>(r)) << 4);
  }

  auto kslot = [&](auto c) -> unsigned char * {
    constexpr int S = decltype(c)::value;
    return S == 0 ? k0 : (S == 1 ? k1 : k2);
  };
  auto vslot = [&](auto c) -> unsigned char * {
    constexpr int S = decltype(c)::value;
    return S == 0 ? v0 : (S == 1 ? v1 : v2);
  };

  // Group shifts: the RPI rows of each wave load lie in one KV block
  // (blocks of at least RPI keys, tiles starting on block boundaries), so
  // the block index is wave-uniform.  It is read with a scalar load before
  // the ring barrier (its latency hides behind the wait) and the key row of
  // the load becomes a scalar base; each lane adds its 32-bit offset.
  // The arithmetic is 32-bit unsigned and kept to what memory safety needs
  // (a loop step here is issue-bound: trimming it from about 70 to about 45
  // scalar instructions per tile measured 1-1.5 % faster): entries past the
  // phase's list read its last entry, and a row outside [0, Nk) -- from an
  // invalid entry or past the end -- becomes row 0.  Whether the keys count
  // is decided by the staged group shifts, which are -inf for every such
  // entry, so no other check is needed.  The list's byte offset fits 32
  // bits because the boundary caps max_blocks * kv_block below 2^31.  nvr
  // counts the load's rows below Nk: a load crossing Nk (rare) re-reads its
  // last valid row in the lanes of the rows past it.
  typedef const __attribute__((address_space(4))) int32_t cint_t;
  auto rows_of = [&](int t, int (&row)[LPW], int (&nvr)[LPW]) {
    unsigned blk[LPW];
#pragma unroll
    for (int j = 0; j < LPW; ++j) {  // all loads first (one wait)
      const unsigned e = (unsigned)(t * KT + wave * RPW + j * RPI) >> a.kv_shift;
      const unsigned ec = min(e, (unsigned)pcnt - 1u);
      const unsigned byte = 4u * ((unsigned)pbase + ec);  // a scalar-offset load
      blk[j] = (unsigned)*(cint_t *)((const __attribute__((address_space(4))) char *)idx_row + byte);
    }
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const unsigned pos = (unsigned)(t * KT + wave * RPW + j * RPI);
      const unsigned kk = (blk[j] << a.kv_shift) + (pos & (unsigned)(kvb - 1));
      row[j] = kk < (unsigned)a.Nk ? (int)kk : 0;
      const int left = a.Nk - row[j];
      nvr[j] = PART ? (left < RPI ? left : RPI) : RPI;
    }
  };
  auto issue_rows = [&](auto slot_c, const int (&row)[LPW], const int (&nvr)[LPW]) {
    unsigned char *kt = kslot(slot_c);
    unsigned char *vt = vslot(slot_c);
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const size_t src = (size_t)(unsigned)row[j] * ROWB;
      const int dst = (wave * RPW + j * RPI) * ROWB;
      unsigned ko = (unsigned)g_koff[j], vo = (unsigned)g_voff[j];
      if (PART && nvr[j] < RPI) {  // uniform
        const unsigned rel = (unsigned)((lane / NCH) * ROWB);
        const unsigned cap = (unsigned)((nvr[j] - 1) * ROWB);
        const unsigned fix = rel < cap ? rel : cap;
        ko = ko - rel + fix;
        vo = vo - rel + fix;
      }
      __builtin_amdgcn_global_load_lds((const void *)(kbase + src + ko), (lds_void *)(kt + dst), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void *)(vbase + src + vo), (lds_void *)(vt + dst), 16, 0, 0);
    }
  };

  // HALF: the two halves of wave load j gather one block each (entries
  // e(pos) and e(pos + RPI / 2)); a block past the list or outside
  // [0, Nk) reads row 0, its keys masked by the staged shifts.
  auto rows_of_h = [&](int t, int (&row)[2 * LPW]) {
    unsigned blk[2 * LPW];
#pragma unroll
    for (int i = 0; i < 2 * LPW; ++i) {  // all loads first (one wait)
      const unsigned pos = (unsigned)(t * KT + wave * RPW + (i >> 1) * RPI + (i & 1) * (RPI / 2));
      const unsigned ec = min(pos >> a.kv_shift, (unsigned)pcnt - 1u);
      const unsigned byte = 4u * ((unsigned)pbase + ec);
      blk[i] = (unsigned)*(cint_t *)((const __attribute__((address_space(4))) char *)idx_row + byte);
    }
#pragma unroll
    for (int i = 0; i < 2 * LPW; ++i) {
      const unsigned kk = blk[i] << a.kv_shift;
      row[i] = kk < (unsigned)a.Nk ? (int)kk : 0;
    }
  };
  auto issue_rows_h = [&](auto slot_c, const int (&row)[2 * LPW]) {
    unsigned char *kt = kslot(slot_c);
    unsigned char *vt = vslot(slot_c);
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      // scalar base at the lower of the two rows, 32-bit lane offsets (the
      // launch keeps Nk rows below 4 GiB)
      const unsigned r0 = (unsigned)row[2 * j], r1 = (unsigned)row[2 * j + 1];
      const unsigned rmin = min(r0, r1);
      const unsigned dl = ((hh ? r1 : r0) - rmin) * (unsigned)ROWB;
      const size_t src = (size_t)rmin * ROWB;
      const int dst = (wave * RPW + j * RPI) * ROWB;
      __builtin_amdgcn_global_load_lds((const void *)(kbase + src + (dl + (unsigned)g_koff[j])), (lds_void *)(kt + dst), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void *)(vbase + src + (dl + (unsigned)g_voff[j])), (lds_void *)(vt + dst), 16, 0, 0);
    }
  };

  // Per-key shifts: gather tile t into slot S; this wave loads rows
  // [RPW w, RPW w + RPW).  Masked keys (invalid or padded list entries, rows
  // past Nk) load row 0 and get a -inf shift.
  auto issue = [&](auto slot_c, int t) {
    constexpr int S = decltype(slot_c)::value;
    unsigned char *kt = kslot(slot_c);
    unsigned char *vt = vslot(slot_c);
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int pos = t * KT + g_row[j];
      const int e = pos >> a.kv_shift;  // staged entries cover whole tiles
      const int kk = (idx_s[e] << a.kv_shift) + (pos & (kvb - 1));
      const bool ok = kk < a.Nk;        // rows past the last valid key
      const size_t src = (size_t)(ok ? kk : 0) * ROWB;
      const int dst = (wave * RPW + j * RPI) * ROWB;  // wave-uniform
      __builtin_amdgcn_global_load_lds((const void *)(kbase + src + g_koff[j]), (lds_void *)(kt + dst), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void *)(vbase + src + g_voff[j]), (lds_void *)(vt + dst), 16, 0, 0);
      if (lane % NCH == 0) bring[S * KT + g_row[j]] = ok ? bias_s[e] : -__builtin_inff();
    }
  };
  auto issue_any = [&](auto slot_c, int t) {
    if constexpr (HALF) {
      int row[2 * LPW];
      rows_of_h(t, row);
      issue_rows_h(slot_c, row);
    } else if constexpr (QUAD) {
      int row[LPW], nvr[LPW];
      rows_of(t, row, nvr);
      issue_rows(slot_c, row, nvr);
    } else {
      issue(slot_c, t);
    }
  };

  const int krow = key_of_row(l32);
  const int gi = lane & 15;  // index inside a 16-lane group
  const int gg = lane >> 4;  // group 0..3

  // LDS byte offsets of this lane's MFMA operand reads inside a K tile and
  // (for rows 0..3 of each 16-row group) inside a V tile.  The empty asm
  // before each use makes the value opaque to the optimiser, so the slot
  // base goes into the read's immediate offset instead of one full address
  // per slot and read being kept live, which at three workgroups per CU
  // would spill; updating in place costs no copy.
  int koff[DS], voff[DT];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) koff[ds] = krow * ROWB + (((2 * ds + hh) ^ swz_k<D>(krow)) << 4);
  {
    const int r0 = 8 * (gg >> 1) + (gi >> 2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int n0 = dt * 32 + 16 * (gg & 1) + 4 * (gi & 3);
      voff[dt] = r0 * ROWB + (((n0 >> 3) ^ swz_v<D>(r0)) << 4) + ((n0 >> 2) & 1) * 8;
    }
  }
  // S^T of the tile in slot S (32 keys x this wave's 32 queries).
  auto qk = [&](auto slot_c, f32x16 &sacc) {
    const unsigned char *kt = kslot(slot_c);
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      asm volatile("" : "+v"(koff[ds]));
      const bf16x8 af = as_bf16x8(*(const u32x4 *)(kt + koff[ds]));
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[ds], sacc, 0, 0, 0);
    }
  };

  // Softmax of tile t of the phase, in slot S (logits in sacc), and
  // O^T += V^T P^T.
  auto softmax_pv = [&](auto slot_c, f32x16 &sacc, int t) {
    constexpr int S = decltype(slot_c)::value;
    const unsigned char *vt = vslot(slot_c);
    // Base-2 logits relative to the running reference m_run of each query:
    // t = s * scale * log2 e + (shift - m_run), one fma per logit.  The
    // reference is raised (and O, l rescaled) only when some lane sees a
    // logit above it by more than 8, or sees its first valid key; the two
    // lane halves (different keys of the same query) then agree on the new
    // reference through one exchange.
    const float *bt = bring + S * KT;
    if constexpr (QUAD && SG == 2) {
      // pairs (m, half, i) at 8 half + 4 m + i: register r holds pair r / 2
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const f32x4 bq = *(const f32x4 *)&gb_s[t * (KT / 2) + 8 * hh + 4 * m];
#pragma unroll
        for (int r = 8 * m; r < 8 * m + 8; ++r)
          sacc[r] = __builtin_fmaf(sacc[r], a.scale_log2, bq[(r >> 1) & 3] - m_run);
      }
    } else if (QUAD) {
      // groups (m, half): (0,0) (0,1) (1,0) (1,1)
      const f32x4 bq = *(const f32x4 *)&gb_s[t * (KT / 4) + 4 * hh];
      f32x4 bm;
#pragma unroll
      for (int i = 0; i < 4; ++i) bm[i] = bq[i] - m_run;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = __builtin_fmaf(sacc[r], a.scale_log2, bm[r >> 2]);
    } else {
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2) {
        const f32x4 b0 = *(const f32x4 *)&bt[m2 * 16 + hh * 8];
        const f32x4 b1 = *(const f32x4 *)&bt[m2 * 16 + hh * 8 + 4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sacc[m2 * 8 + e] = __builtin_fmaf(sacc[m2 * 8 + e], a.scale_log2, b0[e] - m_run);
          sacc[m2 * 8 + 4 + e] = __builtin_fmaf(sacc[m2 * 8 + 4 + e], a.scale_log2, b1[e] - m_run);
        }
      }
    }
    float mx = sacc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    if (__builtin_amdgcn_ballot_w64(mx > 8.f || (fresh && mx > -__builtin_inff())) != 0ull) {
      const float mt = fmaxf(mx, xor32(mx));
      const bool raise = mt > 8.f || (fresh && mt > -__builtin_inff());
      const float delta = raise ? mt : 0.f;
      const float alpha = fresh ? 0.f : __builtin_amdgcn_exp2f(-delta);
      fresh = fresh && !raise;
      m_run += delta;
      l_run *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] -= delta;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
    }
    if (QUAD && PART) {
      // keys past Nk inside a group of this tile (rare): masked here, after
      // the reference update, which their logits (copies of a valid key's
      // logit in the same group) cannot have moved
      const uint32_t pmt = pmask_s[t];
      if (__builtin_amdgcn_readfirstlane(pmt) != 0u) {
        const uint32_t pm = pmt >> (8 * hh);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sacc[r] = ((pm >> (16 * (r >> 3) + (r & 7))) & 1u) ? -__builtin_inff() : sacc[r];
      }
    }
    bf16x8 pf[2];
    {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = __builtin_amdgcn_exp2f(sacc[r]);
      float rs[2];  // two shorter add chains
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w[e] = pack_bf16x2(sacc[8 * m + 2 * e], sacc[8 * m + 2 * e + 1]);
          const float pr = sacc[8 * m + 2 * e] + sacc[8 * m + 2 * e + 1];
          rs[m] = e == 0 ? pr : rs[m] + pr;
        }
        pf[m] = as_bf16x8(w);
      }
      l_run += rs[0] + rs[1];
    }
    // V^T fragments through the transposing LDS read
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      asm volatile("" : "+v"(voff[dt]));
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        s16x4 part[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          part[p] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4 *)(vt + voff[dt] + (16 * m + 4 * p) * ROWB));
        }
        const u32x2 w0 = __builtin_bit_cast(u32x2, part[0]);
        const u32x2 w1 = __builtin_bit_cast(u32x2, part[1]);
        const u32x4 w = {w0[0], w0[1], w1[0], w1[1]};
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(w), pf[m], oacc[dt], 0, 0, 0);
      }
    }
  };

  // One tile in slot S: wait for it (tile t+1 may still be in flight; the
  // barrier also means every wave is done with tile t-1), prefetch tile t+2
  // into the slot of tile t-1, compute.
  f32x16 sA;
  auto step = [&](auto slot_c, int t) {
    constexpr int S = decltype(slot_c)::value;
    constexpr int SN = (S + 2) % NBUF;
    const bool more = t + 2 < ntiles;
    int row[LPW], nvr[LPW], hrow[2 * LPW];
    if (HALF && more) rows_of_h(t + 2, hrow);
    else if (QUAD && more) rows_of(t + 2, row, nvr);
    if (t + 1 < ntiles) ring_barrier<LPT>();
    else ring_barrier<0>();
    if (more) {
      if constexpr (HALF) issue_rows_h(std::integral_constant<int, SN>(), hrow);
      else if constexpr (QUAD) issue_rows(std::integral_constant<int, SN>(), row, nvr);
      else issue(std::integral_constant<int, SN>(), t + 2);
    }
    qk(slot_c, sA);
    softmax_pv(slot_c, sA, t);
  };
  // Steady state of the group-shift path (tile t + 2 exists): the same step
  // without conditions, and with the backend's hint to interleave LDS reads
  // and matrix operations (1-2 % faster than the conditional step at the
  // Wan2.1-14B 720p shape).
  auto step_full = [&](auto slot_c, int t) {
    constexpr int S = decltype(slot_c)::value;
    __builtin_amdgcn_iglp_opt(0);
    constexpr int SN = (S + 2) % NBUF;
    int row[LPW], nvr[LPW], hrow[2 * LPW];
    if (HALF) rows_of_h(t + 2, hrow);
    else if (QUAD) rows_of(t + 2, row, nvr);
    ring_barrier<LPT>();
    if constexpr (HALF) issue_rows_h(std::integral_constant<int, SN>(), hrow);
    else if constexpr (QUAD) issue_rows(std::integral_constant<int, SN>(), row, nvr);
    else issue(std::integral_constant<int, SN>(), t + 2);
    qk(slot_c, sA);
    softmax_pv(slot_c, sA, t);
  };

  // A phase covers CAP list entries (per-key shifts) or CAPG groups of SG
  // keys (group shifts).
  const int per_phase = QUAD ? (CAPG * SG) >> a.kv_shift : CAP;
  for (int base = 0; base < cnt; base += per_phase) {
    const int pc = min(per_phase, cnt - base);
    pbase = base;
    pcnt = pc;
    nkeys = pc << a.kv_shift;
    ntiles = (nkeys + KT - 1) / KT;
    __syncthreads();
    if constexpr (QUAD) {
      // shift of every SG-key group of the phase's tiles, -inf for groups of
      // padded or invalid entries and wholly past Nk; a group crossing Nk
      // marks its rows past Nk
      if (PART) {
        for (int i = tid; i < ntiles; i += NW * 64) pmask_s[i] = 0u;
        __syncthreads();
      }
      const int ng = ntiles * (KT / SG);
      for (int g = tid; g < ng; g += NW * 64) {
        const int e = (SG * g) >> a.kv_shift;
        float bv = -__builtin_inff();
        if (e < pc) {
          const int blk = idx_row[base + e];
          if (blk >= 0 && blk < a.M) {
            const int k0 = (blk << a.kv_shift) + ((SG * g) & (kvb - 1));
            if (k0 < a.Nk) {
              bv = bias_row ? bias_row[base + e] * kLog2e : 0.f;
              if (PART && k0 + 4 > a.Nk) {
                const uint32_t past = (0xfu << (a.Nk - k0)) & 0xfu;
                atomicOr(&pmask_s[g >> 3], past << (4 * (g & 7)));
              }
            }
          }
        }
        gb_s[SG == 4 ? (g & ~7) | quad_pos(g & 7) : (g & ~15) | pair_pos(g & 15)] = bv;
      }
    } else {
      // entries covering whole tiles (list tail padded with masked entries)
      const int padded = min(CAP, ((ntiles * KT) >> a.kv_shift) + 1);
      for (int e = tid; e < padded; e += NW * 64) {
        int blk = e < pc ? idx_row[base + e] : -1;
        float bv = (e < pc && bias_row) ? bias_row[base + e] * kLog2e : 0.f;
        if (blk < 0 || blk >= a.M) {
          blk = 0;
          bv = -__builtin_inff();
        }
        idx_s[e] = blk;
        bias_s[e] = bv;
      }
    }
    __syncthreads();
    if (ntiles > 0) issue_any(std::integral_constant<int, 0>(), 0);
    if (ntiles > 1) issue_any(std::integral_constant<int, 1>(), 1);
    int t = 0;
    // the per-key path keeps the conditional step: unconditional steps (with or
    // without the hint) made it 13 % slower at KV block 2
    if constexpr (QUAD) for (; t + 4 < ntiles; t += 3) {
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

  // ---- normalise and store (the lane halves hold different keys of the
  // same query: their maxima agree, their partial sums add up)
  const float l = l_run + xor32(l_run);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (qrow < a.Nq) {
    uint16_t *orow = a.out + ((size_t)bh * a.Nq + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w = {pack_bf16x2(oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv),
                   pack_bf16x2(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv)};
        *(u32x2 *)&orow[dt * 32 + g * 8 + hh * 4] = w;
      }
    if (a.lse && hh == 0)
      a.lse[(size_t)bh * a.Nq + qrow] = l > 0.f ? (m_run + __builtin_log2f(l)) * kLn2 : -__builtin_inff();
  }
}

int launch_attn_fwd(const void *q, const void *k, const void *v, int B, int H, int Nq, int Nk,
                    int d, int kv_block, const int32_t *idx, const float *bias,
                    const int32_t *count, int max_blocks, float scale, void *out, float *lse,
                    hipStream_t stream) {
  clear_pending_error();
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
  dim3 grid((unsigned)total), block(256);
  // Group shifts and the scalar gather need every wave load (4 rows at
  // d = 128, 8 at d = 64) inside one KV block: blocks of at least that many
  // keys.  Loads and groups crossing Nk are handled where they occur.
  const int rows_per_load = d == 128 ? 4 : 8;
  const bool quad = kv_block >= rows_per_load;
  const bool part = quad && Nk % rows_per_load != 0;
  // blocks of half a load: each half gathers one block; Nk must be a whole
  // number of blocks (a block crossing Nk takes the per-key path)
  const bool half = 2 * kv_block == rows_per_load && Nk % kv_block == 0 &&
                    (long long)Nk * d * 2 <= (1ll << 32);
  if (d == 128) {
    if (half) hipLaunchKernelGGL((attn_fwd_kernel<128, true, false, true>), grid, block, 0, stream, a);
    else if (part) hipLaunchKernelGGL((attn_fwd_kernel<128, true, true>), grid, block, 0, stream, a);
    else if (quad) hipLaunchKernelGGL((attn_fwd_kernel<128, true, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_fwd_kernel<128, false, false>), grid, block, 0, stream, a);
  } else {
    if (half) hipLaunchKernelGGL((attn_fwd_kernel<64, true, false, true>), grid, block, 0, stream, a);
    else if (part) hipLaunchKernelGGL((attn_fwd_kernel<64, true, true>), grid, block, 0, stream, a);
    else if (quad) hipLaunchKernelGGL((attn_fwd_kernel<64, true, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_fwd_kernel<64, false, false>), grid, block, 0, stream, a);
  }
  return status_of(hipGetLastError());
}

}  // namespace bsa
