// Forward block-pair attention kernels for gfx950.
//
// One workgroup owns a tile of query rows of one (batch, head) and walks the
// KV tiles of its job (one block pair, or a query block's shards in ring
// order) with an online softmax, then writes the normalised output and the
// row log-sum-exp.  The rescaling of a running (O, L) by a new block's
// partial is the FlashAttention-style merge the LV-XAttn review names
// ("What carries the argument"); seeding the state from an incoming
// (O_prev, LSE_prev) continues that merge inside the kernel.
//
// bf16 kernel: both contractions run on v_mfma_f32_16x16x32_bf16 (rather
// than 32x32x16: per FLOP it moves half the accumulator data through the
// register file, which the chip's power limit and the VALU work of the other
// wave on the SIMD both reward).  Each wave owns 32 query rows as two 16-row
// blocks and computes S^T = K Q^T (keys x queries), so that every lane holds
// scores of two query rows, 16 keys of each per 64-key tile; a row's other
// keys sit in three other lanes (a row max or sum takes two lane exchanges).
// The PV product is O^T = V^T P^T, whose B operand is the lane's own scores
// converted to bf16, and whose accumulator rows are rescaled by the lane's
// own factors.  V^T needs keys contiguous in the A operand: V tiles are
// staged row-major like K, and the operand is read with ds_read_b64_tr_b16,
// which hands each lane one column of a 4-row block (four keys of one head
// dim).
//
// The running maximum (the reference P is taken relative to) is only moved
// when some row's maximum grows by more than 8 (log2 units): until then
// probabilities are taken relative to the stale maximum and the O
// accumulator is not rescaled.  A tile's maximum is not even computed unless
// some lane's sum of P over the tile exceeds 2^16, so a P can reach 2^16
// (well inside fp32 and bf16 range).  Output and LSE are unchanged by this:
// O and l always share one reference.
//
// fp32 kernel: plain VALU arithmetic (fp32 products and sums), four lanes per
// query row; used for fp32 inputs where fp32-exact products are required.
#include "bwa_diag.h"
#include "common.h"

namespace bwa {

// ------------------------------------------------------------------ helpers

__device__ inline float wave_swap32_max(float x) {
  // v_permlane32_swap exchanges the upper half of one operand with the lower
  // half of the other; for a symmetric reduction both results combine lane l
  // with lane l^32 whichever way round they come back.
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float wave_swap32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// v_permlane16_swap does the same for lane l and lane l^16.
__device__ inline float wave_swap16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float wave_swap16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Number of leading keys of tile t that a query row may see: keys t.kt ..
// t.kt+lim-1 are visible (segment end t.ke; under causal masking only keys at
// or before the row's position).  Clamped to [0, bn].
//   causal == 1: rows and keys in sequence order, key j visible iff j <= row.
//   causal == 2: striped order over shards of blk rows (shard w holds
//     positions w, w+n, ...): the row at (shard w, index c) sees the first
//     c + 1 keys of shards <= w and the first c keys of later shards; a tile
//     lies inside one segment, which starts at the start t.s0 of shard t.sk,
//     so the tile's first key has index t.kt - t.s0 in that shard.
//     (row_w, row_c) is the row's (shard, index).
__device__ inline int visible_prefix(const TileIter& t, int causal, int64_t row, int bn,
                                     int64_t row_w, int64_t row_c) {
  int64_t lim = t.ke - t.kt;
  if (causal == 1 && row + 1 - t.kt < lim) lim = row + 1 - t.kt;
  if (causal == 2) {
    const int64_t see = row_c + (t.sk <= row_w ? 1 : 0) - (t.kt - t.s0);
    if (see < lim) lim = see;
  }
  return (int)(lim < 0 ? 0 : (lim > bn ? bn : lim));
}

// Materialise a value here: an empty volatile asm that claims to read and
// modify it.  Used to keep a phase's results from being sunk past a barrier
// into the next phase, and to settle outstanding loads of a register at a
// chosen point (the wait-count pass places the wait before the asm).
template <typename T>
__device__ inline void pin(T& x) {
  asm volatile("" : "+v"(x));
}

// Growth of a row maximum (log2 units) tolerated before the O accumulator is rescaled.
constexpr float kLazyRescale = 8.f;
// Largest sum of one lane's P over a tile (relative to the row's reference)
// accepted without looking at the tile's maximum.  Beyond it some P exceeds
// 2^11, so the maximum has grown by more than kLazyRescale and the reference
// is moved.
constexpr float kFastGrowth = 65536.f;

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  bf16 x = (bf16)a, y = (bf16)b;  // round to nearest even (v_cvt_pk_bf16_f32)
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// Store 4 consecutive output elements (fp32 accumulator values) to dtype T.
template <typename T>
__device__ inline void store4(T* dst, float a, float b, float c, float d);
template <>
__device__ inline void store4<float>(float* dst, float a, float b, float c, float d) {
  *(f32x4*)dst = f32x4{a, b, c, d};
}
template <>
__device__ inline void store4<bf16>(bf16* dst, float a, float b, float c, float d) {
  *(u32x2*)dst = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}

// ------------------------------------------------------------------ bf16 MFMA kernel
//
// 256 query rows per workgroup, 8 waves of 32 rows, 64-key tiles.  A wave's
// work per tile alternates between an MFMA phase (PV of tile j followed by S
// of tile j+1) and a VALU phase (mask, exp2, row sums and the bf16 P of tile
// j+1; the row maximum only when P grows past the bound below).  Waves 0-3 (group A) and 4-7 (group B) share the four SIMDs one
// each and run one phase apart: between any two barriers one wave of every
// SIMD is in its MFMA phase while the other is in its VALU phase, so that
// the matrix core and the vector ALU can work at the same time.  Barrier intervals
// ("slots") are numbered from 0; group A runs
//   slot 0: S(0);  slot 2j+1: softmax(j), load K(j+3);  slot 2j+2: PV(j) + S(j+1)
// and group B runs the same sequence one slot later (loading V(j+3) in its
// softmax slot).  K/V tiles rotate through four LDS buffers (tile j in buffer
// j mod 4) and move from global memory to LDS directly (global_load_lds, no
// registers).  Tile j's K is read in slots 2j and 2j+1 and its V in slots
// 2j+2 and 2j+3, so K(j+3) may land in slot 2j+1 (K(j-1) was last read in
// slot 2j-1) and V(j+3) in slot 2j+2 (V(j-1) last read in slot 2j+1).  A
// group waits for its loads of tile j+1 in its next softmax slot (those of
// tile j+2 may stay in flight), before the barrier after which the tile is
// read.

template <int D_>
struct Bf16Fwd {
  static constexpr int D = D_, NW = 8, NT = 512, BM = 256, BN = 64;
  // K and V tiles go from global memory straight to LDS, one 1 KB block (RPB
  // rows of ROWB bytes) per wave and load instruction, so rows are unpadded
  // inside a block and blocks are padded by 32 bytes (byte stride BS).  Key
  // order in a tile is permuted (kperm below) so that the eight rows read
  // together lie in eight blocks, 32 bytes apart in the bank space: K by
  // ds_read_b128 (eight lanes at a time, one row each), V by
  // ds_read_b64_tr_b16 (32 lanes at a time over 8 rows x 32 bytes).
  static constexpr int ROWB = 2 * D, RPB = 1024 / ROWB, NBK = BN / RPB, NBH = NBK / 2;
  static constexpr int BS = 1024 + 32;
  static constexpr int K_TILE = NBK * BS, V_TILE = NBK * BS;  // bytes
  static constexpr int STAGE = K_TILE + V_TILE;
  static constexpr int NBUF = 4;
  static constexpr int KC = NBK / 4;  // blocks per wave and tile (four waves per group)
  static_assert(NBH * RPB == 32 && KC * 4 == NBK && NBH >= 4, "tile geometry");
};

// Storage of row m (0..15) of 16-key block kb (0..3) of a tile: block
// (m mod NBH) + NBH (kb mod 2), row m / NBH + (16 / NBH) (kb / 2); kperm is its
// key offset in the tile (RPB rows per block, in order).
template <int D>
__device__ constexpr int kperm(int kb, int m) {
  using C = Bf16Fwd<D>;
  return C::RPB * (m % C::NBH + C::NBH * (kb % 2)) + m / C::NBH + (16 / C::NBH) * (kb / 2);
}

// ---- phase clock of the bf16 kernel's loop.  Compiled in only when the
// library is built with BWA_SLOT_TIMERS=1 (the diagnostic build); otherwise
// every member is empty and the kernel is unchanged.  Wave 0 (group A) and
// wave 4 (group B) sum s_memtime deltas (shader clock cycles) over the tiles
// they walk: [0] VALU phase (mask, exponentials, row sums, bf16 P), [1] the
// staging step (wait for the landed tile, issue the next tile's direct
// loads), [2] the barrier that opens the MFMA slot, [3] the MFMA phase (PV
// of this tile, S of the next), [4] the barrier that closes it; [5] counts
// the tiles.  Workgroup w < kSlotRecords writes its two records to
// fwd_slot_rec[w] at the end (group A then group B); every launch clears the
// array first.  A stamp is a scalar memory read whose result arrives later,
// so stamps are only used after the next opening barrier (whose lgkmcnt(0)
// has waited for them) and a tile's deltas are summed one tile late.  The
// five stamps per tile still slow the loop down (measured at 2048 x 131072,
// split mode: one stamp per tile costs nothing, two taken after the barriers
// about 2%, all five 13-16%), so the phases are those of a slightly slower
// kernel; the diagnostic summary reports both builds' step times.
#ifndef BWA_SLOT_TIMERS
#define BWA_SLOT_TIMERS 0
#endif
[[maybe_unused]] constexpr int kSlotRecords = BWA_SLOT_RECORDS;
[[maybe_unused]] constexpr int kSlotFields = BWA_SLOT_FIELDS;
#if BWA_SLOT_TIMERS
__device__ long long fwd_slot_rec[kSlotRecords][2][kSlotFields];
#endif

struct PhaseClock {
#if BWA_SLOT_TIMERS
  // 32-bit stamps and sums (a workgroup's loop lasts far less than 2^32
  // cycles): fewer scalar registers live across the tile, so that no stamp
  // has to be moved out of its register (which would wait for it) before the
  // opening barrier.
  uint32_t acc[kSlotFields] = {0, 0, 0, 0, 0, 0};
  // e[i]: stamp after phase i of the current tile (e[4]: of the previous tile
  // until this tile's closing barrier); e1_prev: e[1] of the previous tile
  uint32_t e[5] = {0, 0, 0, 0, 0};
  uint32_t e1_prev = 0;
  bool open = false;  // e[2..4] hold a tile whose last three deltas are unsummed
  static __device__ uint32_t now() { return (uint32_t)__builtin_amdgcn_s_memtime(); }
  __device__ void start() { e[4] = now(); }
  __device__ void after_valu() { e[0] = now(); }
  __device__ void after_staging() { e[1] = now(); }
  // right after the opening barrier: every stamp taken before it has arrived
  __device__ void after_open() {
    close_previous();
    acc[0] += e[0] - e[4];
    acc[1] += e[1] - e[0];
    e1_prev = e[1];
    open = true;
    e[2] = now();
  }
  __device__ void after_mfma() { e[3] = now(); }
  __device__ void after_close() {
    e[4] = now();
    acc[kSlotFields - 1] += 1;
  }
  __device__ void close_previous() {
    if (!open) return;
    acc[2] += e[2] - e1_prev;
    acc[3] += e[3] - e[2];
    acc[4] += e[4] - e[3];
    open = false;
  }
  __device__ void store(int wave, int lane) {
    close_previous();
    if (lane != 0 || (wave != 0 && wave != 4) || blockIdx.x >= kSlotRecords) return;
    long long* rec = fwd_slot_rec[blockIdx.x][wave == 4];
    for (int i = 0; i < kSlotFields; ++i) rec[i] = acc[i];
  }
#else
  __device__ void start() {}
  __device__ void after_valu() {}
  __device__ void after_staging() {}
  __device__ void after_open() {}
  __device__ void after_mfma() {}
  __device__ void after_close() {}
  __device__ void store(int, int) {}
#endif
};

// CM: the causal order (0 none, 1 sequence, 2 striped), a template argument so
// that each instance carries only its own mask code.
template <int D_, int CM>
__global__ __launch_bounds__(512) void fwd_bf16_kernel(FwdParams p) {
  using C = Bf16Fwd<D_>;
  constexpr int D = C::D, BN = C::BN, NKB = BN / 16, NKK = BN / 32, NKS = D / 32, NDB = D / 16;
  __shared__ __attribute__((aligned(16))) char smem[C::NBUF * C::STAGE];

  Job jb;
  if (!make_job(p, C::BM, &jb)) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  // Lane layout of the 16x16x32 blocks: lane l has column l16 = l % 16 and
  // quarter q4 = l / 16.  A wave's 32 query rows are two 16-row blocks qb; the
  // lane owns row wrow0 + 16 qb + l16 of each.  A score block (16 keys x 16
  // rows) gives the lane rows 4 q4 + r (r = 0..3) of key block kb, keys
  // kperm(kb, 4 q4 + r); the row's other keys sit in lanes l16 + 16 q.
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const bool groupB = wave >= 4;
  const int b = jb.bh / p.H, h = jb.bh % p.H;
  const bf16* qg = (const bf16*)p.q + b * p.sqB + h * p.sqH;
  const bf16* kg = (const bf16*)p.k + b * p.skB + h * p.skH;
  const bf16* vg = (const bf16*)p.v + b * p.svB + h * p.svH;

  const int64_t wrow0 = jb.r0 + wave * 32;
  int64_t myrow[2], row_w[2], row_c[2];
  bool row_ok[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    myrow[qb] = wrow0 + 16 * qb + l16;
    row_ok[qb] = myrow[qb] < jb.r1;
    row_w[qb] = CM == 2 ? myrow[qb] / p.blk : 0;  // striped: shard, index
    row_c[qb] = CM == 2 ? myrow[qb] - row_w[qb] * p.blk : 0;
  }
  // B operand of S^T = K Q^T: Q row 16 qb + l16, head dims 32 ks + 8 q4 ..
  bf16x8 qreg[2][NKS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qreg[qb][ks] = row_ok[qb] ? *(const bf16x8*)(qg + myrow[qb] * p.sqS + 32 * ks + 8 * q4) : bf16x8{};

  // O^T blocks (16 head dims x 16 rows): the lane holds dims 16 db + 4 q4 + r
  // of its row of block qb
  float m2[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};
  f32x4 oacc[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db][0] = oacc[db][1] = f32x4{};
  const int64_t BH = (int64_t)p.B * p.H;
  if (jb.epi == EPI_ACC && jb.acc_in) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float lp = row_ok[qb] ? p.lse[jb.bh * p.SQ + myrow[qb]] : -INFINITY;
      if (lp != -INFINITY) {
        m2[qb] = lp * kLog2e;
        lsum[qb] = (q4 == 0) ? 1.f : 0.f;
        const float* src = p.o_acc + (jb.bh * p.SQ + myrow[qb]) * D + 4 * q4;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db][qb] = *(const f32x4*)(src + 16 * db);
      }
    }
  }

  TileIter tv;  // tile of the next softmax phase
  tv.seek(p, jb, 0, BN);
  if (!tv.valid(jb) && jb.epi == EPI_ACC && jb.acc_in) return;  // skipped pair

  // staging: group A moves K tiles, group B moves V tiles, global memory to
  // LDS directly.  Wave wg of a group loads blocks KC wg .. KC wg + KC-1 of a
  // tile; lane l moves 16 bytes: row l / (D/8) of the block, column chunk
  // l % (D/8).  Row offsets fit in 24-bit products (row strides are below
  // 16 MiB, checked on the host).
  const bf16* ssrc = groupB ? vg : kg;
  const int64_t sstr = groupB ? p.svS : p.skS;
  const int soff = groupB ? C::K_TILE : 0;
  const int wg = wave & 3;
  const int drow = lane / (D / 8), dcol = (lane % (D / 8)) * 16;
  const uint32_t sstr2 = (uint32_t)(sstr * 2);  // row stride in bytes, < 2^24
  // the lane's byte offsets from a tile's first row, one per block it loads
  uint32_t doff[C::KC];
#pragma unroll
  for (int i = 0; i < C::KC; ++i)
    doff[i] = __umul24((uint32_t)((C::KC * wg + i) * C::RPB + drow), sstr2) + (uint32_t)dcol;
  // Load the tile at key t.kt into LDS buffer buf.  In a tile that ends
  // early, rows at or past the segment end repeat its last key (their scores
  // are masked, their P is zero and the repeated V row is finite).
  auto dma_tile = [&](const TileIter& t, int buf) {
    const int lim = (int)min(t.ke - t.kt, (int64_t)BN);
    const bf16* base = ssrc + t.kt * sstr;
    const uint32_t lds = lds_addr(smem) + buf * C::STAGE + soff + C::KC * wg * C::BS;
    if (lim == BN) {
#pragma unroll
      for (int i = 0; i < C::KC; ++i) dma16(base, doff[i], lds + i * C::BS);
    } else {
#pragma unroll
      for (int i = 0; i < C::KC; ++i) {
        const int r = min((C::KC * wg + i) * C::RPB + drow, lim - 1);
        dma16(base, __umul24((uint32_t)r, sstr2) + (uint32_t)dcol, lds + i * C::BS);
      }
    }
  };

  // Scores of the tile: sacc[kb][qb] element r is key kperm(kb, 4 q4 + r) of
  // the lane's row in block qb.  PV contracts over 32 keys per MFMA; its k
  // positions 8 q4 + (0..3) and 8 q4 + (4..7) are taken as the keys of
  // blocks 2 kk and 2 kk + 1 that the lane holds, so that the B operand P^T
  // is the lane's own scores, and V^T is read in the same order.
  f32x4 sacc[NKB][2];
  bf16x8 pb[NKK][2];
  // K operand: lane (l16, q4) reads row l16 of key block kb, columns 32 ks + 8 q4 ..
  const int kbase = (l16 % C::NBH) * C::BS + (l16 / C::NBH) * C::ROWB + 16 * q4;
  auto phase_s = [&](int buf) {
    const char* ks_ = smem + buf * C::STAGE + kbase;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 a = *(const bf16x8*)(ks_ + C::NBH * (kb % 2) * C::BS +
                                          (16 / C::NBH) * (kb / 2) * C::ROWB + 64 * ks);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          sacc[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              a, qreg[qb][ks], ks == 0 ? f32x4{} : sacc[kb][qb], 0, 0, 0);
      }
  };
  // V^T operand of key half kk and head-dim block db: a transposing read
  // hands lane l16 of quarter q4 head dim 16 db + l16 of rows 4 q4 + (0..3) of
  // key block 2 kk (lo) and 2 kk + 1 (hi); the 16 lanes address the four rows
  // li / 4 (li = l16), columns 4 (li % 4).
  const int vm = 4 * q4 + (l16 >> 2);
  const int vbase = C::K_TILE + (vm % C::NBH) * C::BS + (vm / C::NBH) * C::ROWB + 8 * (l16 & 3);
  auto phase_pv = [&](int buf) {
    const char* vt_s = smem + buf * C::STAGE + vbase;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const char* a0 = vt_s + (16 / C::NBH) * kk * C::ROWB + 32 * db;
        s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0));
        s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0 + C::NBH * C::BS));
        u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[kk][qb], oacc[db][qb], 0, 0, 0);
      }
  };
  const float c2 = p.scale_log2;
  auto phase_softmax = [&](const TileIter& t) {
    bool need_mask = (t.kt + BN > t.ke) || (CM == 1 && t.kt + BN - 1 > wrow0);
    if constexpr (CM == 2)
      need_mask = __builtin_amdgcn_ballot_w64(
                      visible_prefix(t, 2, myrow[0], BN, row_w[0], row_c[0]) < BN ||
                      visible_prefix(t, 2, myrow[1], BN, row_w[1], row_c[1]) < BN) != 0;
    if (need_mask) {
      // the part of the key that depends on q4 is moved to the limit
      const int gk = kperm<D>(0, 4 * q4) - kperm<D>(0, 0);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int lim =
            visible_prefix(t, CM, myrow[qb], BN, row_w[qb], row_c[qb]) - gk;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kperm<D>(kb, r) >= lim) sacc[kb][qb][r] = -INFINITY;
      }
    }
    // P relative to references m[qb] (log2 units) into pb; ts[qb] is this
    // lane's sum of it
    auto exp_tile = [&](const float* m, float* ts) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float s2[2] = {0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          bf16x8 x;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float pv = fast_exp2(__builtin_fmaf(sacc[2 * kk + e / 4][qb][e % 4], c2, -m[qb]));
            s2[e & 1] += pv;
            x[e] = (bf16)pv;
          }
          pb[kk][qb] = x;
        }
        ts[qb] = s2[0] + s2[1];
      }
    };
    // Common case: every row of the wave has a reference and no P of this
    // tile exceeds kFastGrowth (checked through the lane's sums of P), so the
    // tile's maximum is not needed.  Otherwise the maximum is taken, the
    // reference moved if it grew by more than kLazyRescale, and P recomputed.
    bool slow = __builtin_amdgcn_ballot_w64(m2[0] == -INFINITY || m2[1] == -INFINITY) != 0;
    float ts[2] = {0.f, 0.f};
    if (!slow) {
      exp_tile(m2, ts);
      slow = __builtin_amdgcn_ballot_w64(!(ts[0] <= kFastGrowth) || !(ts[1] <= kFastGrowth)) != 0;
    }
    if (slow) {
      float m_cand[2];
      bool grow = false;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[kb][qb][r]);
        mx = wave_swap32_max(wave_swap16_max(mx));
        m_cand[qb] = fmaxf(m2[qb], mx * c2);
        grow = grow || (m_cand[qb] > m2[qb] + kLazyRescale);
      }
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float alpha = fast_exp2(m2[qb] - ((m_cand[qb] == -INFINITY) ? 0.f : m_cand[qb]));
          lsum[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db) oacc[db][qb] *= alpha;
          m2[qb] = m_cand[qb];
        }
      }
      const float m_use[2] = {(m2[0] == -INFINITY) ? 0.f : m2[0], (m2[1] == -INFINITY) ? 0.f : m2[1]};
      exp_tile(m_use, ts);
    }
    lsum[0] += ts[0];
    lsum[1] += ts[1];
  };

  // ---- prologue: tile 0 into buffer 0, tiles 1 and 2 in flight.  A job
  // without visible tiles skips the prologue and the loop altogether (the
  // condition is uniform over the workgroup), so both groups always pass the
  // same barriers.
  TileIter tw = tv;  // next tile this thread's group loads
  int issued = 0;    // tiles loaded so far (tile i into buffer i mod NBUF)
  PhaseClock clk;
  if (tv.valid(jb)) {
    for (int i = 0; i < 3 && tw.valid(jb); ++i) {
      dma_tile(tw, i);
      tw.advance(p, jb, BN);
      ++issued;
    }
    // tile 0 has landed; the loads of the tiles after it may still be in flight
    if (issued == 3) wait_vm<2 * C::KC>();
    else if (issued == 2) wait_vm<C::KC>();
    else wait_vm<0>();
    slot_barrier();
    if (!groupB) {
      phase_s(0);  // slot 0
      slot_barrier();
    } else {
      slot_barrier();  // slot 0: idle
      phase_s(0);      // slot 1
      slot_barrier();
    }
    // Settle the prologue's global loads (Q, the carried accumulator) here: the
    // wait-count pass cannot tell that the loop's first MFMAs already waited for
    // them, and would otherwise wait on every tile's staging loads as well.
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      pin(qreg[0][ks]);
      pin(qreg[1][ks]);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      pin(oacc[db][0]);
      pin(oacc[db][1]);
    }
    int j = 0;
    clk.start();
    while (tv.valid(jb)) {
      const int cur = j % C::NBUF, nxt = (j + 1) % C::NBUF;
      phase_softmax(tv);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        pin(pb[kk][0]);
        pin(pb[kk][1]);
      }
      pin(lsum[0]);
      pin(lsum[1]);
      clk.after_valu();
      // tile j+1 has landed (published by the barrier below; tile j+2 may still
      // be in flight); load tile j+3
      if (issued > j + 2) wait_vm<C::KC>();
      else wait_vm<0>();
      if (tw.valid(jb)) {
        dma_tile(tw, (j + 3) % C::NBUF);
        tw.advance(p, jb, BN);
        ++issued;
      }
      clk.after_staging();
      slot_barrier();
      clk.after_open();
      TileIter tn = tv;
      tn.advance(p, jb, BN);
      phase_pv(cur);
      if (tn.valid(jb)) phase_s(nxt);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        pin(sacc[kb][0]);
        pin(sacc[kb][1]);
      }
      clk.after_mfma();
      // group A closes this slot; group B's last MFMA slot is the final one
      if (!groupB || tn.valid(jb)) slot_barrier();
      clk.after_close();
      tv = tn;
      ++j;
    }
  }  // tv.valid(jb)
  clk.store(wave, lane);

  // ---- epilogue: a row's sum is spread over the four lanes of its column
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float ltot = wave_swap32_sum(wave_swap16_sum(lsum[qb]));
    const bool empty = (m2[qb] == -INFINITY) || !(ltot > 0.f);
    const float inv = empty ? 0.f : 1.f / ltot;
    const float lse = empty ? -INFINITY : (m2[qb] + __log2f(ltot)) * kLn2;
    if (!row_ok[qb]) continue;
    if (jb.epi == EPI_FINAL) {
      bf16* dst = (bf16*)p.o + b * p.soB + h * p.soH + myrow[qb] * p.soS + 4 * q4;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        store4<bf16>(dst + 16 * db, oacc[db][qb][0] * inv, oacc[db][qb][1] * inv,
                     oacc[db][qb][2] * inv, oacc[db][qb][3] * inv);
      if (q4 == 0) p.lse[jb.bh * p.SQ + myrow[qb]] = lse;
    } else {
      float* obase = p.o_acc;
      float* lbase = p.lse;
      if (jb.epi == EPI_PART) {
        obase += (int64_t)jb.block * BH * p.SQ * D;
        lbase = p.lse_part + (int64_t)jb.block * BH * p.SQ;
      }
      float* dst = obase + (jb.bh * p.SQ + myrow[qb]) * D + 4 * q4;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        store4<float>(dst + 16 * db, oacc[db][qb][0] * inv, oacc[db][qb][1] * inv,
                      oacc[db][qb][2] * inv, oacc[db][qb][3] * inv);
      if (q4 == 0) lbase[jb.bh * p.SQ + myrow[qb]] = lse;
    }
  }
}

// ------------------------------------------------------------------ fp32 VALU kernel

// x of the lane that DPP control CTRL selects (every lane active)
template <int CTRL>
__device__ inline float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

template <int D>
struct F32Fwd {
  static constexpr int BN = 32;    // keys per tile
  static constexpr int LPR = 16;   // lanes per query row (one DPP row)
  static constexpr int BM = 16;    // query rows per workgroup
  static constexpr int NT = BM * LPR;
  static constexpr int DL = D / LPR;  // dims per lane
  static constexpr int KS = D + 4;    // LDS row stride (floats)
};

template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdParams p) {
  using C = F32Fwd<D>;
  constexpr int BN = C::BN, DL = C::DL, KS = C::KS;
  __shared__ __attribute__((aligned(16))) float Ks[BN * KS];
  __shared__ __attribute__((aligned(16))) float Vs[BN * KS];

  Job jb;
  if (!make_job(p, C::BM, &jb)) return;
  const int tid = threadIdx.x;
  const int sub = tid % C::LPR;  // which DL dims of the row this lane owns
  const int64_t myrow = jb.r0 + tid / C::LPR;
  const bool row_ok = myrow < jb.r1;
  const int64_t row_w = p.causal == 2 ? myrow / p.blk : 0;  // striped: shard, index
  const int64_t row_c = p.causal == 2 ? myrow - row_w * p.blk : 0;
  const int b = jb.bh / p.H, h = jb.bh % p.H;
  const float* qg = (const float*)p.q + b * p.sqB + h * p.sqH;
  const float* kg = (const float*)p.k + b * p.skB + h * p.skH;
  const float* vg = (const float*)p.v + b * p.svB + h * p.svH;

  float qv[DL], acc[DL];
#pragma unroll
  for (int e = 0; e < DL; ++e) {
    qv[e] = row_ok ? qg[myrow * p.sqS + sub * DL + e] : 0.f;
    acc[e] = 0.f;
  }
  float m2 = -INFINITY, l = 0.f;
  const int64_t BH = (int64_t)p.B * p.H;
  if (jb.epi == EPI_ACC && jb.acc_in) {
    float lp = row_ok ? p.lse[jb.bh * p.SQ + myrow] : -INFINITY;
    if (lp != -INFINITY) {
      m2 = lp * kLog2e;
      l = 1.f;
      const float* src = p.o_acc + (jb.bh * p.SQ + myrow) * D + sub * DL;
#pragma unroll
      for (int e = 0; e < DL; ++e) acc[e] = src[e];
    }
  }

  TileIter it;
  it.seek(p, jb, 0, BN);
  if (!it.valid(jb) && jb.epi == EPI_ACC && jb.acc_in) return;
  const float c2 = p.scale_log2;
  // Staging: thread tid moves 16-byte chunks tid + i NT (i < NCH) of a tile's
  // K and V (row c / (D/4), column chunk c % (D/4)); keys at or past the
  // segment end are zero.  The next tile's chunks are loaded into registers
  // while the current tile is computed.
  constexpr int NCH = BN * D / 4 / C::NT;
  static_assert(NCH * C::NT == BN * D / 4, "staging split");
  f32x4 kx[NCH], vx[NCH];
  auto load = [&](const TileIter& t) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * C::NT, row = c / (D / 4), col4 = c % (D / 4);
      const int64_t key = t.kt + row;
      kx[i] = key < t.ke ? *(const f32x4*)(kg + key * p.skS + col4 * 4) : f32x4{};
      vx[i] = key < t.ke ? *(const f32x4*)(vg + key * p.svS + col4 * 4) : f32x4{};
    }
  };
  // sum over the 16 lanes of a row (one DPP row): lane pairs l^1 and l^2
  // (quad permutations), then l <-> 7-l within each half row and l <-> 15-l;
  // each step adds two equal-by-construction partial sums, so every lane of
  // the row ends with the same bits
  auto row_sum = [](float x) {
    x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_f32<0x141>(x);  // row_half_mirror
    return x + dpp_f32<0x140>(x);  // row_mirror
  };
  if (it.valid(jb)) load(it);
  while (it.valid(jb)) {
    // keys it.kt + j, j < lim, are visible to this row
    const int lim = visible_prefix(it, p.causal, myrow, BN, row_w, row_c);
    __syncthreads();  // every read of the previous tile is done
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * C::NT, row = c / (D / 4), col4 = c % (D / 4);
      *(f32x4*)(Ks + row * KS + col4 * 4) = kx[i];
      *(f32x4*)(Vs + row * KS + col4 * 4) = vx[i];
    }
    __syncthreads();
    TileIter nx = it;
    nx.advance(p, jb, BN);
    if (nx.valid(jb)) load(nx);
    // one key at a time: score, then the online-softmax update of (m, l,
    // acc).  A key at or past lim leaves them exactly as they are (alpha = 1,
    // p = 0); selects rather than a branch let the unrolled keys overlap.
#pragma unroll 8
    for (int j = 0; j < BN; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < DL; ++e) dot = __builtin_fmaf(qv[e], Ks[j * KS + sub * DL + e], dot);
      dot = row_sum(dot);
      const bool vis = j < lim;
      const float t = vis ? dot * c2 : -INFINITY;
      const float m_new = fmaxf(m2, t);
      const float alpha = vis ? fast_exp2(m2 - m_new) : 1.f;
      const float pj = vis ? fast_exp2(t - m_new) : 0.f;
      m2 = m_new;
      l = l * alpha + pj;
#pragma unroll
      for (int e = 0; e < DL; ++e)
        acc[e] = __builtin_fmaf(pj, Vs[j * KS + sub * DL + e], acc[e] * alpha);
    }
    it = nx;
  }

  const bool empty = (m2 == -INFINITY) || !(l > 0.f);
  const float inv = empty ? 0.f : 1.f / l;
  const float lse = empty ? -INFINITY : (m2 + __log2f(l)) * kLn2;
  if (!row_ok) return;
  float* dst;
  float* ldst;
  if (jb.epi == EPI_FINAL) {
    dst = (float*)p.o + b * p.soB + h * p.soH + myrow * p.soS;
    ldst = p.lse;
  } else if (jb.epi == EPI_ACC) {
    dst = p.o_acc + (jb.bh * p.SQ + myrow) * D;
    ldst = p.lse;
  } else {
    dst = p.o_acc + ((int64_t)jb.block * BH * p.SQ + jb.bh * p.SQ + myrow) * D;
    ldst = p.lse_part + (int64_t)jb.block * BH * p.SQ;
  }
#pragma unroll
  for (int e = 0; e < DL; e += 4)
    store4<float>(dst + sub * DL + e, acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv,
                  acc[e + 3] * inv);
  if (sub == 0) ldst[jb.bh * p.SQ + myrow] = lse;
}

// ------------------------------------------------------------------ launchers

// Query rows per workgroup for a dtype / head dim.
int fwd_tile_rows(int dtype_bf16, int D) {
  (void)D;
  return dtype_bf16 ? Bf16Fwd<128>::BM : F32Fwd<128>::BM;
}

// Launch one forward pass over p.groups x p.tiles workgroups.
hipError_t fwd_launch(FwdParams p, int dtype_bf16, hipStream_t st) {
  const int blocks = xcd_grid_size(p.tiles, p.groups);
  if (blocks == 0) return hipSuccess;
#if BWA_SLOT_TIMERS
  if (dtype_bf16) {
    void* rec = nullptr;
    hipError_t e = hipGetSymbolAddress(&rec, HIP_SYMBOL(fwd_slot_rec));
    if (e == hipSuccess) e = hipMemsetAsync(rec, 0, sizeof(fwd_slot_rec), st);
    if (e != hipSuccess) return e;
  }
#endif
  if (dtype_bf16) {
    const dim3 g(blocks), b128(Bf16Fwd<128>::NT), b64(Bf16Fwd<64>::NT);
    if (p.D == 128) {
      if (p.causal == 2) hipLaunchKernelGGL((fwd_bf16_kernel<128, 2>), g, b128, 0, st, p);
      else if (p.causal == 1) hipLaunchKernelGGL((fwd_bf16_kernel<128, 1>), g, b128, 0, st, p);
      else hipLaunchKernelGGL((fwd_bf16_kernel<128, 0>), g, b128, 0, st, p);
    } else {
      if (p.causal == 2) hipLaunchKernelGGL((fwd_bf16_kernel<64, 2>), g, b64, 0, st, p);
      else if (p.causal == 1) hipLaunchKernelGGL((fwd_bf16_kernel<64, 1>), g, b64, 0, st, p);
      else hipLaunchKernelGGL((fwd_bf16_kernel<64, 0>), g, b64, 0, st, p);
    }
  } else {
    if (p.D == 128)
      hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3(blocks), dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3(blocks), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace bwa

extern "C" int bwa_fwd_slot_timers(long long* out, int64_t max_records, int64_t* n_records) {
  if (!out || !n_records || max_records < 0) return BWA_ERR_INVALID_ARG;
#if BWA_SLOT_TIMERS
  const int64_t n = max_records < bwa::kSlotRecords ? max_records : bwa::kSlotRecords;
  *n_records = bwa::kSlotRecords;
  if (hipDeviceSynchronize() != hipSuccess) return BWA_ERR_HIP;
  if (n > 0 && hipMemcpyFromSymbol(out, HIP_SYMBOL(bwa::fwd_slot_rec),
                                   n * 2 * bwa::kSlotFields * sizeof(long long), 0,
                                   hipMemcpyDeviceToHost) != hipSuccess)
    return BWA_ERR_HIP;
  return BWA_OK;
#else
  *n_records = 0;
  return BWA_ERR_UNSUPPORTED;
#endif
}
