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
// bf16 kernel: both contractions run on v_mfma_f32_32x32x16_bf16.  Each wave
// owns 32 query rows and computes S^T = K Q^T (keys x queries) so that every
// lane holds one query's scores: row max / sum are in-lane reductions plus one
// exchange with lane l^32.  The PV product is O^T = V^T P^T, whose B operand
// is exactly the lane's own scores converted to bf16, and whose accumulator
// rows are rescaled by the lane's own factor.  V^T needs keys contiguous in
// the A operand: V tiles are staged row-major like K, and the operand is read
// with ds_read_b64_tr_b16, which hands each lane one column of a 4-row block
// (four keys of one head dim).
//
// The running maximum is only moved when some row's maximum grows by more
// than 2^8 (log2 units): until then probabilities are taken relative to the
// stale maximum (they stay <= 256, exact in fp32 and bf16 range), and the
// O accumulator is not rescaled.  Output and LSE are unchanged by this: O and
// l always share one reference maximum.
//
// fp32 kernel: plain VALU arithmetic (fp32 products and sums), four lanes per
// query row; used for fp32 inputs where fp32-exact products are required.
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

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Number of leading keys of a tile starting at key kt that a query row may see:
// keys kt .. kt+lim-1 are visible (segment end ke; under causal masking only
// keys at or before the row's position).  Clamped to [0, bn].
//   causal == 1: rows and keys in sequence order, key j visible iff j <= row.
//   causal == 2: striped order over shards of blk rows (shard w holds
//     positions w, w+n, ...): the row at (shard w, index c) sees the first
//     c + 1 keys of shards <= w and the first c keys of later shards; a tile
//     lies inside one shard (ks, starting at index c0).  (row_w, row_c) is the
//     row's (shard, index).
__device__ inline int visible_prefix(int64_t kt, int64_t ke, int causal, int64_t row, int bn,
                                     int64_t blk, int64_t row_w, int64_t row_c) {
  int64_t lim = ke - kt;
  if (causal == 1 && row + 1 - kt < lim) lim = row + 1 - kt;
  if (causal == 2) {
    const int64_t ks = kt / blk, c0 = kt - ks * blk;
    const int64_t see = row_c + (ks <= row_w ? 1 : 0) - c0;
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
// of tile j+1) and a VALU phase (mask, max, exp2, row sums and the bf16 P of
// tile j+1).  Waves 0-3 (group A) and 4-7 (group B) share the four SIMDs one
// each and run one phase apart: between any two barriers one wave of every
// SIMD is in its MFMA phase while the other is in its VALU phase, so the
// matrix core and the vector ALU work at the same time.  Barrier intervals
// ("slots") are numbered from 0; group A runs
//   slot 0: S(0);  slot 2j+1: softmax(j) + write K(j+1);  slot 2j+2: PV(j) + S(j+1)
// and group B runs the same sequence one slot later (writing V(j+1) in its
// softmax slot).  K/V tiles rotate through three LDS buffers; a tile is read
// from slot 2j to slot 2j+3 and the buffer it overwrites was last read two
// slots earlier.  Each thread of a group stages KC 16-byte chunks of a tile:
// loaded from global memory one softmax slot ahead, written to LDS in the next.

template <int D_>
struct Bf16Fwd {
  static constexpr int D = D_, NW = 8, NT = 512, BM = 256, BN = 64;
  // Padded LDS row strides (elements).  K rows are read 16 bytes per lane by
  // ds_read_b128.  A transposing V read covers 8 rows x 64 bytes and is served
  // 32 lanes (4 rows) at a time from 64 banks of 4 bytes: rows 2*(D+32) bytes
  // apart land in distinct 64-byte quarters of the bank space (the stride is
  // 64 or 192 mod 256), so the read is conflict-free; D+16 would pair rows
  // on the same banks and halve the read rate.
  static constexpr int KS = D + 8, VS = D + 32;
  static constexpr int K_TILE = BN * KS, V_TILE = BN * VS;
  static constexpr int STAGE = K_TILE + V_TILE;
  static constexpr int NBUF = 3;
  static constexpr int GT = NT / 2;                // threads per group
  static constexpr int KC = (BN * D / 8) / GT;     // 16-byte chunks per staging thread
  static_assert(KC * GT == BN * D / 8, "staging must divide evenly");
};

template <int D_>
__global__ __launch_bounds__(512) void fwd_bf16_kernel(FwdParams p) {
  using C = Bf16Fwd<D_>;
  constexpr int D = C::D, BN = C::BN, KS = C::KS, VS = C::VS;
  __shared__ __attribute__((aligned(16))) bf16 smem[C::NBUF * C::STAGE];

  Job jb;
  if (!make_job(p, C::BM, &jb)) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int lr = lane & 31;
  const int g = lane >> 5;
  const bool groupB = wave >= 4;
  const int gtid = tid & (C::GT - 1);
  const int b = jb.bh / p.H, h = jb.bh % p.H;
  const bf16* qg = (const bf16*)p.q + b * p.sqB + h * p.sqH;
  const bf16* kg = (const bf16*)p.k + b * p.skB + h * p.skH;
  const bf16* vg = (const bf16*)p.v + b * p.svB + h * p.svH;

  const int64_t wrow0 = jb.r0 + wave * 32;
  const int64_t myrow = wrow0 + lr;
  const bool row_ok = myrow < jb.r1;
  const int64_t row_w = p.causal == 2 ? myrow / p.blk : 0;  // striped: shard, index
  const int64_t row_c = p.causal == 2 ? myrow - row_w * p.blk : 0;
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    qreg[s] = row_ok ? *(const bf16x8*)(qg + myrow * p.sqS + 16 * s + 8 * g) : bf16x8{};

  float m2 = -INFINITY, lsum = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = f32x16{};
  const int64_t BH = (int64_t)p.B * p.H;
  if (jb.epi == EPI_ACC && jb.acc_in) {
    float lp = row_ok ? p.lse[jb.bh * p.SQ + myrow] : -INFINITY;
    if (lp != -INFINITY) {
      m2 = lp * kLog2e;
      lsum = (g == 0) ? 1.f : 0.f;
      const float* src = p.o_acc + (jb.bh * p.SQ + myrow) * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x4 x = *(const f32x4*)(src + 32 * dt + 8 * i + 4 * g);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) oacc[dt][4 * i + jj] = x[jj];
        }
    }
  }

  TileIter tv;  // tile of the next softmax phase
  tv.seek(p, jb, 0, BN);
  if (!tv.valid(jb) && jb.epi == EPI_ACC && jb.acc_in) return;  // skipped pair

  // staging: group A moves K tiles, group B moves V tiles (row-major, padded)
  u32x4 stg[C::KC];
  const bf16* ssrc = groupB ? vg : kg;
  const int64_t sstr = groupB ? p.svS : p.skS;
  const int soff = groupB ? C::K_TILE : 0;
  const int srs = groupB ? VS : KS;
  // This thread's chunks are rows srow0 + i * srstep of a tile, 16 bytes at
  // column chunk scol8.  Their byte offsets from the tile's first row fit in
  // 24-bit products (row strides are below 16 MiB, checked on the host), so a
  // tile is loaded from one uniform base plus cheap per-thread offsets.
  const int srow0 = gtid / (D / 8), scol8 = gtid % (D / 8);
  constexpr int srstep = C::GT / (D / 8);
  const uint32_t sstr2 = (uint32_t)(sstr * 2);  // row stride in bytes, < 2^24
  // Load the tile of `lim` keys (1..BN) starting at row0 of the staged tensor,
  // branch-free: rows at or past lim repeat the last key (their scores are
  // masked, their P is zero and the repeated V row is finite).
  auto load_rows = [&](const bf16* row0, int lim) {
    const char* base = (const char*)row0;
#pragma unroll
    for (int i = 0; i < C::KC; ++i) {
      const int r = min(srow0 + i * srstep, lim - 1);
      const uint32_t off = __umul24((uint32_t)r, sstr2) + (uint32_t)(scol8 * 16);
      stg[i] = *(const u32x4*)(base + off);  // uniform base + 32-bit lane offset
    }
  };
  auto load_tile = [&](const TileIter& t) {
    load_rows(ssrc + t.kt * sstr, (int)min(t.ke - t.kt, (int64_t)BN));
  };
  auto store_tile = [&](int buf) {
    bf16* dst = smem + buf * C::STAGE + soff;
#pragma unroll
    for (int i = 0; i < C::KC; ++i)
      *(u32x4*)(dst + (srow0 + i * srstep) * srs + scol8 * 8) = stg[i];
  };

  f32x16 sacc[BN / 32];
  bf16x8 pb[BN / 16];
  auto phase_s = [&](int buf) {
    const bf16* ks = smem + buf * C::STAGE;
#pragma unroll
    for (int u = 0; u < BN / 32; ++u) sacc[u] = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
#pragma unroll
      for (int u = 0; u < BN / 32; ++u) {
        bf16x8 a = *(const bf16x8*)(ks + (32 * u + lr) * KS + 16 * s + 8 * g);
        sacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], sacc[u], 0, 0, 0);
      }
  };
  auto phase_pv = [&](int buf) {
    const bf16* vt_s = smem + buf * C::STAGE + C::K_TILE;
    const int li = lane & 15;
    const bf16* vbase = vt_s + (li >> 2) * VS + ((lane >> 4) & 1) * 16 + 4 * (li & 3);
#pragma unroll
    for (int t = 0; t < BN / 16; ++t)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const bf16* a0 = vbase + (16 * t + 4 * g) * VS + 32 * dt;
        s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0));
        s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0 + 8 * VS));
        u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[t], oacc[dt], 0, 0, 0);
      }
  };
  const float c2 = p.scale_log2;
  auto phase_softmax = [&](const TileIter& t) {
    bool need_mask = (t.kt + BN > t.ke) || (p.causal == 1 && t.kt + BN - 1 > wrow0);
    if (p.causal == 2)
      need_mask = __builtin_amdgcn_ballot_w64(
                      visible_prefix(t.kt, t.ke, 2, myrow, BN, p.blk, row_w, row_c) < BN) != 0;
    if (need_mask) {
      const int lim = visible_prefix(t.kt, t.ke, p.causal, myrow, BN, p.blk, row_w, row_c);
#pragma unroll
      for (int u = 0; u < BN / 32; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            if (32 * u + 8 * i + 4 * g + jj >= lim) sacc[u][4 * i + jj] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < BN / 32; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[u][e]);
    mx = wave_swap32_max(mx);
    const float m_cand = fmaxf(m2, mx * c2);
    if (__builtin_amdgcn_ballot_w64(m_cand > m2 + kLazyRescale) != 0) {
      const float alpha = fast_exp2(m2 - ((m_cand == -INFINITY) ? 0.f : m_cand));
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
      m2 = m_cand;
    }
    const float m_use = (m2 == -INFINITY) ? 0.f : m2;
    float ts[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < BN / 32; ++u)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        bf16x8 x;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float pv = fast_exp2(__builtin_fmaf(sacc[u][8 * hh + e], c2, -m_use));
          ts[e & 3] += pv;
          x[e] = (bf16)pv;
        }
        pb[2 * u + hh] = x;
      }
    lsum += (ts[0] + ts[1]) + (ts[2] + ts[3]);
  };

  // ---- prologue: tile 0 into buffer 0, tile 1 in flight
  TileIter tw = tv;  // next tile this thread's group stages
  if (tv.valid(jb)) {
    load_tile(tw);
    store_tile(0);
    tw.advance(p, jb, BN);
    if (tw.valid(jb)) load_tile(tw);
  }
  __syncthreads();
  if (!groupB) {
    if (tv.valid(jb)) phase_s(0);  // slot 0
    __syncthreads();
  } else {
    __syncthreads();               // slot 0: idle
    if (tv.valid(jb)) phase_s(0);  // slot 1
    __syncthreads();
  }
  // Settle the prologue's global loads (Q, the carried accumulator) here: the
  // wait-count pass cannot tell that the loop's first MFMAs already waited for
  // them, and would otherwise wait on every tile's staging loads as well.
#pragma unroll
  for (int s = 0; s < D / 16; ++s) pin(qreg[s]);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) pin(oacc[dt]);
  int j = 0;
  while (tv.valid(jb)) {
    const int cur = j % 3, nxt = (j + 1) % 3;
    phase_softmax(tv);
#pragma unroll
    for (int t = 0; t < BN / 16; ++t) pin(pb[t]);
    pin(lsum);
    if (tw.valid(jb)) {  // stage tile j+1, fetch tile j+2
      store_tile(nxt);
      tw.advance(p, jb, BN);
      if (tw.valid(jb)) load_tile(tw);
    }
    __syncthreads();
    TileIter tn = tv;
    tn.advance(p, jb, BN);
    phase_pv(cur);
    if (tn.valid(jb)) phase_s(nxt);
#pragma unroll
    for (int u = 0; u < BN / 32; ++u) pin(sacc[u]);
    // group A closes this slot; group B's last MFMA slot is the final one
    if (!groupB || tn.valid(jb)) __syncthreads();
    tv = tn;
    ++j;
  }

  // ---- epilogue
  const float ltot = wave_swap32_sum(lsum);
  const bool empty = (m2 == -INFINITY) || !(ltot > 0.f);
  const float inv = empty ? 0.f : 1.f / ltot;
  const float lse = empty ? -INFINITY : (m2 + __log2f(ltot)) * kLn2;
  if (!row_ok) return;
  if (jb.epi == EPI_FINAL) {
    bf16* dst = (bf16*)p.o + b * p.soB + h * p.soH + myrow * p.soS;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        store4<bf16>(dst + 32 * dt + 8 * i + 4 * g, oacc[dt][4 * i] * inv,
                     oacc[dt][4 * i + 1] * inv, oacc[dt][4 * i + 2] * inv,
                     oacc[dt][4 * i + 3] * inv);
    if (g == 0) p.lse[jb.bh * p.SQ + myrow] = lse;
  } else {
    float* obase = p.o_acc;
    float* lbase = p.lse;
    if (jb.epi == EPI_PART) {
      obase += (int64_t)jb.block * BH * p.SQ * D;
      lbase = p.lse_part + (int64_t)jb.block * BH * p.SQ;
    }
    float* dst = obase + (jb.bh * p.SQ + myrow) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        store4<float>(dst + 32 * dt + 8 * i + 4 * g, oacc[dt][4 * i] * inv,
                      oacc[dt][4 * i + 1] * inv, oacc[dt][4 * i + 2] * inv,
                      oacc[dt][4 * i + 3] * inv);
    if (g == 0) lbase[jb.bh * p.SQ + myrow] = lse;
  }
}

// ------------------------------------------------------------------ fp32 VALU kernel

template <int D>
struct F32Fwd {
  static constexpr int BN = 32;   // keys per tile
  static constexpr int BM = 64;   // query rows per workgroup (4 lanes per row)
  static constexpr int NT = 256;
  static constexpr int DL = D / 4;  // dims per lane
  static constexpr int KS = D + 4;  // LDS row stride (floats)
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
  const int sub = tid & 3;  // which quarter of D this lane owns
  const int64_t myrow = jb.r0 + (tid >> 2);
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
  for (; it.valid(jb); it.advance(p, jb, BN)) {
    // keys it.kt + j, j < lim, are visible to this row
    const int lim = visible_prefix(it.kt, it.ke, p.causal, myrow, BN, p.blk, row_w, row_c);
    __syncthreads();
    for (int c = tid; c < BN * D / 4; c += C::NT) {
      int row = c / (D / 4), col4 = c % (D / 4);
      int64_t key = it.kt + row;
      f32x4 kx = f32x4{}, vx = f32x4{};
      if (key < it.ke) {
        kx = *(const f32x4*)(kg + key * p.skS + col4 * 4);
        vx = *(const f32x4*)(vg + key * p.svS + col4 * 4);
      }
      *(f32x4*)(Ks + row * KS + col4 * 4) = kx;
      *(f32x4*)(Vs + row * KS + col4 * 4) = vx;
    }
    __syncthreads();
    // one key at a time: score, then the online-softmax update of (m, l, acc)
#pragma unroll 2
    for (int j = 0; j < BN; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < DL; ++e) dot = __builtin_fmaf(qv[e], Ks[j * KS + sub * DL + e], dot);
      dot += __shfl_xor(dot, 1);
      dot += __shfl_xor(dot, 2);
      if (j >= lim) continue;  // uniform across the four lanes of a row
      const float t = dot * c2;
      const float m_new = fmaxf(m2, t);
      const float alpha = fast_exp2(m2 - m_new);
      const float pj = fast_exp2(t - m_new);
      m2 = m_new;
      l = l * alpha + pj;
#pragma unroll
      for (int e = 0; e < DL; ++e)
        acc[e] = __builtin_fmaf(pj, Vs[j * KS + sub * DL + e], acc[e] * alpha);
    }
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
  if (dtype_bf16) {
    if (p.D == 128)
      hipLaunchKernelGGL(fwd_bf16_kernel<128>, dim3(blocks), dim3(Bf16Fwd<128>::NT), 0, st, p);
    else
      hipLaunchKernelGGL(fwd_bf16_kernel<64>, dim3(blocks), dim3(Bf16Fwd<64>::NT), 0, st, p);
  } else {
    if (p.D == 128)
      hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3(blocks), dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3(blocks), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace bwa
