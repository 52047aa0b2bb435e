// Backward of exact blockwise attention for gfx950 (bf16 inputs, D = 64 or 128).
//
// The pages leave the distributed backward unspecified (LV-XAttn review,
// referee report major comment 1, asks for exactly this: the gradient of the
// exact attention formula).  Read plainly, each block pair contributes
// additively once the forward's global row statistics are known:
//   P = exp(scale * Q K^T - LSE),  Delta = rowsum(dO * O),
//   dV += P^T dO,  dP = dO V^T,  dS = P * (dP - Delta),
//   dQ += scale * dS K,  dK += scale * dS^T Q.
// Two deterministic kernels (no atomics) follow the two ring schedules' data
// placement: the KV-stationary kernel keeps a key tile's K, V, dK, dV in
// registers while query tiles stream past (LV-XAttn: KV stays put, Q/dO/LSE/
// Delta rotate); the Q-stationary kernel keeps a query tile's Q, dO, dQ in
// registers while key tiles stream past (Ring Attention).  Every contraction
// is a v_mfma_f32_32x32x16_bf16; operands whose contraction index is the row
// index of their storage (dO^T, Q^T, K^T) are read from the row-major LDS
// tiles with the transposing ds_read_b64_tr_b16.
#include <type_traits>

#include "bwd_args.h"
#include "common.h"

namespace bwa {

struct BwdParams {
  const bf16 *q, *k, *v, *o, *dout;
  int64_t sq[3], sk[3], sv[3], so[3], sdo[3];
  bf16 *dq, *dk, *dv;
  int64_t sdq[3], sdk[3], sdv[3];
  const float* lse;
  float* delta;   // [BH][SQ]
  float* dq_acc;  // ROUNDS: [BH][SQ][D]
  float* dk_acc;  // ROUNDS: [BH][SKV][D]
  float* dv_acc;  // ROUNDS: [BH][SKV][D]
  int B, H, SQ, SKV, n, sched, mode, causal, round;
  int nq;  // dK/dV kernel: query blocks it walks (n, or 1 for the whole range)
  int nk;  // dQ kernel: key shards it walks (n, or 1 for the whole range)
  int kv_tiles;  // dK/dV kernel: key tiles per shard if the grid is head-major, else 0
  int tiles, groups;
  float scale, scale_log2;
};

namespace {

__device__ inline uint32_t pk_bf16(float a, float b) {
  bf16 x = (bf16)a, y = (bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

__device__ inline bf16x8 pack8(const f32x16& c, int h) {
  bf16x8 x;
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (bf16)c[8 * h + e];
  return x;
}

// Ordered segments of a backward job.
//   KV-stationary kernel: a key tile of shard s meets query blocks in round
//     order: (s - r) mod n for the KV-stationary schedule, (s + r) mod n for
//     the Q-stationary one.
//   Q-stationary kernel: a query tile of block j meets shards (j + r) mod n or
//     (j - r) mod n, the same order as the forward merge.
__device__ inline int qblock_at_step(int sched, int n, int s, int r) {
  return sched == SCHED_KV_STATIONARY ? ring_sub(s, r, n) : ring_add(s, r, n);
}

}  // namespace

// ---------------------------------------------------------------- Delta = rowsum(dO * O)

// D/8 consecutive threads per row, 8 elements each.
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdParams p) {
  constexpr int TPR = D / 8;
  const int64_t rows = (int64_t)p.B * p.H * p.SQ;
  int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int64_t row = idx / TPR;
  int c = (int)(idx % TPR);
  float s = 0.f;
  if (row < rows) {
    int64_t bh = row / p.SQ, i = row % p.SQ, b = bh / p.H, h = bh % p.H;
    u32x4 o = *(const u32x4*)(p.o + b * p.so[0] + h * p.so[1] + i * p.so[2] + c * 8);
    u32x4 d = *(const u32x4*)(p.dout + b * p.sdo[0] + h * p.sdo[1] + i * p.sdo[2] + c * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      s += __uint_as_float(o[w] << 16) * __uint_as_float(d[w] << 16);
      s += __uint_as_float(o[w] & 0xffff0000u) * __uint_as_float(d[w] & 0xffff0000u);
    }
  }
  if (TPR > 8) s += __shfl_xor(s, 8);
  s += __shfl_xor(s, 4);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 1);
  if (row < rows && c == 0) p.delta[row] = s;
}

// LDS tiles of the two MFMA kernels below keep their rows in groups of four:
// rows of a group 2(D+32) bytes apart (320 or 192: 64 or 192 mod 256) and
// groups 2(4D+104) bytes apart (1232 or 720: 16 mod 64).  Sixteen consecutive
// rows then start in sixteen distinct 16-byte bank slots (row reads by
// ds_read_b128, one row per lane), and four
// rows of a group cover all 64 banks with 64 bytes each (transposing reads by
// ds_read_b64_tr_b16), while every address stays a lane base plus a constant.
template <int D>
struct Lay {
  static constexpr int kRowStr = D + 32, kGrpStr = 3 * kRowStr + D + 8;
  __device__ static inline int rbase(int r) { return (r >> 2) * kGrpStr + (r & 3) * kRowStr; }
  // A operand of 16 contraction rows (16t + 4g + {0..3}, 16t + 4g + 8 + {0..3};
  // the row order of an MFMA result packed by pack8) x head dims 32dt + lane%32,
  // read transposed from a row-major tile whose lane base is trb (below).
  __device__ static inline bf16x8 tr_rows(const bf16* tile_lane, int t, int dt);
  // Lane base of tr_rows: row 4g + li/4 (li = lane % 16), column 16*(lane/16 % 2) + 4*(li % 4).
  __device__ static inline int trb(int lane) {
    const int li = lane & 15, g = lane >> 5;
    return g * kGrpStr + (li >> 2) * kRowStr + 16 * ((lane >> 4) & 1) + 4 * (li & 3);
  }
};

template <typename T>
__device__ inline void hold(T& x) {  // materialise x here: an empty asm that reads and writes it
  asm volatile("" : "+v"(x));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int D>
__device__ inline bf16x8 Lay<D>::tr_rows(const bf16* tile_lane, int t, int dt) {
  const bf16* a0 = tile_lane + 4 * t * kGrpStr + 32 * dt;
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0 + 2 * kGrpStr));
  u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
}

// ---------------------------------------------------------------- dK, dV (KV-stationary)
//
// 128 keys per workgroup; 8 waves in two roles over the same four 32-key
// groups: waves 0-3 (group A) accumulate dV, waves 4-7 (group B) dK, and wave
// w shares its SIMD with wave w+4.  Splitting by output keeps each wave within
// half the register file (A holds K and dV, B holds V and dK).  A computes
// P and hands it, rounded to bf16, to B through LDS.  Queries stream in tiles
// of 64 rows, and the two groups alternate like the dQ kernel's, one phase
// apart:
//   A: MFMA  dV^T += dO^T P (tile j-1), S = Q K^T (tile j)         32 MFMAs
//      VALU  P = exp2(S scale log2(e) - LSE log2(e)) to LDS, writes Q(j+1), LSE
//   B: MFMA  dK^T += Q^T dS (tile j-1), dP = dO V^T (tile j)       32 MFMAs
//      VALU  dS = P o (dP - Delta) with P from LDS, writes dO(j+1), Delta
// Slots from 0:  A: slot 0: S(0);  2j+1: P(j);  2j+2: dV(j), S(j+1)
//                B: slot 1: dP(0);  2j+2: dS(j);  2j+3: dK(j), dP(j+1)
// Q tiles (with their rows' LSE) and dO tiles (with Delta) rotate through
// three LDS buffers; Q(j) is read from slot 2j to 2j+3 and rewritten (as
// Q(j+3)) in slot 2j+5, dO(j) is read in slots 2j+1 and 2j+2 and rewritten in
// slot 2j+6.  P(j) is written in slot 2j+1 and read in slot 2j+2.

// dK/dV: 8 waves in two roles; dQ: 8 waves, two per SIMD.
constexpr int kDkdvWaves = 8, kDqWaves = 8;

// CM instantiates the masking code (0 none, 1 sequence order, 2 striped
// order); p.causal must agree.  Under either causal order a key sees the
// query rows of a segment from a first row on: key row j from row j (sequence
// order); in the striped order, key index c of shard s from index c of query
// shards w >= s and index c + 1 of shards w < s (its position is c*n + s).
// With qo = (query shard start) - (key shard start) + [s > w] (0 in sequence
// order) the first row that sees key j is j + qo.
template <int D, int CM>
__global__ __launch_bounds__(64 * kDkdvWaves) void bwd_dkdv_kernel(BwdParams p) {
  constexpr bool CAUSAL = CM != 0;
  using Ly = Lay<D>;
  constexpr int kGrpStr = Ly::kGrpStr;
  constexpr int BK = 128, BQ = 64, GT = 64 * kDkdvWaves / 2;
  constexpr int TILE = BQ / 4 * kGrpStr, STAGE = 2 * TILE, NBUF = 3;
  constexpr int KC = (BQ * D / 8) / GT;  // 16-byte chunks per staging thread and tile
  static_assert(KC * GT == BQ * D / 8, "staging must divide evenly");
  __shared__ __attribute__((aligned(16))) bf16 smem[NBUF * STAGE];
  __shared__ float s_lse[NBUF][BQ], s_dlt[NBUF][BQ];
  __shared__ __attribute__((aligned(16))) bf16 s_p[4][BQ / 16][64 * 8];  // P per A wave, B-operand order

  int g_, t_;
  if (!xcd_group_tile(blockIdx.x, p.tiles, p.groups, &g_, &t_)) return;
  const int BH = p.B * p.H;
  // group = (shard or round worker, head), tile = key tile of that shard;
  // or, head-major (FUSED with at least 8 heads): group = head and tile =
  // (shard, key tile), so that all of a head's key tiles run back to back on
  // one XCD and share its Q and dO in that XCD's L2.
  const bool head_major = p.kv_tiles > 0;
  const int bh = head_major ? g_ : g_ % BH;
  if (head_major) {
    g_ = (t_ / p.kv_tiles) * BH + bh;  // the (shard, head) group index
    t_ = t_ % p.kv_tiles;
  }
  int shard, nseg, fixed_qb = -1;
  bool acc_in = false;
  if (p.mode == MODE_ROUNDS) {
    int qb;
    ring_pair(p.sched, p.n, p.round, g_ / BH, &qb, &shard);
    fixed_qb = qb;
    nseg = 1;
    acc_in = p.round > 0;
  } else {
    // FUSED walks p.nq query blocks: n in the schedule's order, or (rows in
    // sequence order) 1, all query rows as one segment; dK and dV are sums
    // over the query rows, the same in any block order up to fp32 rounding,
    // and a switch of segment costs about one query step.  The striped order
    // keeps one segment per query shard (its mask shift changes per shard).
    shard = g_ / BH;
    nseg = p.nq;
  }
  const int qs0 = p.nq == 1 ? 0 : shard;  // the query block walked first
  const int64_t ks = shard_start(p.SKV, p.n, shard), ke = shard_start(p.SKV, p.n, shard + 1);
  const int64_t kt0 = ks + (int64_t)t_ * BK;
  const int64_t kt1 = min(ke, kt0 + BK);
  if (kt0 >= kt1) return;

  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool groupB = wave >= kDkdvWaves / 2;  // B: dK, A: dV
  const int gtid = tid & (GT - 1);
  const int b = bh / p.H, h = bh % p.H;
  const int64_t kw0 = kt0 + (wave & 3) * 32;
  const int64_t mykey = kw0 + lr;
  const bool key_ok = mykey < kt1;

  const bf16* qg = p.q + b * p.sq[0] + h * p.sq[1];
  const bf16* dog = p.dout + b * p.sdo[0] + h * p.sdo[1];
  const float* lseg = p.lse + (int64_t)bh * p.SQ;
  const float* dltg = p.delta + (int64_t)bh * p.SQ;

  // B operand rows of this lane's key: K (role A, for S) or V (role B, for dP)
  bf16x8 breg[D / 16];
  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};

  // query tiles over the ordered segments
  struct It {
    int r;
    int64_t qt, qe;
    int qo;  // causal: the first query row that sees key j is j + qo
  };
  auto seek = [&](It& it, int from) {
    for (it.r = from; it.r < nseg; ++it.r) {
      int qb = fixed_qb >= 0 ? fixed_qb : qblock_at_step(p.sched, p.nq, qs0, it.r);
      int64_t a = shard_start(p.SQ, p.nq, qb), e = shard_start(p.SQ, p.nq, qb + 1);
      it.qo = CM == 2 ? (int)(a - ks) + (shard > qb ? 1 : 0) : 0;
      if (CAUSAL && a < kt0 + it.qo) a = kt0 + it.qo;  // rows before that see none of the tile
      if (e > a) {
        it.qt = a;
        it.qe = e;
        return;
      }
    }
    it.qt = it.qe = it.qo = 0;
  };
  auto advance = [&](It& it) {
    it.qt += BQ;
    if (it.qt >= it.qe) seek(it, it.r + 1);
  };
  It tv;  // tile of the next VALU phase
  seek(tv, 0);
  if (tv.r >= nseg && acc_in) return;  // nothing to add this round

  // staging: group A moves Q tiles and their rows' LSE, group B dO tiles and
  // their rows' Delta; thread chunks are rows srow0 + 16 i of a tile at chunk
  // column scol
  const bf16* ssrc = groupB ? dog : qg;
  const int64_t sstr = groupB ? p.sdo[2] : p.sq[2];
  const int soff = groupB ? TILE : 0;
  const int srow0 = gtid / (D / 8), scol = gtid % (D / 8);
  constexpr int srstep = GT / (D / 8);
  static_assert(srstep % 4 == 0, "staging rows keep their place in a row group");
  u32x4 stg[KC];
  // Per query row of a tile, LDS holds the seeds of its S and dP accumulators,
  // -LSE/scale and -Delta, so that the MFMAs produce S - LSE/scale (P is
  // exp2 of it times scale*log2(e)) and dP - Delta without VALU work or LDS
  // reads in the VALU phase.
  float st_l = 0.f, st_d = 0.f;
  const float rscale = 1.f / p.scale;
  // Rows at or past the segment end repeat its last row and get the S seed
  // -inf (no weight).  Row strides are below 16 MiB (checked on the host), so
  // a chunk's byte offset from the tile's first row is a 24-bit product.
  const uint32_t sstr2 = (uint32_t)(sstr * 2);
  auto load_tile = [&](const It& t) {
    const int lim = (int)min(t.qe - t.qt, (int64_t)BQ);
    const char* base = (const char*)(ssrc + t.qt * sstr);
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int r = min(srow0 + i * srstep, lim - 1);
      const uint32_t off = __umul24((uint32_t)r, sstr2) + (uint32_t)(scol * 16);
      stg[i] = *(const u32x4*)(base + off);
    }
    if (gtid < BQ) {  // raw values; transformed when written, after the VALU work
      const int64_t row = t.qt + gtid;
      if (!groupB)
        st_l = gtid < lim ? lseg[row] : -INFINITY;
      else
        st_d = gtid < lim ? dltg[row] : 0.f;
    }
  };
  const int wbase = soff + Ly::rbase(srow0) + scol * 8;
  auto store_tile = [&](int buf) {
    bf16* dst = smem + buf * STAGE + wbase;
#pragma unroll
    for (int i = 0; i < KC; ++i) *(u32x4*)(dst + i * (srstep / 4) * kGrpStr) = stg[i];
    if (gtid < BQ) {
      if (!groupB)
        s_lse[buf][gtid] = (st_l == -INFINITY) ? -INFINITY : -st_l * rscale;  // -inf: no weight
      else
        s_dlt[buf][gtid] = -st_d;
    }
  };

  f32x16 sacc[BQ / 32], pacc[BQ / 32];
  bf16x8 xb[BQ / 16];  // P (A) or dS (B) of the last VALU phase, bf16, in MFMA B-operand order
  const int rb = Ly::rbase(lr) + 8 * g;  // this lane's row-read base
  const int tb = Ly::trb(lane);
  // One MFMA slot as a fixed sequence: dV or dK of the current tile (16
  // MFMAs), then S (A) or dP (B) of the next (16).  The A operand of MFMA
  // m + DIST is read from LDS just before MFMA m is issued and a scheduling
  // barrier follows every MFMA, so each read has DIST MFMAs to arrive.
  constexpr int NACC = (BQ / 16) * (D / 32), NSP = (D / 16) * (BQ / 32), NM = NACC + NSP;
  constexpr int DIST = 4, NOB = DIST + 1, SEED_AHEAD = 4;
  // S (A) or dP (B) accumulators seeded from LDS; element 4i+jj of block u is
  // query row 32u + 8i + 4g + jj of the tile
  auto seed = [&](auto ROLE_B, int buf) {
    constexpr bool RB = decltype(ROLE_B)::value;
    f32x16* dst = RB ? pacc : sacc;
    const float* src = RB ? s_dlt[buf] : s_lse[buf];
#pragma unroll
    for (int u = 0; u < BQ / 32; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 x4 = *(const f32x4*)(src + 32 * u + 8 * i + 4 * g);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) dst[u][4 * i + jj] = x4[jj];
      }
  };
  auto mfma_slot = [&](auto ROLE_B, int cur_buf, int nxt_buf) {
    constexpr bool RB = decltype(ROLE_B)::value;
    auto rd = [&](auto M) -> bf16x8 {
      constexpr int m = decltype(M)::value;
      if constexpr (m < NACC) {  // dV: dO^T from the dO half; dK: Q^T from the Q half
        return Ly::tr_rows(smem + cur_buf * STAGE + (RB ? 0 : TILE) + tb, m / (D / 32), m % (D / 32));
      } else {  // S: Q rows; dP: dO rows
        constexpr int q = m - NACC, s = q / (BQ / 32), u = q % (BQ / 32);
        return *(const bf16x8*)(smem + nxt_buf * STAGE + (RB ? TILE : 0) + rb + u * 8 * kGrpStr +
                                16 * s);
      }
    };
    auto mf = [&](auto M, const bf16x8& a) {
      constexpr int m = decltype(M)::value;
      if constexpr (m < NACC) {
        constexpr int t = m / (D / 32), dt = m % (D / 32);
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, xb[t], acc[dt], 0, 0, 0);
      } else {
        constexpr int q = m - NACC, s = q / (BQ / 32), u = q % (BQ / 32);
        if constexpr (!RB)
          sacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, breg[s], sacc[u], 0, 0, 0);
        else
          pacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, breg[s], pacc[u], 0, 0, 0);
      }
    };
    bf16x8 ob[NOB];
    static_for<0, DIST>([&](auto M) { ob[decltype(M)::value % NOB] = rd(M); });
    static_for<0, NM>([&](auto M) {
      constexpr int m = decltype(M)::value;
      // seeds late in the dV/dK part, when most of xb is dead
      if constexpr (m == NACC - SEED_AHEAD) seed(ROLE_B, nxt_buf);
      if constexpr (m + DIST < NM) ob[(m + DIST) % NOB] = rd(std::integral_constant<int, m + DIST>{});
      mf(M, ob[m % NOB]);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // S (A) or dP (B) of tile 0, in buffer 0
  auto first_s = [&](auto ROLE_B) {
    constexpr bool RB = decltype(ROLE_B)::value;
    seed(ROLE_B, 0);
    const bf16* src = smem + (RB ? TILE : 0) + rb;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
#pragma unroll
      for (int u = 0; u < BQ / 32; ++u) {
        const bf16x8 a = *(const bf16x8*)(src + u * 8 * kGrpStr + 16 * s);
        if constexpr (!RB)
          sacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, breg[s], sacc[u], 0, 0, 0);
        else
          pacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, breg[s], pacc[u], 0, 0, 0);
      }
  };
  const float c2 = p.scale_log2;
  // A: P of a tile (element 4i+jj of block u is query qt + 32u + 8i + 4g + jj),
  // kept in xb and copied to s_p for B.  B: dS = P o (dP - Delta) with P from s_p.
  bf16* const pslot = &s_p[wave & 3][0][lane * 8];
  auto phase_valu = [&](auto ROLE_B, const It& t) {
    constexpr bool RB = decltype(ROLE_B)::value;
    if constexpr (!RB) {
      const bool need_mask = CAUSAL && t.qt < kw0 + t.qo + 31;
      // query offsets below lim precede this lane's key: no weight
      const int lim =
          need_mask ? (int)max(min(mykey + t.qo - t.qt, (int64_t)BQ), (int64_t)0) : 0;
#pragma unroll
      for (int u = 0; u < BQ / 32; ++u) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[u][e] = __builtin_amdgcn_exp2f(sacc[u][e] * c2);
        if (need_mask) {
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (32 * u + 8 * (e / 4) + 4 * g + (e % 4) < lim) sacc[u][e] = 0.f;
        }
        xb[2 * u] = pack8(sacc[u], 0);
        xb[2 * u + 1] = pack8(sacc[u], 1);
      }
#pragma unroll
      for (int q = 0; q < BQ / 16; ++q) *(bf16x8*)(pslot + q * 64 * 8) = xb[q];
    } else {
#pragma unroll
      for (int u = 0; u < BQ / 32; ++u) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const bf16x8 pv = *(const bf16x8*)(pslot + (2 * u + hh) * 64 * 8);
#pragma unroll
          for (int e = 0; e < 8; ++e) pacc[u][8 * hh + e] *= (float)pv[e];  // dS (unscaled)
        }
        xb[2 * u] = pack8(pacc[u], 0);
        xb[2 * u + 1] = pack8(pacc[u], 1);
      }
    }
  };

  auto run = [&](auto ROLE_B) {
    constexpr bool RB = decltype(ROLE_B)::value;
    {
      const bf16* src = RB ? p.v + b * p.sv[0] + h * p.sv[1] + mykey * p.sv[2]
                           : p.k + b * p.sk[0] + h * p.sk[1] + mykey * p.sk[2];
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
        breg[s] = key_ok ? *(const bf16x8*)(src + 16 * s + 8 * g) : bf16x8{};
    }
    // ---- prologue: tile 0 in buffer 0, each group's next tile in flight
    It tw = tv;  // next tile this thread's group stages
    load_tile(tw);
    store_tile(0);
    advance(tw);
    __syncthreads();
    if constexpr (!RB) {
      first_s(ROLE_B);  // slot 0
    } else {
      __syncthreads();  // slot 0: idle
      first_s(ROLE_B);  // slot 1
    }
#pragma unroll
    for (int u = 0; u < BQ / 32; ++u) {
      if constexpr (!RB) hold(sacc[u]);
      if constexpr (RB) hold(pacc[u]);
    }
    __syncthreads();
    // settle the prologue's global loads here, not inside the loop
#pragma unroll
    for (int s = 0; s < D / 16; ++s) hold(breg[s]);
    int it = 0;
    while (tv.r < nseg) {
      const int cur = it % 3, nxt = (it + 1) % 3;
      // Tile it+1 is loaded at the head of the VALU slot and written to LDS at
      // its end, so the staging registers are free during the MFMA slot.
      const bool stage = tw.r < nseg;
      if (stage) load_tile(tw);
      phase_valu(ROLE_B, tv);
#pragma unroll
      for (int t = 0; t < BQ / 16; ++t) hold(xb[t]);
      if (stage) {
        store_tile(nxt);
        advance(tw);
      }
      __syncthreads();
      It tn = tv;
      advance(tn);
      mfma_slot(ROLE_B, cur, nxt);  // after the last tile S (dP) read a stale buffer, unused
#pragma unroll
      for (int u = 0; u < BQ / 32; ++u) {
        if constexpr (!RB) hold(sacc[u]);
        if constexpr (RB) hold(pacc[u]);
      }
      // group A closes this slot; group B's last MFMA slot is the final one
      if (!RB || tn.r < nseg) __syncthreads();
      tv = tn;
      ++it;
    }
  };
  // (a job without query tiles skips all of it, so both groups meet the same barriers)
  if (tv.r < nseg) {
    if (groupB)
      run(std::true_type{});
    else
      run(std::false_type{});
  }

  if (!key_ok) return;
  const float sc = groupB ? p.scale : 1.f;
  if (p.mode == MODE_ROUNDS) {
    float* dst = (groupB ? p.dk_acc : p.dv_acc) + ((int64_t)bh * p.SKV + mykey) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 32 * dt + 8 * i + 4 * g;
        f32x4 a = f32x4{acc[dt][4 * i] * sc, acc[dt][4 * i + 1] * sc, acc[dt][4 * i + 2] * sc,
                        acc[dt][4 * i + 3] * sc};
        if (acc_in) a += *(const f32x4*)(dst + d);
        *(f32x4*)(dst + d) = a;
      }
  } else {
    bf16* dst = groupB ? p.dk + b * p.sdk[0] + h * p.sdk[1] + mykey * p.sdk[2]
                       : p.dv + b * p.sdv[0] + h * p.sdv[1] + mykey * p.sdv[2];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 32 * dt + 8 * i + 4 * g;
        *(u32x2*)(dst + d) = u32x2{pk_bf16(acc[dt][4 * i] * sc, acc[dt][4 * i + 1] * sc),
                                   pk_bf16(acc[dt][4 * i + 2] * sc, acc[dt][4 * i + 3] * sc)};
      }
  }
}

// ---------------------------------------------------------------- dQ (Q-stationary)
//
// 256 query rows per workgroup, 8 waves of 32 rows, 64-key tiles, arranged
// like the forward kernel: waves 0-3 (group A) and 4-7 (group B) share the
// four SIMDs and run one phase apart, so that between two barriers one wave
// of every SIMD issues MFMAs while the other issues VALU work.  Per tile t a
// wave runs an MFMA phase
//   dQ^T += K^T dS^T (tile t-1),  S^T = K Q^T and dP^T = V dO^T (tile t)
// (48 MFMAs) and a VALU phase  dS^T = P o (dP^T - Delta),
// P = exp2(S^T * scale*log2(e) - LSE*log2(e)),  plus its share of staging.
// Slots (barrier intervals) from 0; group A runs
//   slot 0: S/dP(0);  slot 2t+1: dS(t), write K(t+1);  slot 2t+2: dQ(t), S/dP(t+1)
// and group B the same one slot later, except that it writes V(t+2) in its
// VALU slot 2t+2 (V(1) in slot 0), so a tile's V is visible one slot before
// group A's S/dP of that tile.  Tiles rotate through three LDS buffers; each
// half of a buffer is rewritten only after its last reader's slot.

// CM as in the dK/dV kernel.  Under either causal order a query row sees the
// keys of a segment up to a last key: row i up to key i (sequence order); in
// the striped order, the row at index c of query shard w sees indices up to c
// of key shards s <= w and up to c - 1 of shards s > w.  With ko = (key shard
// start) - (query shard start) - [s > w] (0 in sequence order) the last key
// row that query row i sees is i + ko.
template <int D, int CM>
__global__ __launch_bounds__(64 * kDqWaves) void bwd_dq_kernel(BwdParams p) {
  constexpr bool CAUSAL = CM != 0;
  using Ly = Lay<D>;
  constexpr int kGrpStr = Ly::kGrpStr;
  constexpr int BM = 32 * kDqWaves, BN = 64, GT = 64 * kDqWaves / 2;
  constexpr int TILE = BN / 4 * kGrpStr, STAGE = 2 * TILE, NBUF = 3;
  constexpr int KC = (BN * D / 8) / GT;  // 16-byte chunks per staging thread and tile
  static_assert(KC * GT == BN * D / 8, "staging must divide evenly");
  __shared__ __attribute__((aligned(16))) bf16 smem[NBUF * STAGE];

  int g_, t_;
  if (!xcd_group_tile(blockIdx.x, p.tiles, p.groups, &g_, &t_)) return;
  const int BH = p.B * p.H;
  const int bh = g_ % BH;
  int j, nseg, fixed_kb = -1;
  bool acc_in = false;
  if (p.mode == MODE_ROUNDS) {
    int kb;
    ring_pair(p.sched, p.n, p.round, g_ / BH, &j, &kb);
    fixed_kb = kb;
    nseg = 1;
    acc_in = p.round > 0;
  } else {
    // FUSED walks p.nk key segments: the n shards in the schedule's order, or
    // (rows in sequence order) 1, all keys in sequence order, so that the
    // query tiles of a head stream the same K, V tiles at the same time; dQ
    // is a sum over the keys, the same in any order up to fp32 rounding.
    j = p.causal ? (p.n - 1 - g_ / BH) : (g_ / BH);
    nseg = p.nk;
  }
  const int ks0 = p.nk == 1 ? 0 : j;  // the key segment walked first
  const int64_t qs = shard_start(p.SQ, p.n, j), qe = shard_start(p.SQ, p.n, j + 1);
  const int64_t r0 = qs + (int64_t)t_ * BM;
  const int64_t r1 = min(qe, r0 + BM);
  if (r0 >= r1) return;

  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool groupB = wave >= kDqWaves / 2;
  const int gtid = tid & (GT - 1);
  const int b = bh / p.H, h = bh % p.H;
  const int64_t wrow0 = r0 + wave * 32;
  const int64_t myrow = wrow0 + lr;
  const bool row_ok = myrow < r1;

  const bf16* kg = p.k + b * p.sk[0] + h * p.sk[1];
  const bf16* vg = p.v + b * p.sv[0] + h * p.sv[1];
  bf16x8 qreg[D / 16], doreg[D / 16];
  {
    const bf16* qp = p.q + b * p.sq[0] + h * p.sq[1] + myrow * p.sq[2];
    const bf16* dp = p.dout + b * p.sdo[0] + h * p.sdo[1] + myrow * p.sdo[2];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      qreg[s] = row_ok ? *(const bf16x8*)(qp + 16 * s + 8 * g) : bf16x8{};
      doreg[s] = row_ok ? *(const bf16x8*)(dp + 16 * s + 8 * g) : bf16x8{};
    }
  }
  float lse2 = INFINITY, dlt = 0.f;
  if (row_ok) {
    float l = p.lse[(int64_t)bh * p.SQ + myrow];
    lse2 = (l == -INFINITY) ? INFINITY : l * kLog2e;  // +inf: the row takes no weight
    dlt = p.delta[(int64_t)bh * p.SQ + myrow];
  }
  f32x16 dq[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) dq[dt] = f32x16{};

  // key tiles over the ordered segments
  struct It {
    int r;
    int64_t kt, ke;
    int ko;  // causal: the last key row that query row i sees is i + ko
  };
  auto seek = [&](It& it, int from) {
    for (it.r = from; it.r < nseg; ++it.r) {
      int kb = fixed_kb >= 0 ? fixed_kb : shard_at_step(p.sched, p.nk, ks0, it.r);
      int64_t a = shard_start(p.SKV, p.nk, kb), e = shard_start(p.SKV, p.nk, kb + 1);
      it.ko = CM == 2 ? (int)(a - qs) - (kb > j ? 1 : 0) : 0;
      if (CAUSAL && e > r1 + it.ko) e = r1 + it.ko;  // keys after the job's last row's last key
      if (e > a) {
        it.kt = a;
        it.ke = e;
        return;
      }
    }
    it.kt = it.ke = it.ko = 0;
  };
  auto advance = [&](It& it) {
    it.kt += BN;
    if (it.kt >= it.ke) seek(it, it.r + 1);
  };
  It tv;  // tile of the next VALU phase
  seek(tv, 0);
  if (tv.r >= nseg && acc_in) return;  // nothing to add this round

  // staging: group A moves K tiles, group B V tiles; thread chunks are rows
  // srow0 + 16 i of a tile at chunk column scol
  const bf16* ssrc = groupB ? vg : kg;
  const int64_t sstr = groupB ? p.sv[2] : p.sk[2];
  const int soff = groupB ? TILE : 0;
  const int srow0 = gtid / (D / 8), scol = gtid % (D / 8);
  constexpr int srstep = GT / (D / 8);
  u32x4 stg[KC];
  // Rows at or past the segment end: V rows repeat its last key, K rows are
  // written as zeros, so those keys add nothing to dQ = dS K whatever their dS
  // and need no mask in the VALU slot.  Row strides are below 16 MiB (checked
  // on the host), so a chunk's byte offset from the tile's first row is a
  // 24-bit product.
  const uint32_t sstr2 = (uint32_t)(sstr * 2);
  uint32_t szero = 0;  // chunks of the loaded tile to write as zeros (bit i: chunk i)
  auto load_tile = [&](const It& t) {
    const int lim = (int)min(t.ke - t.kt, (int64_t)BN);
    const char* base = (const char*)(ssrc + t.kt * sstr);
    szero = 0;
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int r = min(srow0 + i * srstep, lim - 1);
      const uint32_t off = __umul24((uint32_t)r, sstr2) + (uint32_t)(scol * 16);
      stg[i] = *(const u32x4*)(base + off);
      if (!groupB && srow0 + i * srstep >= lim) szero |= 1u << i;
    }
  };
  static_assert(srstep % 4 == 0, "staging rows keep their place in a row group");
  const int wbase = soff + Ly::rbase(srow0) + scol * 8;
  auto store_tile = [&](int buf) {
    bf16* dst = smem + buf * STAGE + wbase;
#pragma unroll
    for (int i = 0; i < KC; ++i)
      *(u32x4*)(dst + i * (srstep / 4) * kGrpStr) = ((szero >> i) & 1) ? u32x4{} : stg[i];
  };

  f32x16 sacc[BN / 32], pacc[BN / 32];
  bf16x8 dsb[BN / 16];
  // S^T = K Q^T and dP^T = V dO^T; element 4i+jj of block u is key 32u+8i+4g+jj
  const int rb = Ly::rbase(lr) + 8 * g;  // this lane's row-read base
  auto phase_sdp = [&](int buf) {
    const bf16* ks = smem + buf * STAGE + rb;
    const bf16* vs = ks + TILE;
#pragma unroll
    for (int u = 0; u < BN / 32; ++u) sacc[u] = pacc[u] = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
#pragma unroll
      for (int u = 0; u < BN / 32; ++u) {
        const int off = u * 8 * kGrpStr + 16 * s;  // row 32u + lr, columns 16s + 8g ..
        sacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(ks + off), qreg[s],
                                                          sacc[u], 0, 0, 0);
        pacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(vs + off), doreg[s],
                                                          pacc[u], 0, 0, 0);
      }
  };
  // dQ^T += K^T dS^T: the A operand of step t covers keys 16t+4g+{0..3} and
  // 16t+4g+8+{0..3} of head dims 32dt + lane%32, the key order of dsb[t]
  const int tb = Ly::trb(lane);
  // One MFMA slot as a fixed sequence: dQ of the current tile (16 MFMAs), then
  // S and dP of the next (32).  The A operand of MFMA m + DIST is read from
  // LDS just before MFMA m is issued and a scheduling barrier follows every
  // MFMA, so each read has DIST MFMAs to arrive.
  constexpr int NDQ = (BN / 16) * (D / 32), NSP = 2 * (D / 16) * (BN / 32), NM = NDQ + NSP;
  constexpr int DIST = 2, NB = DIST + 1;
  auto op_read = [&](auto M, int cur_buf, int nxt_buf) -> bf16x8 {
    constexpr int m = decltype(M)::value;
    if constexpr (m < NDQ) {
      return Ly::tr_rows(smem + cur_buf * STAGE + tb, m / (D / 32), m % (D / 32));
    } else {
      constexpr int q = m - NDQ, s = q / 4, u = (q / 2) % 2, kind = q % 2;
      return *(const bf16x8*)(smem + nxt_buf * STAGE + kind * TILE + rb + u * 8 * kGrpStr + 16 * s);
    }
  };
  auto op_mfma = [&](auto M, const bf16x8& a) {
    constexpr int m = decltype(M)::value;
    if constexpr (m < NDQ) {
      constexpr int t = m / (D / 32), dt = m % (D / 32);
      dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsb[t], dq[dt], 0, 0, 0);
    } else {
      constexpr int q = m - NDQ, s = q / 4, u = (q / 2) % 2, kind = q % 2;
      if constexpr (kind == 0)
        sacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], s == 0 ? f32x16{} : sacc[u],
                                                          0, 0, 0);
      else
        pacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, doreg[s], s == 0 ? f32x16{} : pacc[u],
                                                          0, 0, 0);
    }
  };
  auto mfma_slot = [&](int cur_buf, int nxt_buf) {
    bf16x8 ob[NB];
    static_for<0, DIST>([&](auto M) { ob[decltype(M)::value % NB] = op_read(M, cur_buf, nxt_buf); });
    static_for<0, NM>([&](auto M) {
      constexpr int m = decltype(M)::value;
      if constexpr (m + DIST < NM)
        ob[(m + DIST) % NB] = op_read(std::integral_constant<int, m + DIST>{}, cur_buf, nxt_buf);
      op_mfma(M, ob[m % NB]);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  const float c2 = p.scale_log2;
  auto phase_ds = [&](const It& t) {
    // causal: this row sees keys kt .. kt+lim-1 of the tile (keys past the
    // segment end have zero K rows, see load_tile)
    const bool need_mask = CAUSAL && t.kt + BN - 1 > wrow0 + t.ko;
    const int lim =
        need_mask ? (int)max(min(myrow + t.ko + 1 - t.kt, (int64_t)BN), (int64_t)0) : BN;
#pragma unroll
    for (int u = 0; u < BN / 32; ++u)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        bf16x8 x;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int idx = 8 * hh + e;
          float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[u][idx], c2, -lse2));
          if (need_mask && 32 * u + 8 * (idx / 4) + 4 * g + (idx % 4) >= lim) pv = 0.f;
          x[e] = (bf16)(pv * (pacc[u][idx] - dlt));  // dS^T (unscaled)
        }
        dsb[2 * u + hh] = x;
      }
  };

  // ---- prologue: tile 0 in buffer 0, each group's next tile in flight
  // (a job without key tiles skips all of it, so both groups meet the same barriers)
  It tw = tv;  // next tile this thread's group stages
  if (tv.r < nseg) {
    load_tile(tw);
    store_tile(0);
    advance(tw);
    if (tw.r < nseg) load_tile(tw);
    __syncthreads();
    if (!groupB) {
      phase_sdp(0);  // slot 0
    } else {
      if (tw.r < nseg) {  // slot 0: V(1)
        store_tile(1);
        advance(tw);
        if (tw.r < nseg) load_tile(tw);
      }
      __syncthreads();
      phase_sdp(0);  // slot 1
    }
#pragma unroll
    for (int u = 0; u < BN / 32; ++u) {
      hold(sacc[u]);
      hold(pacc[u]);
    }
    __syncthreads();
    // settle the prologue's global loads here, not inside the loop
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      hold(qreg[s]);
      hold(doreg[s]);
    }
    hold(lse2);
    hold(dlt);
    int it = 0;
    while (tv.r < nseg) {
      const int cur = it % 3;
      // Staged chunks go to LDS first, so that their registers are free during
      // dS; the next tile's loads are issued last and have the following MFMA
      // slot to land.
      const bool stage = tw.r < nseg;  // group A: K(it+1); group B: V(it+2)
      if (stage) store_tile(groupB ? (it + 2) % 3 : (it + 1) % 3);
      phase_ds(tv);
#pragma unroll
      for (int t = 0; t < BN / 16; ++t) hold(dsb[t]);
      if (stage) {
        advance(tw);
        if (tw.r < nseg) load_tile(tw);
      }
      __syncthreads();
      It tn = tv;
      advance(tn);
      mfma_slot(cur, (it + 1) % 3);  // after the last tile S/dP read a stale buffer, unused
#pragma unroll
      for (int u = 0; u < BN / 32; ++u) {
        hold(sacc[u]);
        hold(pacc[u]);
      }
      // group A closes this slot; group B's last MFMA slot is the final one
      if (!groupB || tn.r < nseg) __syncthreads();
      tv = tn;
      ++it;
    }
  }

  if (!row_ok) return;
  const float sc = p.scale;
  if (p.mode == MODE_ROUNDS) {
    float* dst = p.dq_acc + ((int64_t)bh * p.SQ + myrow) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 32 * dt + 8 * i + 4 * g;
        f32x4 a = f32x4{dq[dt][4 * i] * sc, dq[dt][4 * i + 1] * sc, dq[dt][4 * i + 2] * sc,
                        dq[dt][4 * i + 3] * sc};
        if (acc_in) a += *(const f32x4*)(dst + d);
        *(f32x4*)(dst + d) = a;
      }
  } else {
    bf16* dst = p.dq + b * p.sdq[0] + h * p.sdq[1] + myrow * p.sdq[2];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 32 * dt + 8 * i + 4 * g;
        *(u32x2*)(dst + d) = u32x2{pk_bf16(dq[dt][4 * i] * sc, dq[dt][4 * i + 1] * sc),
                                   pk_bf16(dq[dt][4 * i + 2] * sc, dq[dt][4 * i + 3] * sc)};
      }
  }
}

// fp32 [BH][S][D] accumulator -> bf16 tensor (ROUNDS mode, after the last round).
template <int D>
__global__ __launch_bounds__(256) void bwd_convert_kernel(const float* acc, bf16* out, int B,
                                                          int H, int S, int64_t s0, int64_t s1,
                                                          int64_t s2) {
  int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int64_t total = (int64_t)B * H * S * (D / 4);
  if (idx >= total) return;
  int64_t row = idx / (D / 4);
  int c = (int)(idx % (D / 4)) * 4;
  int64_t bh = row / S, i = row % S, b = bh / H, h = bh % H;
  f32x4 x = *(const f32x4*)(acc + row * D + c);
  *(u32x2*)(out + b * s0 + h * s1 + i * s2 + c) = u32x2{pk_bf16(x[0], x[1]), pk_bf16(x[2], x[3])};
}

// ---------------------------------------------------------------- host side

bool bwd_supported(int dtype, int Dh) { return dtype == 1 && (Dh == 64 || Dh == 128); }

static size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t bwd_workspace_bytes(int64_t BH, int64_t SQ, int64_t SKV, int Dh, int n, int mode) {
  (void)n;
  size_t bytes = a256((size_t)BH * SQ * 4);  // Delta
  if (mode == MODE_ROUNDS)
    bytes += a256((size_t)BH * SQ * Dh * 4) + 2 * a256((size_t)BH * SKV * Dh * 4);
  return bytes;
}

static void strides(const bwa_tensor* t, int64_t* s) {
  s[0] = t->sB;
  s[1] = t->sH;
  s[2] = t->sS;
}

// The launches of one backward pass for head dim D and causal order CM.
template <int D, int CM>
static hipError_t bwd_launch_all(BwdParams p, hipStream_t st) {
  const int64_t BH = (int64_t)p.B * p.H;
  int64_t nthr = BH * p.SQ * (D / 8);
  hipLaunchKernelGGL(bwd_delta_kernel<D>, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, st,
                     p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int BK = 128, BM = 32 * kDqWaves;
  const int kv_tiles = (int)(((p.SKV + p.n - 1) / p.n + BK - 1) / BK);
  const int q_tiles = (int)(((p.SQ + p.n - 1) / p.n + BM - 1) / BM);
  const int groups = (int)(BH * p.n);
  const int rounds = p.mode == MODE_ROUNDS ? p.n : 1;
  // FUSED dK/dV with at least one head per XCD: head-major grid
  const bool head_major = p.mode != MODE_ROUNDS && BH >= kNumXcd;
  for (int r = 0; r < rounds; ++r) {
    p.round = r;
    p.kv_tiles = head_major ? kv_tiles : 0;
    p.groups = head_major ? (int)BH : groups;
    p.tiles = head_major ? kv_tiles * p.n : kv_tiles;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CM>), dim3(xcd_grid_size(p.tiles, p.groups)),
                       dim3(64 * kDkdvWaves), 0, st, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    p.tiles = q_tiles;
    p.groups = groups;
    p.kv_tiles = 0;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CM>), dim3(xcd_grid_size(q_tiles, groups)),
                       dim3(64 * kDqWaves), 0, st, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (p.mode == MODE_ROUNDS) {
    int64_t tq = BH * p.SQ * (D / 4), tk = BH * p.SKV * (D / 4);
    hipLaunchKernelGGL(bwd_convert_kernel<D>, dim3((unsigned)((tq + 255) / 256)), dim3(256), 0, st,
                       p.dq_acc, p.dq, p.B, p.H, p.SQ, p.sdq[0], p.sdq[1], p.sdq[2]);
    hipLaunchKernelGGL(bwd_convert_kernel<D>, dim3((unsigned)((tk + 255) / 256)), dim3(256), 0, st,
                       p.dk_acc, p.dk, p.B, p.H, p.SKV, p.sdk[0], p.sdk[1], p.sdk[2]);
    hipLaunchKernelGGL(bwd_convert_kernel<D>, dim3((unsigned)((tk + 255) / 256)), dim3(256), 0, st,
                       p.dv_acc, p.dv, p.B, p.H, p.SKV, p.sdv[0], p.sdv[1], p.sdv[2]);
    e = hipGetLastError();
  }
  return e;
}

template <int D>
static hipError_t bwd_launch_d(const BwdParams& p, hipStream_t st) {
  if (p.causal == 2) return bwd_launch_all<D, 2>(p, st);
  if (p.causal == 1) return bwd_launch_all<D, 1>(p, st);
  return bwd_launch_all<D, 0>(p, st);
}

hipError_t bwd_run(const BwdArgs& a, hipStream_t st) {
  BwdParams p = {};
  p.q = (const bf16*)a.q->ptr;
  p.k = (const bf16*)a.k->ptr;
  p.v = (const bf16*)a.v->ptr;
  p.o = (const bf16*)a.o->ptr;
  p.dout = (const bf16*)a.dout->ptr;
  p.dq = (bf16*)a.dq->ptr;
  p.dk = (bf16*)a.dk->ptr;
  p.dv = (bf16*)a.dv->ptr;
  strides(a.q, p.sq);
  strides(a.k, p.sk);
  strides(a.v, p.sv);
  strides(a.o, p.so);
  strides(a.dout, p.sdo);
  strides(a.dq, p.sdq);
  strides(a.dk, p.sdk);
  strides(a.dv, p.sdv);
  p.lse = a.lse;
  p.B = (int)a.q->B;
  p.H = (int)a.q->H;
  p.SQ = (int)a.q->S;
  p.SKV = (int)a.k->S;
  p.n = a.n;
  p.sched = a.sched;
  p.mode = a.mode == MODE_ROUNDS ? MODE_ROUNDS : MODE_FUSED;
  p.causal = a.causal;
  p.nq = (p.mode == MODE_ROUNDS || p.causal == 2) ? p.n : 1;
  p.nk = p.nq;
  p.scale = a.scale;
  p.scale_log2 = a.scale * kLog2e;
  const int Dh = (int)a.q->D;
  const int64_t BH = (int64_t)p.B * p.H;
  char* ws = (char*)a.workspace;
  p.delta = (float*)ws;
  ws += a256((size_t)BH * p.SQ * 4);
  if (p.mode == MODE_ROUNDS) {
    p.dq_acc = (float*)ws;
    ws += a256((size_t)BH * p.SQ * Dh * 4);
    p.dk_acc = (float*)ws;
    ws += a256((size_t)BH * p.SKV * Dh * 4);
    p.dv_acc = (float*)ws;
  }
  return Dh == 64 ? bwd_launch_d<64>(p, st) : bwd_launch_d<128>(p, st);
}

}  // namespace bwa
