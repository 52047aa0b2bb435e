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
#include <cstdlib>

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

// Materialise a value here: an empty volatile asm that claims to modify it.  Used
// to keep a phase's results from being sunk past a barrier into the next phase.
template <typename T>
__device__ inline void pin(T& x) {
  asm volatile("" : "+v"(x));
}

// Growth of a row maximum (log2 units) tolerated before the O accumulator is rescaled.
constexpr float kLazyRescale = 8.f;

#ifndef BWA_INTERLEAVE
#define BWA_INTERLEAVE 1
#endif
// Ask the scheduler to alternate MFMAs with VALU work and LDS reads in the
// pipelined main loop.
constexpr bool kInterleave = BWA_INTERLEAVE != 0;

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

template <int D, int NW, int BN_ = 8192 / D, bool VOCT_ = false>
struct Bf16Fwd {
  static constexpr int BN = BN_;               // keys per tile
  // V^T operand layout: false = row-major with a 32-byte pad, read by two
  // ds_read_b64_tr_b16; true = "octets": for each head dim the 8 keys one MFMA
  // lane needs (16t+4g+{0..3}, 16t+8+4g+{0..3}) are 16 contiguous bytes, read by
  // one ds_read_b128; entry d of an octet row sits at slot d ^ ((d >> 3) & 15)
  // (with a 16-byte row pad) so staging writes and operand reads avoid bank
  // conflicts.  The octet layout is transposed in registers while staging.
  static constexpr bool VOCT = VOCT_;
  static constexpr int OSTR = D * 8 + 8;       // octet row stride (elements)
  static constexpr int BM = 32 * NW;           // query rows per workgroup
  static constexpr int NT = 64 * NW;           // threads
  static constexpr int KS = D + 8;             // K row stride in LDS (elements), 16 B pad
  static constexpr int VS = D + 16;            // V row stride (elements), 32 B pad: the four
                                               // rows of a transposing read hit disjoint banks
  static constexpr int K_TILE = BN * KS;       // elements
  static constexpr int V_TILE = VOCT ? (BN / 8) * OSTR : BN * VS;
  static constexpr int HALF = NT / 2;          // threads staging K (first half) / V (second)
  static constexpr int KC = (BN * D / 8) / HALF;   // 16-byte chunks per staging thread
  static constexpr int NLD = KC;                    // 16-byte loads in flight per thread
  static_assert(KC * HALF == BN * D / 8, "staging must divide evenly");
  // octet staging: V threads take 4-row x 8-column items, KC / 4 each
  static_assert(!VOCT || (KC % 4 == 0 && (KC / 4) * HALF == (BN / 4) * (D / 8)),
                "octet staging must divide evenly");
  static constexpr int LDS_BYTES = (2 * K_TILE + 2 * V_TILE) * 2;
};

template <int D, int NW, int BN_ = 8192 / D, int MINB = 1, bool VOCT = false>
__global__ __launch_bounds__(64 * NW, MINB) void fwd_bf16_kernel(FwdParams p) {
  using C = Bf16Fwd<D, NW, BN_, VOCT>;
  constexpr int BN = C::BN, KS = C::KS, VS = C::VS, HALF = C::HALF;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * C::K_TILE + 2 * C::V_TILE];
  bf16* Ks = smem;                     // [2][BN][KS]
  bf16* Vs = smem + 2 * C::K_TILE;     // [2][BN][KS]

  Job jb;
  if (!make_job(p, C::BM, &jb)) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 31;  // query column of this lane within the wave
  const int g = lane >> 5;   // half-wave
  const int b = jb.bh / p.H, h = jb.bh % p.H;

  const bf16* qg = (const bf16*)p.q + b * p.sqB + h * p.sqH;
  const bf16* kg = (const bf16*)p.k + b * p.skB + h * p.skH;
  const bf16* vg = (const bf16*)p.v + b * p.svB + h * p.svH;

  const int64_t wrow0 = jb.r0 + wave * 32;  // first query row of this wave
  const int64_t myrow = wrow0 + lr;
  const bool row_ok = myrow < jb.r1;

  // Q^T as MFMA B operands: lane holds query myrow, dims 16s + 8g .. +7.
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    if (row_ok) qreg[s] = *(const bf16x8*)(qg + myrow * p.sqS + 16 * s + 8 * g);
    else qreg[s] = bf16x8{};
  }

  // Running state: m2 (log2 domain, scale folded in), lane-partial l, O^T accumulators.
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

  TileIter it;
  it.seek(p, jb, 0, BN);
  if (!it.valid(jb) && jb.epi == EPI_ACC && jb.acc_in) return;  // skipped pair: state unchanged

  // ---- staging: global -> registers -> LDS
  u32x4 stg[C::NLD];
  auto load_tile = [&](int64_t kt, int64_t ke) {
    const bf16* src = tid < HALF ? kg : vg;
    const int64_t ss = tid < HALF ? p.skS : p.svS;
    const int t2 = tid < HALF ? tid : tid - HALF;
    if (VOCT && tid >= HALF) {
#pragma unroll
      for (int i = 0; i < C::KC / 4; ++i) {
        const int itm = t2 + i * HALF;
        const int quad = itm / (D / 8), col8 = itm % (D / 8);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          int64_t key = kt + 4 * quad + rr;
          stg[4 * i + rr] = key < ke ? *(const u32x4*)(vg + key * p.svS + col8 * 8) : u32x4{};
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < C::KC; ++i) {
      int c = t2 + i * HALF;
      int row = c / (D / 8), col8 = c % (D / 8);
      int64_t key = kt + row;
      stg[i] = key < ke ? *(const u32x4*)(src + key * ss + col8 * 8) : u32x4{};
    }
  };
  auto store_tile = [&](int buf) {
    bf16* dst = (tid < HALF ? Ks + buf * C::K_TILE : Vs + buf * C::V_TILE);
    const int t2 = tid < HALF ? tid : tid - HALF;
    const int rs = tid < HALF ? KS : VS;
    if (VOCT && tid >= HALF) {
#pragma unroll
      for (int i = 0; i < C::KC / 4; ++i) {
        // rows 4q..4q+3 = keys 16t + 8ii + 4g + 0..3, columns 8*col8 .. +7
        const int itm = t2 + i * HALF;
        const int quad = itm / (D / 8), col8 = itm % (D / 8);
        const int oct = 2 * (quad >> 2) + (quad & 1), ii = (quad >> 1) & 1;
        bf16* orow = dst + oct * C::OSTR + 4 * ii;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const u32x4 r0 = stg[4 * i], r1 = stg[4 * i + 1], r2 = stg[4 * i + 2], r3 = stg[4 * i + 3];
          const uint32_t lo01 = (r0[w] & 0xffffu) | (r1[w] << 16);
          const uint32_t lo23 = (r2[w] & 0xffffu) | (r3[w] << 16);
          const uint32_t hi01 = (r0[w] >> 16) | (r1[w] & 0xffff0000u);
          const uint32_t hi23 = (r2[w] >> 16) | (r3[w] & 0xffff0000u);
          const int d0 = 8 * col8 + 2 * w, d1 = d0 + 1;
          *(u32x2*)(orow + 8 * (d0 ^ ((d0 >> 3) & 15))) = u32x2{lo01, lo23};
          *(u32x2*)(orow + 8 * (d1 ^ ((d1 >> 3) & 15))) = u32x2{hi01, hi23};
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < C::KC; ++i) {
      int c = t2 + i * HALF;
      int row = c / (D / 8), col8 = c % (D / 8);
      *(u32x4*)(dst + row * rs + col8 * 8) = stg[i];
    }
  };

  int buf = 0;
  if (it.valid(jb)) {
    load_tile(it.kt, it.ke);
    store_tile(0);
  }
  __syncthreads();

  const float c2 = p.scale_log2;
  while (it.valid(jb)) {
    TileIter nx = it;
    nx.advance(p, jb, BN);
    const bool more = nx.valid(jb);
    if (more) load_tile(nx.kt, nx.ke);

    const bf16* kt_s = Ks + buf * C::K_TILE;
    const bf16* vt_s = Vs + buf * C::V_TILE;

    // S^T = K Q^T for BN keys x 32 queries
    f32x16 sacc[BN / 32];
#pragma unroll
    for (int u = 0; u < BN / 32; ++u) sacc[u] = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
#pragma unroll
      for (int u = 0; u < BN / 32; ++u) {
        bf16x8 a = *(const bf16x8*)(kt_s + (32 * u + lr) * KS + 16 * s + 8 * g);
        sacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], sacc[u], 0, 0, 0);
      }
    }

    // mask keys past the segment end and, under causal masking, keys after the row
    const int64_t kt = it.kt;
    const bool need_mask = (kt + BN > it.ke) || (p.causal && kt + BN - 1 > wrow0);
    if (need_mask) {
#pragma unroll
      for (int u = 0; u < BN / 32; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            int64_t key = kt + 32 * u + 8 * i + 4 * g + jj;
            bool vis = key < it.ke && (!p.causal || key <= myrow);
            if (!vis) sacc[u][4 * i + jj] = -INFINITY;
          }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < BN / 32; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[u][e]);
    mx = wave_swap32_max(mx);
    const float m_cand = fmaxf(m2, mx * c2);
    if (__builtin_amdgcn_ballot_w64(m_cand > m2 + kLazyRescale) != 0) {
      // some row's maximum grew by more than 2^8: move every row to its new maximum
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
    bf16x8 pb[BN / 16];
#pragma unroll
    for (int u = 0; u < BN / 32; ++u)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = fast_exp2(__builtin_fmaf(sacc[u][8 * hh + e], c2, -m_use));
          ts[e & 3] += pv[e];
        }
        bf16x8 x;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (bf16)pv[e];
        pb[2 * u + hh] = x;
      }
    lsum += (ts[0] + ts[1]) + (ts[2] + ts[3]);

    // O^T += V^T P^T.  A operand rows d = 32*dt + lane%32, keys 16t + 4g + {0..3}
    // and 16t + 8 + 4g + {0..3}: two transposing reads of 4-row blocks.
    const int li = lane & 15;
    const bf16* vbase = vt_s + (li >> 2) * VS + ((lane >> 4) & 1) * 16 + 4 * (li & 3);
#pragma unroll
    for (int t = 0; t < BN / 16; ++t) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        bf16x8 av;
        if constexpr (VOCT) {
          const int d = 32 * dt + lr;
          av = *(const bf16x8*)(vt_s + (2 * t + g) * C::OSTR + 8 * (d ^ ((d >> 3) & 15)));
        } else {
          const bf16* a0 = vbase + (16 * t + 4 * g) * VS + 32 * dt;
          s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0));
          s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0 + 8 * VS));
          u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
          av = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
        }
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[t], oacc[dt], 0, 0, 0);
      }
    }

    if (!more) break;
    store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    it = nx;
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

// ------------------------------------------------------------------ bf16 MFMA kernel, 64 rows per wave
//
// D = 128.  Four waves, each owning 64 query rows as two 32-column blocks, so
// every K operand and every V^T operand read from LDS feeds two MFMAs (half
// the LDS bytes per MFMA of the 32-row kernel).  One wave per SIMD; the
// MFMA/softmax overlap comes from software pipelining inside the wave:
// while tile j's exponentials are computed, the S^T MFMAs of tile j+1 are
// already in flight, and tile j+1's row maxima are reduced while tile j's PV
// MFMAs run.  K/V tiles rotate through three LDS buffers (tile j+2 is written
// while j and j+1 are read), so one barrier per tile suffices.

template <int NCB_, int NW_, int BN_, bool VOCT_>
struct PipeFwd {
  static constexpr int D = 128, NCB = NCB_, NW = NW_, NT = 64 * NW_, BN = BN_;
  static constexpr int BM = 32 * NCB * NW;  // query rows per workgroup
  static constexpr int NU = BN / 32;        // 32-key blocks per tile
  static constexpr int KS = D + 8;
  // V^T operand layout ("octets"): for each head dim d, the 8 keys one MFMA lane
  // needs -- 16t+4g+{0..3} and 16t+8+4g+{0..3} -- are 16 contiguous bytes, so the
  // operand is a single ds_read_b128.  Octet o = 2t+g is a row of D entries
  // (plus a 16-byte pad); entry d sits at slot d ^ ((d >> 3) & 15), which keeps
  // both the staging writes and the operand reads free of bank conflicts.
  static constexpr bool VOCT = VOCT_;
  static constexpr int NOCT = BN / 8;
  static constexpr int OSTR = D * 8 + 8;             // octet row stride (elements)
  // Alternative V layout: row-major with a 32-byte pad, read with ds_read_b64_tr_b16.
  static constexpr int VS = D + 16;
  static constexpr int K_TILE = BN * KS, V_TILE = VOCT ? NOCT * OSTR : BN * VS;
  static constexpr int STAGE = K_TILE + V_TILE;      // elements per buffer
  static constexpr int NBUF = 3;
  static constexpr int KTHR = NT / 2;                // threads staging K (the rest stage V)
  static constexpr int KC = (BN * D / 8) / KTHR;     // 16-byte chunks per staging thread
  static constexpr int VITEMS = (BN / 4) * (D / 8);  // octet layout: 4-row x 8-column items
  static_assert(KC * KTHR == BN * D / 8, "K staging must divide evenly");
  static_assert(!VOCT || VITEMS <= NT - KTHR, "one V item per V thread");
  static constexpr int NSTG = (VOCT && KC < 4) ? 4 : KC;  // staging registers (u32x4)
};

template <int NCB, int NW, int BN_, bool VOCT>
__global__ __launch_bounds__(64 * NW) void fwd_bf16_pipe_kernel(FwdParams p) {
  using C = PipeFwd<NCB, NW, BN_, VOCT>;
  constexpr int D = C::D, BN = C::BN, KS = C::KS, NU = C::NU, KTHR = C::KTHR;
  __shared__ __attribute__((aligned(16))) bf16 smem[C::NBUF * C::STAGE];

  Job jb;
  if (!make_job(p, C::BM, &jb)) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 31;
  const int g = lane >> 5;
  const int b = jb.bh / p.H, h = jb.bh % p.H;
  const bf16* qg = (const bf16*)p.q + b * p.sqB + h * p.sqH;
  const bf16* kg = (const bf16*)p.k + b * p.skB + h * p.skH;
  const bf16* vg = (const bf16*)p.v + b * p.svB + h * p.svH;

  const int64_t wrow0 = jb.r0 + wave * 32 * NCB;  // rows wrow0 + 32c + lane%32
  int64_t myrow[NCB];
  bool row_ok[NCB];
  bf16x8 qreg[NCB][D / 16];
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    myrow[c] = wrow0 + 32 * c + lr;
    row_ok[c] = myrow[c] < jb.r1;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qreg[c][s] = row_ok[c] ? *(const bf16x8*)(qg + myrow[c] * p.sqS + 16 * s + 8 * g)
                             : bf16x8{};
  }

  float m2[NCB], lsum[NCB];
  f32x16 oacc[NCB][D / 32];
#pragma unroll
  for (int c = 0; c < NCB; ++c) { m2[c] = -INFINITY; lsum[c] = 0.f; }
#pragma unroll
  for (int c = 0; c < NCB; ++c)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) oacc[c][dt] = f32x16{};

  const int64_t BH = (int64_t)p.B * p.H;
  if (jb.epi == EPI_ACC && jb.acc_in) {
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      float lp = row_ok[c] ? p.lse[jb.bh * p.SQ + myrow[c]] : -INFINITY;
      if (lp != -INFINITY) {
        m2[c] = lp * kLog2e;
        lsum[c] = (g == 0) ? 1.f : 0.f;
        const float* src = p.o_acc + (jb.bh * p.SQ + myrow[c]) * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            f32x4 x = *(const f32x4*)(src + 32 * dt + 8 * i + 4 * g);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) oacc[c][dt][4 * i + jj] = x[jj];
          }
      }
    }
  }

  TileIter it;
  it.seek(p, jb, 0, BN);
  if (!it.valid(jb) && jb.epi == EPI_ACC && jb.acc_in) return;  // skipped pair

  u32x4 stg[C::NSTG];
  const bool kthr = tid < KTHR;
  const int vitem = tid - KTHR;  // V item of this thread (if in range)
  auto load_tile = [&](const TileIter& t) {
    if (kthr) {
#pragma unroll
      for (int i = 0; i < C::KC; ++i) {
        int cc = tid + i * KTHR;
        int row = cc / (D / 8), col8 = cc % (D / 8);
        int64_t key = t.kt + row;
        stg[i] = key < t.ke ? *(const u32x4*)(kg + key * p.skS + col8 * 8) : u32x4{};
      }
    } else if (!VOCT) {
#pragma unroll
      for (int i = 0; i < C::KC; ++i) {
        int cc = vitem + i * KTHR;
        int row = cc / (D / 8), col8 = cc % (D / 8);
        int64_t key = t.kt + row;
        stg[i] = key < t.ke ? *(const u32x4*)(vg + key * p.svS + col8 * 8) : u32x4{};
      }
    } else if (vitem < C::VITEMS) {
      const int quad = vitem / (D / 8), col8 = vitem % (D / 8);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        int64_t key = t.kt + 4 * quad + rr;
        stg[rr] = key < t.ke ? *(const u32x4*)(vg + key * p.svS + col8 * 8) : u32x4{};
      }
    }
  };
  auto store_tile = [&](int buf) {
    bf16* base = smem + buf * C::STAGE;
    if (kthr) {
#pragma unroll
      for (int i = 0; i < C::KC; ++i) {
        int cc = tid + i * KTHR;
        int row = cc / (D / 8), col8 = cc % (D / 8);
        *(u32x4*)(base + row * KS + col8 * 8) = stg[i];
      }
    } else if (!VOCT) {
#pragma unroll
      for (int i = 0; i < C::KC; ++i) {
        int cc = vitem + i * KTHR;
        int row = cc / (D / 8), col8 = cc % (D / 8);
        *(u32x4*)(base + C::K_TILE + row * C::VS + col8 * 8) = stg[i];
      }
    } else if (vitem < C::VITEMS) {
      // rows 4q..4q+3 (keys 16t + 8ii + 4g + 0..3), columns 8*col8 .. +7
      const int quad = vitem / (D / 8), col8 = vitem % (D / 8);
      const int oct = 2 * (quad >> 2) + (quad & 1), ii = (quad >> 1) & 1;
      bf16* orow = base + C::K_TILE + oct * C::OSTR + 4 * ii;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t lo01 = (stg[0][w] & 0xffffu) | (stg[1][w] << 16);
        const uint32_t lo23 = (stg[2][w] & 0xffffu) | (stg[3][w] << 16);
        const uint32_t hi01 = (stg[0][w] >> 16) | (stg[1][w] & 0xffff0000u);
        const uint32_t hi23 = (stg[2][w] >> 16) | (stg[3][w] & 0xffff0000u);
        const int d0 = 8 * col8 + 2 * w, d1 = d0 + 1;
        *(u32x2*)(orow + 8 * (d0 ^ ((d0 >> 3) & 15))) = u32x2{lo01, lo23};
        *(u32x2*)(orow + 8 * (d1 ^ ((d1 >> 3) & 15))) = u32x2{hi01, hi23};
      }
    }
  };
  // S^T (keys x queries) of the tile in `buf` for both column blocks
  auto s_mfma = [&](int buf, f32x16 (&out)[NCB][NU]) {
    const bf16* ks = smem + buf * C::STAGE;
#pragma unroll
    for (int c = 0; c < NCB; ++c)
#pragma unroll
      for (int u = 0; u < NU; ++u) out[c][u] = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        bf16x8 a = *(const bf16x8*)(ks + (32 * u + lr) * KS + 16 * s + 8 * g);
#pragma unroll
        for (int c = 0; c < NCB; ++c)
          out[c][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[c][s], out[c][u], 0, 0, 0);
      }
  };
  // mask keys past the segment end and, under causal masking, keys after the row
  auto apply_mask = [&](const TileIter& t, f32x16 (&sc)[NCB][NU]) {
    const bool need = (t.kt + BN > t.ke) || (p.causal && t.kt + BN - 1 > wrow0);
    if (!need) return;
#pragma unroll
    for (int c = 0; c < NCB; ++c)
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            int64_t key = t.kt + 32 * u + 8 * i + 4 * g + jj;
            bool vis = key < t.ke && (!p.causal || key <= myrow[c]);
            if (!vis) sc[c][u][4 * i + jj] = -INFINITY;
          }
  };
  auto row_max = [&](const f32x16 (&sc)[NCB][NU], float (&mx)[NCB]) {
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      float m = -INFINITY;
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) m = fmaxf(m, sc[c][u][e]);
      mx[c] = wave_swap32_max(m);
    }
  };

  // ---- prologue: tiles 0 and 1 into buffers 0 and 1, S of tile 0, loads of tile 2
  TileIter it1 = it;
  if (it1.valid(jb)) it1.advance(p, jb, BN);
  TileIter it2 = it1;
  if (it2.valid(jb)) it2.advance(p, jb, BN);
  if (it.valid(jb)) {
    load_tile(it);
    store_tile(0);
  }
  if (it1.valid(jb)) {
    load_tile(it1);
    store_tile(1);
  }
  __syncthreads();
  f32x16 scur[NCB][NU];
  float mx[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) mx[c] = -INFINITY;
  if (it.valid(jb)) {
    s_mfma(0, scur);
    apply_mask(it, scur);
    row_max(scur, mx);
  }
  if (it2.valid(jb)) load_tile(it2);

  const float c2 = p.scale_log2;
  int cur = 0;
  bool first = true;
  while (it.valid(jb)) {
    const int nxt = cur == 2 ? 0 : cur + 1;
    const int nn = nxt == 2 ? 0 : nxt + 1;
    if (!first) {
      apply_mask(it, scur);
      row_max(scur, mx);
    }
    first = false;
    // lazy rescale (rare): only when some row maximum grew by more than 2^8
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const float m_cand = fmaxf(m2[c], mx[c] * c2);
      if (__builtin_amdgcn_ballot_w64(m_cand > m2[c] + kLazyRescale) != 0) {
        const float alpha = fast_exp2(m2[c] - ((m_cand == -INFINITY) ? 0.f : m_cand));
        lsum[c] *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[c][dt][e] *= alpha;
        m2[c] = m_cand;
      }
    }

    // S^T of the next tile (stale buffer contents when there is none: result unused)
    f32x16 snext[NCB][NU];
    s_mfma(nxt, snext);

    // P of this tile: exp2, row sums, bf16 B operands
    bf16x8 pb[NCB][BN / 16];
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const float mu = (m2[c] == -INFINITY) ? 0.f : m2[c];
      float ts[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          bf16x8 x;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float pv = fast_exp2(__builtin_fmaf(scur[c][u][8 * hh + e], c2, -mu));
            ts[e & 3] += pv;
            x[e] = (bf16)pv;
          }
          pb[c][2 * u + hh] = x;
        }
      lsum[c] += (ts[0] + ts[1]) + (ts[2] + ts[3]);
    }

    // O^T += V^T P^T; each V^T operand feeds every column block
    {
      const bf16* vt_s = smem + cur * C::STAGE + C::K_TILE;
      const int li = lane & 15;
      const bf16* vbase = vt_s + (li >> 2) * C::VS + ((lane >> 4) & 1) * 16 + 4 * (li & 3);
#pragma unroll
      for (int t = 0; t < BN / 16; ++t)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          bf16x8 av;
          if constexpr (VOCT) {
            const int d = 32 * dt + lr;
            av = *(const bf16x8*)(vt_s + (2 * t + g) * C::OSTR + 8 * (d ^ ((d >> 3) & 15)));
          } else {
            // two transposing reads of 4-row blocks: keys 16t+4g+{0..3}, 16t+8+4g+{0..3}
            const bf16* a0 = vbase + (16 * t + 4 * g) * C::VS + 32 * dt;
            s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0));
            s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0 + 8 * C::VS));
            u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
            av = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
          }
#pragma unroll
          for (int c = 0; c < NCB; ++c)
            oacc[c][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[c][t], oacc[c][dt], 0, 0, 0);
        }
    }
    // interleave the region's MFMAs with its VALU work and LDS reads
    if constexpr (kInterleave) {
#pragma unroll
      for (int i = 0; i < 2 * NCB * NU * (D / 16); ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // three VALU
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      }
    }


    // stage tile j+2 into the buffer tile j-1 used, then fetch tile j+3
    if (it2.valid(jb)) store_tile(nn);
    TileIter it3 = it2;
    if (it3.valid(jb)) {
      it3.advance(p, jb, BN);
      if (it3.valid(jb)) load_tile(it3);
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < NCB; ++c)
#pragma unroll
      for (int u = 0; u < NU; ++u) scur[c][u] = snext[c][u];
    cur = nxt;
    it = it1;
    it1 = it2;
    it2 = it3;
  }

  // ---- epilogue
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    const float ltot = wave_swap32_sum(lsum[c]);
    const bool empty = (m2[c] == -INFINITY) || !(ltot > 0.f);
    const float inv = empty ? 0.f : 1.f / ltot;
    const float lse = empty ? -INFINITY : (m2[c] + __log2f(ltot)) * kLn2;
    if (!row_ok[c]) continue;
    if (jb.epi == EPI_FINAL) {
      bf16* dst = (bf16*)p.o + b * p.soB + h * p.soH + myrow[c] * p.soS;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          store4<bf16>(dst + 32 * dt + 8 * i + 4 * g, oacc[c][dt][4 * i] * inv,
                       oacc[c][dt][4 * i + 1] * inv, oacc[c][dt][4 * i + 2] * inv,
                       oacc[c][dt][4 * i + 3] * inv);
      if (g == 0) p.lse[jb.bh * p.SQ + myrow[c]] = lse;
    } else {
      float* obase = p.o_acc;
      float* lbase = p.lse;
      if (jb.epi == EPI_PART) {
        obase += (int64_t)jb.block * BH * p.SQ * D;
        lbase = p.lse_part + (int64_t)jb.block * BH * p.SQ;
      }
      float* dst = obase + (jb.bh * p.SQ + myrow[c]) * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          store4<float>(dst + 32 * dt + 8 * i + 4 * g, oacc[c][dt][4 * i] * inv,
                        oacc[c][dt][4 * i + 1] * inv, oacc[c][dt][4 * i + 2] * inv,
                        oacc[c][dt][4 * i + 3] * inv);
      if (g == 0) lbase[jb.bh * p.SQ + myrow[c]] = lse;
    }
  }
}

// ------------------------------------------------------------------ bf16 MFMA kernel, ping-pong
//
// D = 128, 256 query rows per workgroup, 8 waves of 32 rows, 64-key tiles.
// A wave's work per tile alternates between an MFMA phase (PV of tile j
// followed by S of tile j+1) and a VALU phase (mask, max, exp2, row sums and
// the bf16 P of tile j+1).  Waves 0-3 (group A) and 4-7 (group B) share the
// four SIMDs one each and run one phase apart: between any two barriers one
// wave of every SIMD is in its MFMA phase while the other is in its VALU
// phase, so the matrix core and the vector ALU work at the same time.
// Barrier intervals ("slots") are numbered from 0; group A runs
//   slot 0: S(0);  slot 2j+1: softmax(j) + write K(j+1);  slot 2j+2: PV(j) + S(j+1)
// and group B runs the same sequence one slot later (writing V(j+1) in its
// softmax slot).  K/V tiles rotate through three LDS buffers; a tile is read
// from slot 2j to slot 2j+3 and the buffer it overwrites was last read two
// slots earlier.

template <int BN_>
struct PPFwd {
  static constexpr int D = 128, NW = 8, NT = 512, BM = 256, BN = BN_;
  static constexpr int KS = D + 8, VS = D + 16;
  static constexpr int K_TILE = BN * KS, V_TILE = BN * VS;
  static constexpr int STAGE = K_TILE + V_TILE;
  static constexpr int NBUF = 3;
  static constexpr int GT = NT / 2;                // threads per group
  static constexpr int KC = (BN * D / 8) / GT;     // 16-byte chunks per staging thread
  static_assert(KC * GT == BN * D / 8, "staging must divide evenly");
};

template <int BN_, bool GROUP = false>
__global__ __launch_bounds__(512) void fwd_bf16_pp_kernel(FwdParams p) {
  using C = PPFwd<BN_>;
  constexpr int D = C::D, BN = C::BN, KS = C::KS, VS = C::VS;
  __shared__ __attribute__((aligned(16))) bf16 smem[C::NBUF * C::STAGE];

  Job jb;
  if (!make_job(p, C::BM, &jb)) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
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
  auto load_tile = [&](const TileIter& t) {
#pragma unroll
    for (int i = 0; i < C::KC; ++i) {
      int cc = gtid + i * C::GT;
      int row = cc / (D / 8), col8 = cc % (D / 8);
      int64_t key = t.kt + row;
      stg[i] = key < t.ke ? *(const u32x4*)(ssrc + key * sstr + col8 * 8) : u32x4{};
    }
  };
  auto store_tile = [&](int buf) {
    bf16* dst = smem + buf * C::STAGE + soff;
#pragma unroll
    for (int i = 0; i < C::KC; ++i) {
      int cc = gtid + i * C::GT;
      int row = cc / (D / 8), col8 = cc % (D / 8);
      *(u32x4*)(dst + row * srs + col8 * 8) = stg[i];
    }
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
    const bool need_mask = (t.kt + BN > t.ke) || (p.causal && t.kt + BN - 1 > wrow0);
    if (need_mask) {
#pragma unroll
      for (int u = 0; u < BN / 32; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            int64_t key = t.kt + 32 * u + 8 * i + 4 * g + jj;
            bool vis = key < t.ke && (!p.causal || key <= myrow);
            if (!vis) sacc[u][4 * i + jj] = -INFINITY;
          }
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
    if constexpr (GROUP) {
      // issue every PV operand read first, then let the K reads of the next S
      // overlap the PV MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (BN / 16) * (D / 32), 0);
      __builtin_amdgcn_sched_group_barrier(0x008, (BN / 16) * (D / 32) / 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, (BN / 32) * (D / 16) / 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, (BN / 16) * (D / 32) / 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, (BN / 32) * (D / 16) / 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, (BN / 32) * (D / 16), 0);
    }
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
      int64_t key = it.kt + j;
      bool vis = key < it.ke && (!p.causal || key <= myrow);
      if (!vis) continue;  // uniform across the four lanes of a row
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

template <int D, int NW, int BN = 8192 / D, int MINB = 1, bool VOCT = false>
static hipError_t launch_bf16(FwdParams p, int blocks, hipStream_t st) {
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, BN, MINB, VOCT>), dim3(blocks), dim3(64 * NW), 0, st,
                     p);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_f32(FwdParams p, int blocks, hipStream_t st) {
  hipLaunchKernelGGL((fwd_f32_kernel<D>), dim3(blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

constexpr int kFwdWaves = 8;

static int fwd_variant() {
  static const int variant = [] {
    const char* e = getenv("BWA_FWD_VARIANT");
    return e ? atoi(e) : 0;
  }();
  return variant;
}

// Query rows per workgroup for a dtype / head dim.
int fwd_tile_rows(int dtype_bf16, int D) {
  if (!dtype_bf16) return F32Fwd<128>::BM;
  if (D == 128 && (fwd_variant() == 5 || fwd_variant() == 6)) return 128;
  return 256;
}

// Launch one forward pass over p.groups x p.tiles workgroups.
hipError_t fwd_launch(FwdParams p, int dtype_bf16, hipStream_t st) {
  int blocks = xcd_grid_size(p.tiles, p.groups);
  if (blocks == 0) return hipSuccess;
  if (dtype_bf16) {
    if (p.D == 128) {
      switch (fwd_variant()) {
        case 1: hipLaunchKernelGGL((fwd_bf16_pipe_kernel<1, 8, 32, true>), dim3(blocks), dim3(512), 0, st, p); break;
        case 2: hipLaunchKernelGGL((fwd_bf16_pipe_kernel<1, 8, 32, false>), dim3(blocks), dim3(512), 0, st, p); break;
        case 3: hipLaunchKernelGGL((fwd_bf16_pipe_kernel<2, 4, 32, false>), dim3(blocks), dim3(256), 0, st, p); break;
        case 4: return launch_bf16<128, 8, 32>(p, blocks, st);
        case 5: return launch_bf16<128, 4, 32, 3>(p, blocks, st);
        case 6: return launch_bf16<128, 4, 32, 2>(p, blocks, st);
        case 7: return launch_bf16<128, 8, 64, 1, true>(p, blocks, st);
        case 8: hipLaunchKernelGGL((fwd_bf16_pp_kernel<64>), dim3(blocks), dim3(512), 0, st, p); break;
        case 9: hipLaunchKernelGGL((fwd_bf16_pp_kernel<32>), dim3(blocks), dim3(512), 0, st, p); break;
        case 10: hipLaunchKernelGGL((fwd_bf16_pp_kernel<32, true>), dim3(blocks), dim3(512), 0, st, p); break;
        default: return launch_bf16<128, kFwdWaves>(p, blocks, st);
      }
      return hipGetLastError();
    }
    return launch_bf16<64, kFwdWaves>(p, blocks, st);
  }
  if (p.D == 128) return launch_f32<128>(p, blocks, st);
  return launch_f32<64>(p, blocks, st);
}

}  // namespace bwa
