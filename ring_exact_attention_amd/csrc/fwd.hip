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

template <int D, int NW>
struct Bf16Fwd {
  static constexpr int BN = 8192 / D;          // keys per tile (64 for D=128)
  static constexpr int BM = 32 * NW;           // query rows per workgroup
  static constexpr int NT = 64 * NW;           // threads
  static constexpr int KS = D + 8;             // K row stride in LDS (elements), 16 B pad
  static constexpr int VS = D + 16;            // V row stride (elements), 32 B pad: the four
                                               // rows of a transposing read hit disjoint banks
  static constexpr int K_TILE = BN * KS;       // elements
  static constexpr int V_TILE = BN * VS;       // elements, row-major
  static constexpr int HALF = NT / 2;          // threads staging K (first half) / V (second)
  static constexpr int KC = (BN * D / 8) / HALF;   // 16-byte chunks per staging thread
  static constexpr int NLD = KC;                    // 16-byte loads in flight per thread
  static_assert(KC * HALF == BN * D / 8, "staging must divide evenly");
  static constexpr int LDS_BYTES = (2 * K_TILE + 2 * V_TILE) * 2;
};

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void fwd_bf16_kernel(FwdParams p) {
  using C = Bf16Fwd<D, NW>;
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
        const bf16* a0 = vbase + (16 * t + 4 * g) * VS + 32 * dt;
        s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0));
        s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0 + 8 * VS));
        u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        u32x4 av = u32x4{l2[0], l2[1], h2[0], h2[1]};
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pb[t],
                                                           oacc[dt], 0, 0, 0);
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

template <int D, int NW>
static hipError_t launch_bf16(FwdParams p, int blocks, hipStream_t st) {
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW>), dim3(blocks), dim3(64 * NW), 0, st, p);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_f32(FwdParams p, int blocks, hipStream_t st) {
  hipLaunchKernelGGL((fwd_f32_kernel<D>), dim3(blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

constexpr int kFwdWaves = 8;

// Query rows per workgroup for a dtype / head dim.
int fwd_tile_rows(int dtype_bf16, int D) {
  (void)D;
  return dtype_bf16 ? Bf16Fwd<128, kFwdWaves>::BM : F32Fwd<128>::BM;
}

// Launch one forward pass over p.groups x p.tiles workgroups.
hipError_t fwd_launch(FwdParams p, int dtype_bf16, hipStream_t st) {
  int blocks = xcd_grid_size(p.tiles, p.groups);
  if (blocks == 0) return hipSuccess;
  if (dtype_bf16) {
    if (p.D == 128) return launch_bf16<128, kFwdWaves>(p, blocks, st);
    return launch_bf16<64, kFwdWaves>(p, blocks, st);
  }
  if (p.D == 128) return launch_f32<128>(p, blocks, st);
  return launch_f32<64>(p, blocks, st);
}

}  // namespace bwa
