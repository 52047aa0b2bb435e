// K/V recompute from the one shared copy of the visual features (LV-XAttn
// review, "What carries the argument": all cross-attention layers read the
// same y, so y is kept once and K = y W_k, V = y W_v are recomputed when
// needed).
//
//   out[b, h, s, d] = sum_e y[b, s, e] * W[e, h*D + d],  W stored transposed
//   as w_t[n, e] (n = h*D + d), the [out, in] layout of a linear layer.
//
// The kernel computes the transposed product C^T[n, s] = w_t[n, :] . y[s, :]
// on v_mfma_f32_16x16x32_bf16, so that each lane of a 16x16 output block owns
// four consecutive n (= four consecutive head dims d) of one key row s and
// stores them as one 8-byte write into the [B, H, S, D] output.  Both
// operands keep the contraction index e contiguous in memory and in LDS.
//
// Tiling: 256 (n) x 256 (s) per workgroup of 8 waves (2 x 4, two per SIMD),
// 128 x 64 per wave (8 x 4 MFMA blocks, fp32 accumulators), 64 e per LDS
// stage (128 contiguous bytes per row and load), double buffered in 160 KB of
// LDS with rows padded by 32 bytes: rows 160 bytes apart (an odd multiple of
// 32 mod 256) keep the 16-byte operand reads of the 16x16x32 layout free of
// bank conflicts, where 144-byte rows conflicted in 37% of the LDS cycles.
// Within a stage the 64 MFMAs of a wave are issued in a fixed order, rows of
// blocks one after the other: a row's A operand is read three rows ahead, and
// the B operands of the next 32-element k-step while its row 5 runs.  The chunks staged for the next stage go to the
// other buffer one every four MFMAs of the first k-step, each followed one
// MFMA later by the load (into the same registers) of that chunk for the
// stage after it, which then has a whole stage to land.  Bursts of wide LDS
// writes fill the LDS data FIFO and stall every wave's LDS reads; spreading
// them and the reads over the MFMAs is worth 14% here.  The stage's barrier
// comes before the last three block rows, whose operands are already in
// registers, so the next stage's first operand reads overlap those MFMAs
// instead of idling the matrix core after the barrier.
//
// The 16x16x32 MFMA rather than 32x32x16: under sustained load the chip's
// clock is set by its power draw, and per FLOP the smaller block moves half
// the accumulator data through the register file.  Measured on the recompute
// shape, the same MFMA-busy cycles ran at 1.87 against 1.67 GHz, 2-3% faster
// overall, with identical results (each block is a sum over e in the same
// order).
//
// Workgroups that share a y tile are placed consecutively on one XCD so the
// tile is read from HBM once and served from that XCD's L2; W (both
// projections, 64 MB) stays in the MALL.
#include "bwa.h"
#include "common.h"

namespace bwa {

namespace {

struct GemmParams {
  const bf16* y;     // [B*S, E]
  const bf16* w[2];  // [HD, E] for K and V
  bf16* out[2];
  int64_t so[2][3];  // output strides (B, H, S) in elements
  int S, E, HD, H, D, BS;
  int n_tiles, s_tiles;
};

__device__ inline uint32_t pk(float a, float b) {
  bf16 x = (bf16)a, y = (bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

}  // namespace

// Tiling: GM x GN per workgroup of WM x WN waves, GK per LDS stage.
template <int GM_, int GN_, int GK_, int WM_, int WN_>
struct GemmTile {
  static constexpr int GM = GM_, GN = GN_, GK = GK_, WM = WM_, WN = WN_;
  static constexpr int NW = WM * WN, NT = 64 * NW;
  static constexpr int WTM = GM / WM, WTN = GN / WN;  // per-wave tile (n x s)
  static constexpr int FA = WTM / 16, FB = WTN / 16;  // 16x16 MFMA blocks per wave
  static constexpr int GS = GK + 16;                  // LDS row stride (elements)
  static constexpr int A_EL = GM * GS, B_EL = GN * GS;
  static constexpr int CPR = GK / 8;                  // 16-byte chunks per row
  static constexpr int KC = (GM + GN) * CPR / NT;     // chunks per thread per stage
  static_assert(KC * NT == (GM + GN) * CPR, "staging must divide evenly");
  static_assert((GM * CPR) % NT == 0, "A chunks must fill whole passes");
};

template <typename T>
__global__ __launch_bounds__(T::NT) void gemm_kv_kernel(GemmParams p) {
  constexpr int GM = T::GM, GN = T::GN, GK = T::GK, GS = T::GS, CPR = T::CPR, KC = T::KC;
  constexpr int KA = GM * CPR / T::NT;  // passes of A chunks
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * (T::A_EL + T::B_EL)];

  int grp, nt;
  if (!xcd_group_tile(blockIdx.x, p.n_tiles, 2 * p.s_tiles, &grp, &nt)) return;
  const int proj = grp / p.s_tiles;
  const int st = grp % p.s_tiles;
  const int n0 = nt * GM, s0 = st * GN;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave / T::WN, wn = wave % T::WN;
  const bf16* wsrc = p.w[proj];

  // thread's chunks: passes i < KA are W rows, the rest y rows; 8-lane groups
  // cover one row's GK elements (128 contiguous bytes for GK = 64).  Rows past
  // the end repeat the last row.  Byte offsets from the operand's base fit in
  // 32 bits (rows x E x 2 < 2^31, checked on the host).
  uint32_t goff[KC];
  int sdst[KC];  // LDS element offsets
  const bf16* ysrc = p.y;
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    const int c = tid + T::NT * i;
    if (i < KA) {
      const int row = c / CPR, col8 = c % CPR;
      const int n = min(n0 + row, p.HD - 1);
      goff[i] = ((uint32_t)n * (uint32_t)p.E + (uint32_t)(col8 * 8)) * 2u;
      sdst[i] = row * GS + col8 * 8;
    } else {
      const int cb = c - GM * CPR;
      const int row = cb / CPR, col8 = cb % CPR;
      const int sr = min(s0 + row, p.BS - 1);
      goff[i] = ((uint32_t)sr * (uint32_t)p.E + (uint32_t)(col8 * 8)) * 2u;
      sdst[i] = T::A_EL + row * GS + col8 * 8;
    }
  }
  u32x4 stg[KC];
  auto load1 = [&](int i, int e0) __attribute__((always_inline)) {
    const char* base = (const char*)((i < KA ? wsrc : ysrc) + e0);
    stg[i] = *(const u32x4*)(base + goff[i]);
  };
  auto store1 = [&](int i, int buf) __attribute__((always_inline)) {
    *(u32x4*)(smem + sdst[i] + buf * (T::A_EL + T::B_EL)) = stg[i];
  };

  f32x4 acc[T::FA][T::FB];
#pragma unroll
  for (int a = 0; a < T::FA; ++a)
#pragma unroll
    for (int b = 0; b < T::FB; ++b) acc[a][b] = f32x4{};

  // operand reads: A rows (n) of this wave's block a, B rows (s) of block b,
  // 32 contraction elements at step ks (lane: row lane%16, elements 8*(lane/16) on)
  const int l16 = lane & 15, q4 = lane >> 4;
  const bf16* aread = smem + (wm * T::WTM + l16) * GS + 8 * q4;
  const bf16* bread = smem + T::A_EL + (wn * T::WTN + l16) * GS + 8 * q4;
  constexpr int KSN = GK / 32, NM = KSN * T::FA * T::FB;
  auto rd = [&](int buf, int ks, int o) __attribute__((always_inline)) {
    const int bo = buf * (T::A_EL + T::B_EL) + 32 * ks;
    return o < T::FA ? *(const bf16x8*)(aread + bo + 16 * o * GS)
                     : *(const bf16x8*)(bread + bo + 16 * (o - T::FA) * GS);
  };

  // One stage: the MFMAs of buffer buf in a fixed issue order, block rows
  // a-major over its KSN k-steps; a row's A block is read AD rows ahead, the
  // next k-step's B blocks while row XR of the current one runs.  (WR) The
  // staged chunks of the next stage are written into buf^1 over the first
  // KSN-1 k-steps and (LD) the loads of the stage after it issued one after
  // each write.  (NEXT) The workgroup barrier sits before row XR of the last
  // k-step: by then every wave has written the next stage and issued its last
  // read of this one (the A blocks of the rows after it are AD rows ahead),
  // so after it the next stage's first operands are read from buf^1 while
  // the last AD rows' MFMAs run on registers, and no wave writes buf (in the
  // next stage) while another still reads it.
  constexpr int NW_ = (KSN - 1) * T::FA * T::FB;  // MFMAs carrying the writes
  static_assert(NW_ % KC == 0, "staging chunks spread evenly over the first k-steps");
  constexpr int AD = 3, NAB = 4, XR = T::FA - AD;
  static_assert(AD < NAB && (KSN * T::FA) % NAB == 0 && XR >= AD,
                "A registers rotate evenly over stages; rows after the barrier read before it");
  constexpr int NX = NM - AD * T::FB;  // the barrier's place in a NEXT stage
  static_assert(NX >= NW_, "the next stage's chunks are written before the barrier");
  // operands: the A blocks of rows r .. r+AD (rows counted over the stage),
  // all B blocks of the current k-step and of the next
  bf16x8 abuf[NAB], bbuf[2][T::FB];
  auto stage = [&](auto wr_, auto ld_, auto next_, int buf, int e_next) __attribute__((always_inline)) {
    constexpr bool WR = decltype(wr_)::value, LD = decltype(ld_)::value;
    constexpr bool NEXT = decltype(next_)::value;
    static_for<0, NM>([&](auto mi) __attribute__((always_inline)) {
      constexpr int m = decltype(mi)::value;
      constexpr int ks = m / (T::FA * T::FB), idx = m % (T::FA * T::FB);
      constexpr int a = idx / T::FB, b = idx % T::FB, r = ks * T::FA + a;
      if constexpr (NEXT && m == NX) __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abuf[r % NAB], bbuf[ks & 1][b], acc[a][b], 0, 0, 0);
      if constexpr (b == 0) {  // the A block AD rows on
        constexpr int r2 = r + AD;
        if constexpr (r2 < KSN * T::FA) abuf[r2 % NAB] = rd(buf, r2 / T::FA, r2 % T::FA);
        else if constexpr (NEXT) abuf[r2 % NAB] = rd(buf ^ 1, 0, r2 - KSN * T::FA);
      }
      if constexpr (a == XR) {  // the next k-step's B block b
        if constexpr (ks + 1 < KSN) bbuf[(ks + 1) & 1][b] = rd(buf, ks + 1, T::FA + b);
        else if constexpr (NEXT) bbuf[0][b] = rd(buf ^ 1, 0, T::FA + b);
      }
      if constexpr (WR && m < NW_ && m % (NW_ / KC) == 0) store1(m / (NW_ / KC), buf ^ 1);
      if constexpr (LD && m < NW_ && m % (NW_ / KC) == 1) load1(m / (NW_ / KC), e_next);
    });
    __builtin_amdgcn_sched_barrier(0);
  };

  const int nk = p.E / GK;
  using T_ = std::true_type;
  using F_ = std::false_type;
  // prologue: stage 0 in buffer 0, stage 1 in flight
#pragma unroll
  for (int i = 0; i < KC; ++i) load1(i, 0);
#pragma unroll
  for (int i = 0; i < KC; ++i) store1(i, 0);
  if (nk > 1) {
#pragma unroll
    for (int i = 0; i < KC; ++i) load1(i, GK);
  }
  __syncthreads();
#pragma unroll
  for (int o = 0; o < AD; ++o) abuf[o] = rd(0, 0, o);
#pragma unroll
  for (int o = 0; o < T::FB; ++o) bbuf[0][o] = rd(0, 0, T::FA + o);
  int kt = 0;
  for (; kt + 2 < nk; ++kt) stage(T_{}, T_{}, T_{}, kt & 1, (kt + 2) * GK);
  if (kt + 1 < nk) {
    stage(T_{}, F_{}, T_{}, kt & 1, 0);
    ++kt;
  }
  stage(F_{}, F_{}, F_{}, kt & 1, 0);

  bf16* out = p.out[proj];
#pragma unroll
  for (int b = 0; b < T::FB; ++b) {
    const int s = s0 + wn * T::WTN + 16 * b + l16;
    if (s >= p.BS) continue;
    const int bb = s / p.S, si = s % p.S;
#pragma unroll
    for (int a = 0; a < T::FA; ++a) {
      const int n = n0 + wm * T::WTM + 16 * a + 4 * q4;
      if (n >= p.HD) continue;
      const int hh = n / p.D, d = n % p.D;
      bf16* dst = out + bb * p.so[proj][0] + hh * p.so[proj][1] + (int64_t)si * p.so[proj][2] + d;
      *(u32x2*)dst = u32x2{pk(acc[a][b][0], acc[a][b][1]), pk(acc[a][b][2], acc[a][b][3])};
    }
  }
}

using KvTile = GemmTile<256, 256, 64, 2, 4>;

template <typename T>
static void launch_gemm(GemmParams p, hipStream_t st) {
  p.n_tiles = (p.HD + T::GM - 1) / T::GM;
  p.s_tiles = (p.BS + T::GN - 1) / T::GN;
  const int blocks = xcd_grid_size(p.n_tiles, 2 * p.s_tiles);
  hipLaunchKernelGGL(gemm_kv_kernel<T>, dim3(blocks), dim3(T::NT), 0, st, p);
}

hipError_t gemm_kv_launch(const void* y, const void* wk_t, const void* wv_t, int64_t B, int64_t S,
                          int64_t E, int64_t H, int64_t Dh, const bwa_tensor* k,
                          const bwa_tensor* v, hipStream_t st) {
  GemmParams p = {};
  p.y = (const bf16*)y;
  p.w[0] = (const bf16*)wk_t;
  p.w[1] = (const bf16*)wv_t;
  p.out[0] = (bf16*)k->ptr;
  p.out[1] = (bf16*)v->ptr;
  p.so[0][0] = k->sB; p.so[0][1] = k->sH; p.so[0][2] = k->sS;
  p.so[1][0] = v->sB; p.so[1][1] = v->sH; p.so[1][2] = v->sS;
  p.S = (int)S;
  p.E = (int)E;
  p.H = (int)H;
  p.D = (int)Dh;
  p.HD = (int)(H * Dh);
  p.BS = (int)(B * S);
  launch_gemm<KvTile>(p, st);
  return hipGetLastError();
}

}  // namespace bwa
