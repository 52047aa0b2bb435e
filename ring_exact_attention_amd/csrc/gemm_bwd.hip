// Gradients through the K/V recompute (LV-XAttn review, "What carries the
// argument": y is kept once and K = y W_k, V = y W_v are recomputed, so the
// backward also produces the gradients of W_k, W_v and y):
//   dW_k^T[n, e] = sum_{b,s} dK[b, h, s, d] * y[b, s, e]        (n = h*D + d)
//   dy[b, s, e]  = sum_n dK[b, h, s, d] * W_k^T[n, e] + (same with dV, W_v)
// with W_k^T the [H*D, E] weight layout of bwa_kv_recompute.
//
// Both are 256 x 256-tiled MFMA GEMMs on 8 waves (2 x 4, 128 x 64 per wave),
// 64 contraction rows per LDS stage, double buffered, with the MFMAs of a
// stage in a fixed order beside the operand reads of the next k-step, the
// LDS writes of the next stage and the global loads of the one after; the
// stage's barrier precedes its last k-step (see mma_stage).  An operand whose
// contraction index is its storage row (dK and y in the weight gradient, W^T
// in dy) is staged row-major as [k][m] and read with ds_read_b64_tr_b16: each
// lane takes rows k0..k0+3 and k0+4..k0+7 of its column, the same k order as
// a 16-byte read of an operand stored with k contiguous ([m][k], dK in dy).
#include "bwa.h"
#include "common.h"

namespace bwa {

namespace {

constexpr int TM = 256, TN = 256, TK = 64;  // workgroup tile
constexpr int NT = 512;                     // 8 waves: 2 (m) x 4 (n)
constexpr int WTM = 128, WTN = 64;          // per wave
constexpr int FA = WTM / 32, FB = WTN / 32; // 32x32 blocks per wave
// Row stride of a [k][m] tile (elements): a transposing read serves 32 lanes
// as 4 rows x 64 bytes from 64 banks of 4 bytes; rows 2*(TM+32) bytes apart
// (64 mod 256) fall in distinct quarters of the bank space, conflict-free.
constexpr int TSK = TM + 32;
constexpr int NSK = TK + 8;                 // row stride of a [m][k] tile (elements)
constexpr int T_EL = TK * TSK;              // [k][m] tile elements (TM == TN)
constexpr int N_EL = TM * NSK;              // [m][k] tile elements

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

struct GradParams {
  const bf16* y;                 // [B*S, E]
  const bf16* wt[2];             // W_k^T, W_v^T: [HD, E]
  const bf16* g[2];              // dK, dV: [B, H, S, D] by strides
  int64_t gs[2][3];              // their strides (B, H, S), elements
  float* dwt[2];                 // [HD, E] fp32, or NULL
  float* dy;                     // [B*S, E] fp32, or NULL
  int B, S, E, H, D, HD, accumulate;
  int m_tiles, n_tiles;
};

// A [k][m] operand fragment (rows k0..k0+7 of column m0 + lane%32).
__device__ inline bf16x8 read_t(const bf16* t, int k0, int m0, int lane) {
  const int li = lane & 15;
  const bf16* a = t + (k0 + (li >> 2)) * TSK + m0 + ((lane >> 4) & 1) * 16 + 4 * (li & 3);
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a);
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 4 * TSK));
  u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
}

// Operand o of k-step ks: o < FA is A block o (rows m of this wave), the
// rest B block o - FA (columns n).  A is [k][m] (AT) or [m][k]; B is [k][n].
template <bool AT>
__device__ inline bf16x8 read_op(const bf16* As, const bf16* Bs, int ks, int o, int wm, int wn,
                                 int lane) {
  const int lr = lane & 31, g = lane >> 5;
  if (o < FA)
    return AT ? read_t(As, 16 * ks + 8 * g, wm * WTM + 32 * o, lane)
              : *(const bf16x8*)(As + (wm * WTM + 32 * o + lr) * NSK + 16 * ks + 8 * g);
  return read_t(Bs, 16 * ks + 8 * g, wn * WTN + 32 * (o - FA), lane);
}

// One stage of MFMAs from (As, Bs) in a fixed issue order, each k-step's
// operands read during the previous one (op[0] holds the first k-step's on
// entry).  Chunk hooks run beside the MFMAs of the first KSN-1 k-steps, one of
// each every NW/NCH MFMAs: write(i) (the next stage's staged chunk i into the
// other buffer), then load(i) (chunk i of the stage after it, into the
// registers just written out), so neither LDS writes nor global loads come in
// bursts and every load has a whole stage to land.  With NEXT the
// workgroup's barrier sits before the last k-step (every wave has written
// the next stage and read this one by then) and the next stage's first
// operands are read from (Asn, Bsn) while the last k-step's MFMAs run on
// registers.
constexpr int NCH = 8;  // 16-byte staging chunks per thread and stage
constexpr int NOP = FA + FB;
template <bool AT, bool WR, bool LD, bool NEXT, typename W, typename L>
__device__ inline __attribute__((always_inline)) void mma_stage(
    const bf16* As, const bf16* Bs, const bf16* Asn, const bf16* Bsn, int wm, int wn, int lane,
    f32x16 (&acc)[FA][FB], bf16x8 (&op)[2][NOP], W&& write, L&& load) {
  constexpr int KSN = TK / 16, NM = KSN * FA * FB, NW = (KSN - 1) * FA * FB;
  static_assert(NW % NCH == 0, "staging chunks spread evenly over the first k-steps");
  static_for<0, NM>([&](auto mi) __attribute__((always_inline)) {
    constexpr int m = decltype(mi)::value;
    constexpr int ks = m / (FA * FB), idx = m % (FA * FB);
    constexpr int a = idx / FB, b = idx % FB;
    if constexpr (NEXT && m == NW) __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[ks & 1][a], op[ks & 1][FA + b],
                                                        acc[a][b], 0, 0, 0);
    if constexpr (ks + 1 < KSN && idx < NOP)
      op[(ks + 1) & 1][idx] = read_op<AT>(As, Bs, ks + 1, idx, wm, wn, lane);
    if constexpr (NEXT && ks + 1 == KSN && idx < NOP)
      op[0][idx] = read_op<AT>(Asn, Bsn, 0, idx, wm, wn, lane);
    if constexpr (WR && m < NW && m % (NW / NCH) == 0) write(m / (NW / NCH));
    if constexpr (LD && m < NW && m % (NW / NCH) == 1) load(m / (NW / NCH));
  });
  __builtin_amdgcn_sched_barrier(0);
}

// Write a 256 x 256 fp32 tile: C rows m (out row m0 + m), columns n (n0 + n);
// lane column n = wn*64 + 32b + lane%32, rows wm*128 + 32a + 8i + 4g + j.
__device__ inline void store_tile(float* out, int64_t ld, int64_t m0, int64_t m_end, int n0,
                                  int wm, int wn, int lane, bool accumulate,
                                  const f32x16 (&acc)[FA][FB]) {
  const int lr = lane & 31, g = lane >> 5;
#pragma unroll
  for (int a = 0; a < FA; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t m = m0 + wm * WTM + 32 * a + 8 * i + 4 * g + j;
        if (m >= m_end) continue;
#pragma unroll
        for (int b = 0; b < FB; ++b) {
          float* dst = out + m * ld + n0 + wn * WTN + 32 * b + lr;
          const float v = acc[a][b][4 * i + j];
          *dst = accumulate ? *dst + v : v;
        }
      }
}

}  // namespace

// dW^T[n, e] for both projections: M = HD (n), N = E (e), K = B*S rows.
// Workgroups that share an n tile (and so the dK/dV slab they stream) are
// consecutive on one XCD.
__global__ __launch_bounds__(NT) void gemm_dw_kernel(GradParams p) {
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * 2 * T_EL];
  int grp, et;
  if (!xcd_group_tile(blockIdx.x, p.n_tiles, 2 * p.m_tiles, &grp, &et)) return;
  const int proj = grp / p.m_tiles, nt = grp % p.m_tiles;
  if (!p.dwt[proj]) return;
  const int n0 = nt * TM, e0 = et * TN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave / 4, wn = wave % 4;

  // staging: 64 rows x 32 chunks per operand; thread covers rows r0 + 16 i,
  // chunk column c (8 elements) of both the dK/dV tile and the y tile
  const int c = tid % 32, r0 = tid / 32;
  const int n = n0 + 8 * c, hh = n / p.D, dd = n % p.D;
  const bf16* gsrc = p.g[proj] + hh * p.gs[proj][1] + dd;
  const int64_t gss = p.gs[proj][2];
  const bf16* ysrc = p.y + e0 + 8 * c;
  u32x4 st[NCH];  // chunks 0..3: dK/dV rows, 4..7: y rows
  const bf16* ga = nullptr;  // first row of the stage being loaded, per operand
  const bf16* yb = nullptr;
  auto aim = [&](int64_t k0) {  // k0: first flat row (b*S + s) of a stage
    const int64_t b = k0 / p.S, s0 = k0 % p.S;
    ga = gsrc + b * p.gs[proj][0] + s0 * gss;
    yb = ysrc + k0 * p.E;
  };
  auto load1 = [&](int i) __attribute__((always_inline)) {
    const int r = r0 + 16 * (i & 3);
    st[i] = i < 4 ? *(const u32x4*)(ga + r * gss) : *(const u32x4*)(yb + (int64_t)r * p.E);
  };
  auto store1 = [&](int i, int buf) __attribute__((always_inline)) {
    bf16* At = smem + buf * 2 * T_EL + (i < 4 ? 0 : T_EL);
    *(u32x4*)(At + (r0 + 16 * (i & 3)) * TSK + 8 * c) = st[i];
  };

  f32x16 acc[FA][FB];
#pragma unroll
  for (int a = 0; a < FA; ++a)
#pragma unroll
    for (int b = 0; b < FB; ++b) acc[a][b] = f32x16{};
  const int64_t nk = (int64_t)p.B * p.S / TK;
  // prologue: stage 0 in buffer 0, stage 1 in flight
  aim(0);
#pragma unroll
  for (int i = 0; i < NCH; ++i) load1(i);
#pragma unroll
  for (int i = 0; i < NCH; ++i) store1(i, 0);
  if (nk > 1) {
    aim(TK);
#pragma unroll
    for (int i = 0; i < NCH; ++i) load1(i);
  }
  __syncthreads();
  bf16x8 op[2][NOP];
#pragma unroll
  for (int o = 0; o < NOP; ++o) op[0][o] = read_op<true>(smem, smem + T_EL, 0, o, wm, wn, lane);
  int64_t kt = 0;
  for (; kt + 2 < nk; ++kt) {
    const int buf = (int)(kt & 1);
    const bf16 *As = smem + buf * 2 * T_EL, *An = smem + (buf ^ 1) * 2 * T_EL;
    aim((kt + 2) * TK);
    mma_stage<true, true, true, true>(As, As + T_EL, An, An + T_EL, wm, wn, lane, acc, op,
                                      [&](int i) { store1(i, buf ^ 1); }, load1);
  }
  if (kt + 1 < nk) {
    const int buf = (int)(kt & 1);
    const bf16 *As = smem + buf * 2 * T_EL, *An = smem + (buf ^ 1) * 2 * T_EL;
    mma_stage<true, true, false, true>(As, As + T_EL, An, An + T_EL, wm, wn, lane, acc, op,
                                       [&](int i) { store1(i, buf ^ 1); }, load1);
    ++kt;
  }
  {
    const bf16* As = smem + (int)(kt & 1) * 2 * T_EL;
    mma_stage<true, false, false, false>(As, As + T_EL, As, As + T_EL, wm, wn, lane, acc, op,
                                         load1, load1);
  }
  store_tile(p.dwt[proj], p.E, n0, p.HD, e0, wm, wn, lane, p.accumulate != 0, acc);
}

// dy[m, e] = sum over k = (projection, n) of g[proj][m, n] * W^T[proj][n, e]:
// M = B*S rows, N = E, K = 2*HD.  Workgroups that share an m tile (its dK/dV
// rows) are consecutive on one XCD.
__global__ __launch_bounds__(NT) void gemm_dy_kernel(GradParams p) {
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * (N_EL + T_EL)];
  int mt, et;
  if (!xcd_group_tile(blockIdx.x, p.n_tiles, p.m_tiles, &mt, &et)) return;
  const int64_t m0 = (int64_t)mt * TM, M = (int64_t)p.B * p.S;
  const int e0 = et * TN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave / 4, wn = wave % 4;

  // A staging ([m][k], k = n contiguous): thread covers rows ra + 64 i, chunk ca
  const int ca = tid % 8, ra = tid / 8;
  // element offset of row (b, s) in dK and dV (which share strides); rows
  // past the end repeat the last one (loaded, never stored)
  int64_t arow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = min(m0 + ra + 64 * i, M - 1);
    arow[i] = m / p.S * p.gs[0][0] + m % p.S * p.gs[0][2];
  }
  // B staging ([k][e], W^T rows): thread covers rows rb + 16 i, chunk cb
  const int cb = tid % 32, rb = tid / 32;
  u32x4 st[NCH];  // chunks 0..3: dK/dV rows ([m][k]), 4..7: W^T rows ([k][e])
  const bf16* gb = nullptr;  // stage bases of the operands being loaded
  const bf16* wb = nullptr;
  auto aim = [&](int kt) {  // kt: stage index over K = 2*HD
    const int kk = kt * TK, proj = kk / p.HD, n = kk % p.HD;
    const int hh = n / p.D, dd = n % p.D;
    gb = p.g[proj] + hh * p.gs[proj][1] + dd + ca * 8;
    wb = p.wt[proj] + (int64_t)n * p.E + e0 + 8 * cb;
  };
  auto load1 = [&](int i) __attribute__((always_inline)) {
    st[i] = i < 4 ? *(const u32x4*)(gb + arow[i & 3])
                  : *(const u32x4*)(wb + (int64_t)(rb + 16 * (i & 3)) * p.E);
  };
  auto store1 = [&](int i, int buf) __attribute__((always_inline)) {
    bf16* As = smem + buf * (N_EL + T_EL);
    if (i < 4) *(u32x4*)(As + (ra + 64 * i) * NSK + ca * 8) = st[i];
    else *(u32x4*)(As + N_EL + (rb + 16 * (i & 3)) * TSK + 8 * cb) = st[i];
  };

  f32x16 acc[FA][FB];
#pragma unroll
  for (int a = 0; a < FA; ++a)
#pragma unroll
    for (int b = 0; b < FB; ++b) acc[a][b] = f32x16{};
  const int nk = 2 * p.HD / TK;
  aim(0);
#pragma unroll
  for (int i = 0; i < NCH; ++i) load1(i);
#pragma unroll
  for (int i = 0; i < NCH; ++i) store1(i, 0);
  if (nk > 1) {
    aim(1);
#pragma unroll
    for (int i = 0; i < NCH; ++i) load1(i);
  }
  __syncthreads();
  bf16x8 op[2][NOP];
#pragma unroll
  for (int o = 0; o < NOP; ++o) op[0][o] = read_op<false>(smem, smem + N_EL, 0, o, wm, wn, lane);
  int kt = 0;
  for (; kt + 2 < nk; ++kt) {
    const int buf = kt & 1;
    const bf16 *As = smem + buf * (N_EL + T_EL), *An = smem + (buf ^ 1) * (N_EL + T_EL);
    aim(kt + 2);
    mma_stage<false, true, true, true>(As, As + N_EL, An, An + N_EL, wm, wn, lane, acc, op,
                                       [&](int i) { store1(i, buf ^ 1); }, load1);
  }
  if (kt + 1 < nk) {
    const int buf = kt & 1;
    const bf16 *As = smem + buf * (N_EL + T_EL), *An = smem + (buf ^ 1) * (N_EL + T_EL);
    mma_stage<false, true, false, true>(As, As + N_EL, An, An + N_EL, wm, wn, lane, acc, op,
                                        [&](int i) { store1(i, buf ^ 1); }, load1);
    ++kt;
  }
  {
    const bf16* As = smem + (kt & 1) * (N_EL + T_EL);
    mma_stage<false, false, false, false>(As, As + N_EL, As, As + N_EL, wm, wn, lane, acc, op,
                                          load1, load1);
  }
  store_tile(p.dy, p.E, m0, M, e0, wm, wn, lane, p.accumulate != 0, acc);
}

hipError_t gemm_grad_launch(const void* y, const void* wk_t, const void* wv_t,
                            const bwa_tensor* dk, const bwa_tensor* dv, int64_t B, int64_t S,
                            int64_t E, int64_t H, int64_t Dh, float* dwk_t, float* dwv_t,
                            float* dy, int accumulate, hipStream_t st) {
  GradParams p = {};
  p.y = (const bf16*)y;
  p.wt[0] = (const bf16*)wk_t;
  p.wt[1] = (const bf16*)wv_t;
  p.g[0] = (const bf16*)dk->ptr;
  p.g[1] = (const bf16*)dv->ptr;
  p.gs[0][0] = dk->sB; p.gs[0][1] = dk->sH; p.gs[0][2] = dk->sS;
  p.gs[1][0] = dv->sB; p.gs[1][1] = dv->sH; p.gs[1][2] = dv->sS;
  p.dwt[0] = dwk_t;
  p.dwt[1] = dwv_t;
  p.dy = dy;
  p.B = (int)B;
  p.S = (int)S;
  p.E = (int)E;
  p.H = (int)H;
  p.D = (int)Dh;
  p.HD = (int)(H * Dh);
  p.accumulate = accumulate;
  if (dwk_t || dwv_t) {
    p.m_tiles = p.HD / TM;
    p.n_tiles = p.E / TN;
    hipLaunchKernelGGL(gemm_dw_kernel, dim3(xcd_grid_size(p.n_tiles, 2 * p.m_tiles)), dim3(NT),
                       0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dy) {
    p.m_tiles = (int)((B * S + TM - 1) / TM);
    p.n_tiles = p.E / TN;
    hipLaunchKernelGGL(gemm_dy_kernel, dim3(xcd_grid_size(p.n_tiles, p.m_tiles)), dim3(NT), 0,
                       st, p);
  }
  return hipGetLastError();
}

}  // namespace bwa
