// K/V recompute from the one shared copy of the visual features (LV-XAttn
// review, "What carries the argument": all cross-attention layers read the
// same y, so y is kept once and K = y W_k, V = y W_v are recomputed when
// needed).
//
//   out[b, h, s, d] = sum_e y[b, s, e] * W[e, h*D + d],  W stored transposed
//   as w_t[n, e] (n = h*D + d), the [out, in] layout of a linear layer.
//
// The kernel computes the transposed product C^T[n, s] = w_t[n, :] . y[s, :]
// on v_mfma_f32_32x32x16_bf16, so that each lane of a 32x32 output block owns
// four consecutive n (= four consecutive head dims d) of one key row s and
// stores them as one 8-byte write into the [B, H, S, D] output.  Both
// operands keep the contraction index e contiguous in memory and in LDS.
//
// Tiling: 256 (n) x 128 (s) per workgroup of 4 waves (2 x 2), 128 x 64 per
// wave (4 x 2 MFMA blocks, fp32 accumulators), BK = 32 per LDS stage, double
// buffered.  Workgroups that share a y tile are placed consecutively on one
// XCD so the tile is read from HBM once and served from that XCD's L2.
#include "bwa.h"
#include "common.h"

namespace bwa {

namespace {

constexpr int GM = 256;  // n per workgroup
constexpr int GN = 128;  // s per workgroup
constexpr int GK = 32;   // e per stage
constexpr int GS = GK + 8;  // LDS row stride (elements), 16 B pad

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

__global__ __launch_bounds__(256) void gemm_kv_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) bf16 As[2][GM * GS];
  __shared__ __attribute__((aligned(16))) bf16 Bs[2][GN * GS];

  // groups = (projection, s tile); tiles = n tiles sharing that y tile
  int grp, nt;
  if (!xcd_group_tile(blockIdx.x, p.n_tiles, 2 * p.s_tiles, &grp, &nt)) return;
  const int proj = grp / p.s_tiles;
  const int st = grp % p.s_tiles;
  const int n0 = nt * GM, s0 = st * GN;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 31, g = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const bf16* wsrc = p.w[proj];

  u32x4 stg[6];
  auto load = [&](int e0) {
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      int c = tid + 256 * i;     // 1536 chunks: 1024 from W (256 rows), then 512 from y (128 rows)
      int row = c < 1024 ? (c >> 2) : ((c - 1024) >> 2), col8 = c & 3;
      if (c < 1024) {
        int n = n0 + row;
        stg[i] = n < p.HD ? *(const u32x4*)(wsrc + (int64_t)n * p.E + e0 + col8 * 8) : u32x4{};
      } else {
        int s = s0 + row;
        stg[i] = s < p.BS ? *(const u32x4*)(p.y + (int64_t)s * p.E + e0 + col8 * 8) : u32x4{};
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      int c = tid + 256 * i;
      int row = c < 1024 ? (c >> 2) : ((c - 1024) >> 2), col8 = c & 3;
      bf16* dst = (c < 1024 ? As[buf] : Bs[buf]) + row * GS + col8 * 8;
      *(u32x4*)dst = stg[i];
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};

  const int nk = p.E / GK;
  load(0);
  store(0);
  __syncthreads();
  int buf = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) load((kt + 1) * GK);
#pragma unroll
    for (int ks = 0; ks < GK / 16; ++ks) {
      bf16x8 av[4], bv[2];
#pragma unroll
      for (int a = 0; a < 4; ++a)
        av[a] = *(const bf16x8*)(As[buf] + (wm * 128 + 32 * a + lr) * GS + 16 * ks + 8 * g);
#pragma unroll
      for (int b = 0; b < 2; ++b)
        bv[b] = *(const bf16x8*)(Bs[buf] + (wn * 64 + 32 * b + lr) * GS + 16 * ks + 8 * g);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
    if (!more) break;
    store(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // C^T block (a, b): lane column s = s0 + wn*64 + 32b + lr,
  // rows n = n0 + wm*128 + 32a + 8i + 4g + j  (j = 0..3 consecutive head dims)
  bf16* out = p.out[proj];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int s = s0 + wn * 64 + 32 * b + lr;
    if (s >= p.BS) continue;
    const int bb = s / p.S, si = s % p.S;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n0 + wm * 128 + 32 * a + 8 * i + 4 * g;
        if (n >= p.HD) continue;
        const int hh = n / p.D, d = n % p.D;
        bf16* dst = out + bb * p.so[proj][0] + hh * p.so[proj][1] + (int64_t)si * p.so[proj][2] + d;
        *(u32x2*)dst = u32x2{pk(acc[a][b][4 * i], acc[a][b][4 * i + 1]),
                             pk(acc[a][b][4 * i + 2], acc[a][b][4 * i + 3])};
      }
  }
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
  p.n_tiles = (p.HD + GM - 1) / GM;
  p.s_tiles = (p.BS + GN - 1) / GN;
  int blocks = xcd_grid_size(p.n_tiles, 2 * p.s_tiles);
  hipLaunchKernelGGL(gemm_kv_kernel, dim3(blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace bwa
