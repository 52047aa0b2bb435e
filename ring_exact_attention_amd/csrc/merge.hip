// fp32 rescale-merge kernels (LV-XAttn review, "What carries the argument":
// partial outputs and their softmax statistics are combined by FlashAttention
// rescaling; "Assumptions": that rescaling is exact).
//
// For two partials (O_a, L_a), (O_b, L_b) of one row over disjoint key sets:
//   M = max(L_a, L_b),  L = M + ln(e^(L_a-M) + e^(L_b-M)),
//   O = e^(L_a-L) O_a + e^(L_b-L) O_b,  with (0, -inf) the identity.
// These kernels are HBM-bound: one thread moves 16 bytes of O per partial.
#include "common.h"

namespace bwa {

struct MergeWeights {
  float wa, wb, L;
};

__device__ inline MergeWeights merge_weights(float la, float lb) {
  MergeWeights w;
  float M = fmaxf(la, lb);
  if (M == -INFINITY) {
    w.wa = 0.f;
    w.wb = 0.f;
    w.L = -INFINITY;
    return w;
  }
  float ea = __expf(la - M), eb = __expf(lb - M);
  w.L = M + __logf(ea + eb);
  w.wa = __expf(la - w.L);
  w.wb = __expf(lb - w.L);
  return w;
}

// Two-way merge, rows x D fp32.  One thread per 4 columns of a row.
__global__ __launch_bounds__(256) void merge2_kernel(int64_t rows, int D, const float* oa,
                                                     const float* la, const float* ob,
                                                     const float* lb, float* oo, float* lo) {
  const int per_row = D / 4;
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * per_row) return;
  int64_t r = idx / per_row;
  int c = (int)(idx % per_row) * 4;
  float a = la[r], bb = lb[r];
  MergeWeights w = merge_weights(a, bb);
  f32x4 xa = *(const f32x4*)(oa + r * D + c);
  f32x4 xb = *(const f32x4*)(ob + r * D + c);
  f32x4 y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = w.wa * xa[e] + w.wb * xb[e];
  // every thread of the row has read its inputs before any writes (outputs may alias)
  *(f32x4*)(oo + r * D + c) = y;
  if (c == 0) lo[r] = w.L;
}

// Merge the n per-shard partials of every row in its query block's schedule
// order and write the final output (q's dtype) and LSE.
template <typename T>
__global__ __launch_bounds__(256) void split_merge_kernel(FwdParams p) {
  const int D = p.D;
  const int per_row = D / 4;
  const int64_t BH = (int64_t)p.B * p.H;
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= BH * p.SQ * per_row) return;
  int64_t row = idx / per_row;  // bh * SQ + i
  int c = (int)(idx % per_row) * 4;
  int64_t bh = row / p.SQ, i = row % p.SQ;
  int j = (int)(((i + 1) * p.n - 1) / p.SQ);  // query block holding row i
  const int64_t slot = BH * p.SQ;
  f32x4 o = f32x4{};
  float L = -INFINITY;
  for (int r = 0; r < p.n; ++r) {
    int s = shard_at_step(p.sched, p.n, j, r);
    float ls = p.lse_part[s * slot + row];
    MergeWeights w = merge_weights(L, ls);
    if (w.L == -INFINITY) continue;
    f32x4 x = *(const f32x4*)(p.o_acc + (s * slot + row) * D + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = w.wa * o[e] + w.wb * x[e];
    L = w.L;
  }
  int64_t b = bh / p.H, h = bh % p.H;
  T* dst = (T*)p.o + b * p.soB + h * p.soH + i * p.soS + c;
  if constexpr (sizeof(T) == 4) {
    *(f32x4*)dst = o;
  } else {
    bf16 v0 = (bf16)o[0], v1 = (bf16)o[1], v2 = (bf16)o[2], v3 = (bf16)o[3];
    uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, v0) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
    uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, v2) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, v3) << 16);
    *(u32x2*)dst = u32x2{w0, w1};
  }
  if (c == 0) p.lse[row] = L;
}

// Running fp32 O -> output tensor in q's dtype (ROUNDS mode, after the last round).
template <typename T>
__global__ __launch_bounds__(256) void finalize_kernel(FwdParams p) {
  const int D = p.D;
  const int per_row = D / 4;
  const int64_t BH = (int64_t)p.B * p.H;
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= BH * p.SQ * per_row) return;
  int64_t row = idx / per_row;
  int c = (int)(idx % per_row) * 4;
  int64_t bh = row / p.SQ, i = row % p.SQ;
  f32x4 o = *(const f32x4*)(p.o_acc + row * D + c);
  int64_t b = bh / p.H, h = bh % p.H;
  T* dst = (T*)p.o + b * p.soB + h * p.soH + i * p.soS + c;
  if constexpr (sizeof(T) == 4) {
    *(f32x4*)dst = o;
  } else {
    bf16 v0 = (bf16)o[0], v1 = (bf16)o[1], v2 = (bf16)o[2], v3 = (bf16)o[3];
    uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, v0) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
    uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, v2) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, v3) << 16);
    *(u32x2*)dst = u32x2{w0, w1};
  }
}

static inline int blocks_for(int64_t threads) { return (int)((threads + 255) / 256); }

hipError_t merge2_launch(int64_t rows, int D, const float* oa, const float* la, const float* ob,
                         const float* lb, float* oo, float* lo, hipStream_t st) {
  int64_t n = rows * (D / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(merge2_kernel, dim3(blocks_for(n)), dim3(256), 0, st, rows, D, oa, la, ob,
                     lb, oo, lo);
  return hipGetLastError();
}

hipError_t split_merge_launch(FwdParams p, int dtype_bf16, hipStream_t st) {
  int64_t n = (int64_t)p.B * p.H * p.SQ * (p.D / 4);
  if (n == 0) return hipSuccess;
  if (dtype_bf16)
    hipLaunchKernelGGL(split_merge_kernel<bf16>, dim3(blocks_for(n)), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(split_merge_kernel<float>, dim3(blocks_for(n)), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t finalize_launch(FwdParams p, int dtype_bf16, hipStream_t st) {
  int64_t n = (int64_t)p.B * p.H * p.SQ * (p.D / 4);
  if (n == 0) return hipSuccess;
  if (dtype_bf16)
    hipLaunchKernelGGL(finalize_kernel<bf16>, dim3(blocks_for(n)), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(finalize_kernel<float>, dim3(blocks_for(n)), dim3(256), 0, st, p);
  return hipGetLastError();
}

// Copy a [B, H, S] array of rows (row_bytes each, a multiple of 16) from
// element-strided storage (strides in bytes) into contiguous storage.
__global__ __launch_bounds__(256) void copy_rows_kernel(const char* src, int64_t sB, int64_t sH,
                                                        int64_t sS, char* dst, int B, int H,
                                                        int64_t S, int row_bytes) {
  const int per_row = row_bytes / 16;
  const int64_t total = (int64_t)B * H * S * per_row;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = idx / per_row;
    const int c = (int)(idx % per_row);
    const int64_t i = row % S, bh = row / S, b = bh / H, h = bh % H;
    *(u32x4*)(dst + row * row_bytes + 16 * c) =
        *(const u32x4*)(src + b * sB + h * sH + i * sS + 16 * c);
  }
}

hipError_t copy_rows_launch(const void* src, int64_t sB, int64_t sH, int64_t sS, void* dst, int B,
                            int H, int64_t S, int row_bytes, hipStream_t st) {
  const int64_t total = (int64_t)B * H * S * (row_bytes / 16);
  if (total == 0) return hipSuccess;
  const int64_t want = (total + 255) / 256;
  const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(copy_rows_kernel, dim3(blocks), dim3(256), 0, st, (const char*)src, sB, sH,
                     sS, (char*)dst, B, H, S, row_bytes);
  return hipGetLastError();
}

}  // namespace bwa
