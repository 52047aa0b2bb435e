// Internal definitions shared by the HIP kernels and the host-side API.
// Target: gfx950 (CDNA4) only, wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace bwa {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, 32 CUs each

enum Mode { MODE_ROUNDS = 0, MODE_FUSED = 1, MODE_SPLIT = 2 };
enum Sched { SCHED_KV_STATIONARY = 0, SCHED_Q_STATIONARY = 1 };
enum Epilogue { EPI_FINAL = 0, EPI_ACC = 1, EPI_PART = 2 };

// Calls f(integral_constant<int, i>) for i = B .. E-1: compile-time indices for
// scheduling builtins and register arrays in hand-ordered instruction streams.
template <int B, int E, typename F>
__device__ inline __attribute__((always_inline)) void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// ---- direct global-to-LDS staging (global_load_lds) for the MFMA kernels

// Barrier without the memory fence of __syncthreads: direct-to-LDS loads
// stay in flight across it (their completion is awaited explicitly before the
// barrier that publishes them); this wave's LDS reads are complete first.
__device__ inline void slot_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// One direct global->LDS load: 16 bytes per lane from base + off to LDS byte
// address lds + 16 * lane (base and lds wave-uniform; lds passed in m0, with
// the one wait state an LDS DMA needs after m0 is written).  Issued from asm
// so that the compiler adds no waits of its own for it; every read of the
// loaded data follows an explicit wait_vm and a barrier.  Nothing else in the
// kernel keeps a value in m0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved: the asm sets it itself
__device__ inline void dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base),
               "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop
// A wave-uniform pointer moved to scalar registers (for dma16's base where
// the compiler cannot prove the value uniform).
template <typename Tp>
__device__ inline const Tp* uniform_ptr(const Tp* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const Tp*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ inline uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding)
template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Start of shard k of a length-S sequence split n ways: floor(k*S/n).
__host__ __device__ inline int64_t shard_start(int64_t S, int n, int k) {
  return (int64_t)k * S / n;
}

// (a - b) mod n and (a + b) mod n for 0 <= a, b < n, without a division.
__host__ __device__ inline int ring_sub(int a, int b, int n) { return a >= b ? a - b : a - b + n; }
__host__ __device__ inline int ring_add(int a, int b, int n) { return a + b < n ? a + b : a + b - n; }

// Pair held by virtual worker w in round r (0 <= w, r < n).
//   KV-stationary: Q block (w - r) mod n with KV shard w.
//   Q-stationary:  Q block w with KV shard (w - r) mod n.
__host__ __device__ inline void ring_pair(int sched, int n, int r, int w, int* qb, int* kb) {
  int moved = ring_sub(w, r, n);
  if (sched == SCHED_KV_STATIONARY) { *qb = moved; *kb = w; }
  else { *qb = w; *kb = moved; }
}

// KV shard merged into query block j at step r of its schedule order
// (0 <= j, r < n): KV-stationary visits j, j+1, ...; Q-stationary visits
// j, j-1, ... (mod n).
__host__ __device__ inline int shard_at_step(int sched, int n, int j, int r) {
  return sched == SCHED_KV_STATIONARY ? ring_add(j, r, n) : ring_sub(j, r, n);
}


// Forward launch description (one struct for every mode and dtype).
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  int64_t sqB, sqH, sqS;
  int64_t skB, skH, skS;
  int64_t svB, svH, svS;
  void* o;  // EPI_FINAL output, q's dtype
  int64_t soB, soH, soS;
  float* lse;       // [B,H,SQ]: EPI_FINAL output / EPI_ACC running LSE
  float* o_acc;     // EPI_ACC running O fp32 [B,H,SQ,D]; EPI_PART partial O [n][B,H,SQ,D]
  float* lse_part;  // EPI_PART partial LSE [n][B,H,SQ]
  int B, H, SQ, SKV, D, n;
  int sched, mode, round;
  int causal;   // 0 none, 1 rows in sequence order, 2 rows in the striped order
  int64_t blk;  // causal == 2: rows per shard (S / n)
  int tiles;   // query tiles per group
  int groups;  // groups of tiles (each group shares one KV range at a time)
  int accumulate;
  int single_pair;  // bwa_partial_fwd: one explicit pair
  int64_t q0, nq, k0, nk;
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
};

// A workgroup's job: one (batch*head, query row range) and the ordered list
// of KV segments it attends to.
struct Job {
  int bh;
  int64_t r0, r1;  // query rows [r0, r1)
  int block;       // query block (ROUNDS, FUSED) or KV shard slot (SPLIT)
  int kb;          // the one KV shard of a ROUNDS / SPLIT job
  int nseg;        // number of segment steps
  int epi;         // Epilogue
  bool acc_in;     // EPI_ACC: seed from the running (O, L)
};

// XCD-aware mapping of a linear workgroup id to (group, tile).  Workgroups are
// dispatched round-robin over the 8 XCDs (id % 8); the `tiles` workgroups of
// one group share a KV range and land on one XCD with consecutive slots, so
// they stream the same K/V tiles through that XCD's L2 at about the same time.
__device__ inline bool xcd_group_tile(int wg, int tiles, int groups, int* g, int* t) {
  int xcd = wg % kNumXcd;
  int k = wg / kNumXcd;
  *g = (k / tiles) * kNumXcd + xcd;
  *t = k % tiles;
  return *g < groups;
}

inline int xcd_grid_size(int tiles, int groups) {
  return kNumXcd * tiles * ((groups + kNumXcd - 1) / kNumXcd);
}

__device__ inline bool make_job(const FwdParams& p, int BM, Job* jb) {
  int g, t;
  if (!xcd_group_tile(blockIdx.x, p.tiles, p.groups, &g, &t)) return false;
  const int BH = p.B * p.H;
  if (p.single_pair) {
    jb->bh = g;
    jb->r0 = p.q0 + (int64_t)t * BM;
    jb->r1 = min(p.q0 + p.nq, jb->r0 + BM);
    jb->block = 0;
    jb->kb = 0;
    jb->nseg = 1;
    jb->epi = EPI_ACC;
    jb->acc_in = p.accumulate != 0;
    return jb->r0 < jb->r1;
  }
  if (p.mode == MODE_SPLIT) {
    jb->bh = g % BH;
    jb->block = g / BH;
    jb->kb = jb->block;
    jb->r0 = (int64_t)t * BM;
    jb->r1 = min((int64_t)p.SQ, jb->r0 + BM);
    jb->nseg = 1;
    jb->epi = EPI_PART;
    jb->acc_in = false;
    return jb->r0 < jb->r1;
  }
  int j;
  jb->bh = g % BH;
  if (p.mode == MODE_ROUNDS) {
    int kb;
    ring_pair(p.sched, p.n, p.round, g / BH, &j, &kb);
    jb->kb = kb;
    jb->nseg = 1;
    jb->epi = EPI_ACC;
    jb->acc_in = p.round > 0;
  } else {  // FUSED; under causal masking later query blocks do more work: start them first
    j = p.causal ? (p.n - 1 - g / BH) : (g / BH);
    jb->kb = -1;
    jb->nseg = p.n;
    jb->epi = EPI_FINAL;
    jb->acc_in = false;
    // and within a block later rows see more keys (in either causal order):
    // its row tiles go last to first
    if (p.causal) t = p.tiles - 1 - t;
  }
  jb->block = j;
  int64_t qs = shard_start(p.SQ, p.n, j), qe = shard_start(p.SQ, p.n, j + 1);
  jb->r0 = qs + (int64_t)t * BM;
  jb->r1 = min(qe, jb->r0 + BM);
  return jb->r0 < jb->r1;
}

// KV segment [*k0, *k1) of step r of a job (empty when nothing is visible).
// Under causal masking no key at or beyond the job's last row + 1 is visible.
// In the striped order (shard w holds positions w, w+n, ...; a row's shard w
// and index c give position c*n + w) a row at (w, c) sees the first c + 1
// keys of shards up to w and the first c keys of later shards, so a shard is
// cut after the job's largest such count.
__device__ inline void job_segment(const FwdParams& p, const Job& jb, int r, int64_t* k0,
                                   int64_t* k1) {
  if (p.single_pair) {
    *k0 = p.k0;
    *k1 = p.k0 + p.nk;
  } else {
    int kb = jb.kb >= 0 ? jb.kb : shard_at_step(p.sched, p.n, jb.block, r);
    *k0 = shard_start(p.SKV, p.n, kb);
    *k1 = shard_start(p.SKV, p.n, kb + 1);
  }
  if (p.causal == 1 && *k1 > jb.r1) *k1 = jb.r1;
  if (p.causal == 2) {
    const int64_t w0 = jb.r0 / p.blk, w1 = (jb.r1 - 1) / p.blk, ks = *k0 / p.blk;
    const int64_t cnt = w0 == w1 ? (jb.r1 - 1) % p.blk + (ks <= w1 ? 1 : 0) : p.blk;
    if (*k1 > *k0 + cnt) *k1 = *k0 + cnt;
  }
  if (*k1 < *k0) *k1 = *k0;
}

// Iterates the KV tiles of a job in order: segment by segment, BN keys at a time.
struct TileIter {
  int r;           // segment step
  int64_t kt, ke;  // current tile start, end of current segment
  // start of the current segment and, in the striped order, the shard it
  // starts (every segment there begins at a shard start)
  int64_t s0, sk;
  __device__ inline void seek(const FwdParams& p, const Job& jb, int from, int BN) {
    (void)BN;
    for (r = from; r < jb.nseg; ++r) {
      int64_t a, b;
      job_segment(p, jb, r, &a, &b);
      if (b > a) {
        kt = a;
        ke = b;
        s0 = a;
        sk = p.causal == 2 ? a / p.blk : 0;
        return;
      }
    }
    kt = ke = s0 = sk = 0;
  }
  __device__ inline bool valid(const Job& jb) const { return r < jb.nseg; }
  __device__ inline void advance(const FwdParams& p, const Job& jb, int BN) {
    kt += BN;
    if (kt >= ke) seek(p, jb, r + 1, BN);
  }
};

}  // namespace bwa
