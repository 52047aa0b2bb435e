// Host side of the C ABI declared in include/bwa.h: argument validation,
// workspace carving, and the stream-ordered round loop that stands in for the
// ring on one GPU.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "bwa.h"
#include "bwd_args.h"
#include "common.h"

namespace bwa {
hipError_t fwd_launch(FwdParams p, int dtype_bf16, hipStream_t st);
int fwd_tile_rows(int dtype_bf16, int D);
hipError_t merge2_launch(int64_t rows, int D, const float* oa, const float* la, const float* ob,
                         const float* lb, float* oo, float* lo, hipStream_t st);
hipError_t split_merge_launch(FwdParams p, int dtype_bf16, hipStream_t st);
hipError_t finalize_launch(FwdParams p, int dtype_bf16, hipStream_t st);
hipError_t copy_rows_launch(const void* src, int64_t sB, int64_t sH, int64_t sS, void* dst, int B,
                            int H, int64_t S, int row_bytes, hipStream_t st);
bool bwd_supported(int dtype, int D);
size_t bwd_workspace_bytes(int64_t BH, int64_t SQ, int64_t SKV, int D, int n, int mode);
hipError_t bwd_run(const BwdArgs& a, hipStream_t st);
hipError_t gemm_grad_launch(const void* y, const void* wk_t, const void* wv_t,
                            const bwa_tensor* dk, const bwa_tensor* dv, int64_t B, int64_t S,
                            int64_t E, int64_t H, int64_t Dh, float* dwk_t, float* dwv_t,
                            float* dy, int accumulate, hipStream_t st);
size_t scratch_bytes();
hipError_t scratch_ptr(void** out);
hipError_t gemm_kv_launch(const void* y, const void* wk_t, const void* wv_t, int64_t B, int64_t S,
                          int64_t E, int64_t H, int64_t D, const bwa_tensor* k,
                          const bwa_tensor* v, hipStream_t st);
}  // namespace bwa

namespace {

thread_local std::string g_last_error;

bwa_status fail(bwa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

bwa_status hip_fail(hipError_t e, const char* what) {
  return fail(BWA_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

size_t elem_size(int32_t dt) { return dt == BWA_BF16 ? 2 : 4; }

constexpr int64_t kMaxDim = (int64_t)1 << 31;
// Rows over all (batch, head) pairs of one tensor: row-parallel kernels launch
// one thread per 4 to 16 elements of a row, and their grids stay below 2^31.
constexpr int64_t kMaxRows = (int64_t)1 << 33;
// Workgroups of any one launch (gridDim.x must stay below 2^31; the XCD-aware
// mapping rounds the group count up to a multiple of 8).
constexpr int64_t kMaxGrid = (int64_t)1 << 30;

// Structural checks shared by every tensor argument.
bwa_status check_tensor(const bwa_tensor* t, const char* name, bool allow_empty_seq) {
  if (!t) return fail(BWA_ERR_INVALID_ARG, "%s is NULL", name);
  if (t->dtype != BWA_F32 && t->dtype != BWA_BF16)
    return fail(BWA_ERR_UNSUPPORTED, "%s: dtype %d not supported (fp32=0, bf16=1)", name,
                (int)t->dtype);
  if (t->B <= 0 || t->H <= 0 || t->S < 0 || (t->S == 0 && !allow_empty_seq))
    return fail(BWA_ERR_INVALID_ARG, "%s: bad shape B=%lld H=%lld S=%lld", name,
                (long long)t->B, (long long)t->H, (long long)t->S);
  if (t->D != 64 && t->D != 128)
    return fail(BWA_ERR_UNSUPPORTED, "%s: head dim %lld not supported (64 or 128)", name,
                (long long)t->D);
  if (t->B * t->H >= kMaxDim || t->S >= kMaxDim)
    return fail(BWA_ERR_UNSUPPORTED, "%s: sizes beyond 2^31 rows", name);
  if (t->B * t->H * t->S > kMaxRows)
    return fail(BWA_ERR_UNSUPPORTED, "%s: more than 2^33 rows over all heads", name);
  if (t->sB < 0 || t->sH < 0 || t->sS < 0)
    return fail(BWA_ERR_INVALID_ARG, "%s: negative stride", name);
  if (t->S == 0) return BWA_OK;
  if (!t->ptr) return fail(BWA_ERR_INVALID_ARG, "%s: NULL data pointer", name);
  size_t es = elem_size(t->dtype);
  if ((uintptr_t)t->ptr % 16 != 0 || (t->sB * es) % 16 != 0 || (t->sH * es) % 16 != 0 ||
      (t->sS * es) % 16 != 0)
    return fail(BWA_ERR_UNSUPPORTED, "%s: base and strides must be 16-byte aligned", name);
  if (t->sS * es >= ((int64_t)1 << 24))
    return fail(BWA_ERR_UNSUPPORTED, "%s: row stride of 16 MiB or more", name);
  return BWA_OK;
}

bwa_status check_qkv(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v, int causal) {
  bwa_status s;
  if ((s = check_tensor(q, "q", true)) != BWA_OK) return s;
  if ((s = check_tensor(k, "k", false)) != BWA_OK) return s;
  if ((s = check_tensor(v, "v", false)) != BWA_OK) return s;
  if (q->dtype != k->dtype || q->dtype != v->dtype)
    return fail(BWA_ERR_INVALID_ARG, "q, k, v must share one dtype");
  if (q->B != k->B || q->B != v->B || q->H != k->H || q->H != v->H)
    return fail(BWA_ERR_INVALID_ARG, "q, k, v batch/head counts differ");
  if (q->D != k->D || q->D != v->D) return fail(BWA_ERR_INVALID_ARG, "q, k, v head dims differ");
  if (k->S != v->S) return fail(BWA_ERR_INVALID_ARG, "k and v lengths differ");
  if (causal < 0 || causal > 2)
    return fail(BWA_ERR_INVALID_ARG, "causal must be 0, 1 (sequence order) or 2 (striped)");
  if (causal && q->S != k->S)
    return fail(BWA_ERR_UNSUPPORTED, "causal masking needs S_Q == S_KV (self-attention)");
  return BWA_OK;
}

bwa_status check_like(const bwa_tensor* t, const bwa_tensor* ref, int64_t S, const char* name) {
  bwa_status s = check_tensor(t, name, true);
  if (s != BWA_OK) return s;
  if (t->dtype != ref->dtype || t->B != ref->B || t->H != ref->H || t->S != S || t->D != ref->D)
    return fail(BWA_ERR_INVALID_ARG, "%s: shape or dtype does not match", name);
  return BWA_OK;
}

bwa_status check_scale(float scale) {
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(BWA_ERR_INVALID_ARG, "scale must be finite and positive");
  return BWA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ROUNDS_TRANSFER workspace: the stationary (O, L) of the Q-stationary
// schedule, then two receive slots, each large enough for either schedule's
// rotating blocks: (Q, O, L) or (K, V).
struct XferLayout {
  size_t o, l, q, kv, slot;
  XferLayout(int64_t BH, int64_t SQ, int64_t SKV, int D, size_t es) {
    o = align256((size_t)(BH * SQ * D) * 4);
    l = align256((size_t)(BH * SQ) * 4);
    q = align256((size_t)(BH * SQ * D) * es);
    kv = align256((size_t)(BH * SKV * D) * es);
    slot = q + o + l > 2 * kv ? q + o + l : 2 * kv;
  }
  size_t total() const { return o + l + 2 * slot; }
};

size_t fwd_ws_bytes(int64_t BH, int64_t SQ, int64_t SKV, int D, size_t es, int n, int mode) {
  if (mode == BWA_MODE_ROUNDS) return align256((size_t)(BH * SQ * D) * 4);
  if (mode == BWA_MODE_SPLIT)
    return align256((size_t)n * BH * SQ * D * 4) + align256((size_t)n * BH * SQ * 4);
  if (mode == BWA_MODE_ROUNDS_TRANSFER) return XferLayout(BH, SQ, SKV, D, es).total();
  return 0;
}

bwa::FwdParams base_params(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v,
                           float scale, int causal) {
  bwa::FwdParams p = {};
  p.q = q->ptr;
  p.k = k->ptr;
  p.v = v->ptr;
  p.sqB = q->sB; p.sqH = q->sH; p.sqS = q->sS;
  p.skB = k->sB; p.skH = k->sH; p.skS = k->sS;
  p.svB = v->sB; p.svH = v->sH; p.svS = v->sS;
  p.B = (int)q->B;
  p.H = (int)q->H;
  p.SQ = (int)q->S;
  p.SKV = (int)k->S;
  p.D = (int)q->D;
  p.causal = causal;
  p.scale = scale;
  p.scale_log2 = scale * bwa::kLog2e;
  return p;
}

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

bwa_status check_ring(const bwa_tensor* q, const bwa_tensor* k, int n, int mode) {
  if (n < 1 || n > k->S)
    return fail(BWA_ERR_INVALID_ARG, "n = %d shards must be in [1, S_KV = %lld]", n,
                (long long)k->S);
  if (n > 4096) return fail(BWA_ERR_UNSUPPORTED, "n = %d above 4096", n);
  // Largest grid of any ring launch: at most (B*H + 7) * n groups of at most
  // ceil(ceil(S / n) / 16) tiles (16 rows is the smallest tile of any kernel).
  const int64_t S = q->S > k->S ? q->S : k->S;
  const int64_t tiles = ((S + n - 1) / n + 15) / 16;
  if ((q->B * q->H + 7) * n * tiles > kMaxGrid)
    return fail(BWA_ERR_UNSUPPORTED, "B*H*n = %lld pairs of shards need a grid above 2^30",
                (long long)(q->B * q->H * n));
  if (mode != BWA_MODE_ROUNDS && mode != BWA_MODE_FUSED && mode != BWA_MODE_SPLIT &&
      mode != BWA_MODE_ROUNDS_TRANSFER)
    return fail(BWA_ERR_INVALID_ARG, "unknown mode %d", mode);
  return BWA_OK;
}

bwa_status check_sched(int sched) {
  if (sched != BWA_SCHED_KV_STATIONARY && sched != BWA_SCHED_Q_STATIONARY)
    return fail(BWA_ERR_INVALID_ARG, "unknown schedule %d", sched);
  return BWA_OK;
}

}  // namespace

extern "C" {

const char* bwa_status_string(bwa_status s) {
  switch (s) {
    case BWA_OK: return "BWA_OK";
    case BWA_ERR_INVALID_ARG: return "BWA_ERR_INVALID_ARG";
    case BWA_ERR_UNSUPPORTED: return "BWA_ERR_UNSUPPORTED";
    case BWA_ERR_WORKSPACE: return "BWA_ERR_WORKSPACE";
    case BWA_ERR_HIP: return "BWA_ERR_HIP";
    case BWA_ERR_INTERNAL: return "BWA_ERR_INTERNAL";
  }
  return "BWA_ERR_UNKNOWN";
}

const char* bwa_last_error(void) { return g_last_error.c_str(); }

int bwa_version(void) { return BWA_VERSION; }

bwa_status bwa_choose_schedule(int64_t S_Q, int64_t S_KV, int64_t d_model, int32_t n,
                               double flops_per_s, double bytes_per_s, int32_t elem_bytes,
                               int32_t* choice, bwa_schedule_model* model) {
  if (S_Q <= 0 || S_KV <= 0 || d_model <= 0 || n <= 0 || elem_bytes <= 0)
    return fail(BWA_ERR_INVALID_ARG, "sizes, n and elem_bytes must be positive");
  if (!(flops_per_s > 0.0) || !(bytes_per_s > 0.0) || flops_per_s == HUGE_VAL ||
      bytes_per_s == HUGE_VAL)
    return fail(BWA_ERR_INVALID_ARG, "rates must be positive and finite");
  if (!choice) return fail(BWA_ERR_INVALID_ARG, "choice is NULL");
  const double sq = (double)S_Q / n, skv = (double)S_KV / n, d = (double)d_model;
  bwa_schedule_model m;
  m.t_compute = 4.0 * sq * skv * d / flops_per_s;
  m.t_comm_kv_stationary = (2.0 * sq * d + sq) * elem_bytes / bytes_per_s;
  m.t_comm_q_stationary = 2.0 * skv * d * elem_bytes / bytes_per_s;
  m.t_round_kv_stationary = m.t_compute > m.t_comm_kv_stationary ? m.t_compute
                                                                 : m.t_comm_kv_stationary;
  m.t_round_q_stationary = m.t_compute > m.t_comm_q_stationary ? m.t_compute
                                                               : m.t_comm_q_stationary;
  *choice = m.t_round_kv_stationary <= m.t_round_q_stationary ? BWA_SCHED_KV_STATIONARY
                                                              : BWA_SCHED_Q_STATIONARY;
  if (model) *model = m;
  return BWA_OK;
}

bwa_status bwa_partial_fwd(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v,
                           int64_t q0, int64_t nq, int64_t k0, int64_t nk, float scale,
                           int causal, float* o_acc, float* lse_acc, int accumulate,
                           void* stream) {
  bwa_status s;
  if ((s = check_qkv(q, k, v, causal)) != BWA_OK) return s;
  if (causal == 2)
    return fail(BWA_ERR_UNSUPPORTED, "the striped order is defined by a ring's shards (ring_fwd)");
  if ((s = check_scale(scale)) != BWA_OK) return s;
  if (q0 < 0 || nq < 0 || q0 + nq > q->S)
    return fail(BWA_ERR_INVALID_ARG, "query range [%lld, %lld) outside [0, %lld)",
                (long long)q0, (long long)(q0 + nq), (long long)q->S);
  if (k0 < 0 || nk < 0 || k0 + nk > k->S)
    return fail(BWA_ERR_INVALID_ARG, "key range [%lld, %lld) outside [0, %lld)", (long long)k0,
                (long long)(k0 + nk), (long long)k->S);
  if (nq == 0) return BWA_OK;
  if ((q->B * q->H + 7) * ((nq + 15) / 16) > kMaxGrid)
    return fail(BWA_ERR_UNSUPPORTED, "B*H*nq needs a grid above 2^30");
  if (!o_acc || !lse_acc) return fail(BWA_ERR_INVALID_ARG, "o_acc / lse_acc is NULL");
  if ((uintptr_t)o_acc % 16 != 0) return fail(BWA_ERR_UNSUPPORTED, "o_acc must be 16-byte aligned");
  bwa::FwdParams p = base_params(q, k, v, scale, causal);
  p.single_pair = 1;
  p.q0 = q0; p.nq = nq; p.k0 = k0; p.nk = nk;
  p.accumulate = accumulate ? 1 : 0;
  p.o_acc = o_acc;
  p.lse = lse_acc;
  p.mode = bwa::MODE_ROUNDS;
  p.n = 1;
  const int bf = q->dtype == BWA_BF16;
  p.tiles = ceil_div(nq, bwa::fwd_tile_rows(bf, p.D));
  p.groups = p.B * p.H;
  hipError_t e = bwa::fwd_launch(p, bf, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "partial forward launch");
  return BWA_OK;
}

bwa_status bwa_merge(int64_t rows, int64_t D, const float* o_a, const float* lse_a,
                     const float* o_b, const float* lse_b, float* o_out, float* lse_out,
                     void* stream) {
  if (rows < 0) return fail(BWA_ERR_INVALID_ARG, "rows < 0");
  if (rows > kMaxRows) return fail(BWA_ERR_UNSUPPORTED, "more than 2^33 rows");
  if (D != 64 && D != 128) return fail(BWA_ERR_UNSUPPORTED, "D must be 64 or 128");
  if (rows == 0) return BWA_OK;
  if (!o_a || !lse_a || !o_b || !lse_b || !o_out || !lse_out)
    return fail(BWA_ERR_INVALID_ARG, "NULL pointer argument");
  if ((uintptr_t)o_a % 16 || (uintptr_t)o_b % 16 || (uintptr_t)o_out % 16)
    return fail(BWA_ERR_UNSUPPORTED, "O buffers must be 16-byte aligned");
  hipError_t e = bwa::merge2_launch(rows, (int)D, o_a, lse_a, o_b, lse_b, o_out, lse_out,
                                    (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return BWA_OK;
}

bwa_status bwa_merge_partials(int n, bwa_schedule sched, const float* o_parts,
                              const float* lse_parts, const bwa_tensor* o, float* lse,
                              void* stream) {
  bwa_status s;
  if ((s = check_tensor(o, "o", true)) != BWA_OK) return s;
  if ((s = check_sched(sched)) != BWA_OK) return s;
  if (n < 1 || n > 4096) return fail(BWA_ERR_INVALID_ARG, "n = %d outside [1, 4096]", n);
  if (o->S == 0) return BWA_OK;
  if (!o_parts || !lse_parts || !lse) return fail(BWA_ERR_INVALID_ARG, "NULL pointer argument");
  if ((uintptr_t)o_parts % 16 != 0)
    return fail(BWA_ERR_UNSUPPORTED, "o_parts must be 16-byte aligned");
  bwa::FwdParams p = {};
  p.B = (int)o->B;
  p.H = (int)o->H;
  p.SQ = (int)o->S;
  p.D = (int)o->D;
  p.n = n;
  p.sched = sched;
  p.o = o->ptr;
  p.soB = o->sB; p.soH = o->sH; p.soS = o->sS;
  p.lse = lse;
  p.o_acc = (float*)o_parts;
  p.lse_part = (float*)lse_parts;
  hipError_t e = bwa::split_merge_launch(p, o->dtype == BWA_BF16, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "merge partials launch");
  return BWA_OK;
}

size_t bwa_ring_fwd_workspace(const bwa_tensor* q, const bwa_tensor* k, int n, bwa_mode mode) {
  if (!q || !k || q->B <= 0 || q->H <= 0 || q->S < 0 || (q->D != 64 && q->D != 128) || n < 1)
    return 0;
  if (k->S < 0) return 0;
  return fwd_ws_bytes(q->B * q->H, q->S, k->S, (int)q->D, elem_size(q->dtype), n, mode);
}

bwa_status bwa_ring_fwd(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v, int n,
                        bwa_schedule sched, bwa_mode mode, int causal, float scale,
                        const bwa_tensor* o, float* lse, void* workspace, size_t ws_bytes,
                        void* stream) {
  bwa_status s;
  if ((s = check_qkv(q, k, v, causal)) != BWA_OK) return s;
  if ((s = check_like(o, q, q->S, "o")) != BWA_OK) return s;
  if ((s = check_scale(scale)) != BWA_OK) return s;
  if ((s = check_ring(q, k, n, mode)) != BWA_OK) return s;
  if ((s = check_sched(sched)) != BWA_OK) return s;
  if (q->S == 0) return BWA_OK;
  if (!lse) return fail(BWA_ERR_INVALID_ARG, "lse is NULL");
  const int64_t BH = q->B * q->H;
  size_t need = fwd_ws_bytes(BH, q->S, k->S, (int)q->D, elem_size(q->dtype), n, mode);
  if (need > 0) {
    if (!workspace || ws_bytes < need)
      return fail(BWA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
    if ((uintptr_t)workspace % 256 != 0)
      return fail(BWA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  if (causal == 2 && q->S % n != 0)
    return fail(BWA_ERR_UNSUPPORTED, "striped causal order needs n to divide S");
  bwa::FwdParams p = base_params(q, k, v, scale, causal);
  p.n = n;
  p.blk = causal == 2 ? q->S / n : 0;
  p.sched = sched;
  p.mode = mode == BWA_MODE_ROUNDS_TRANSFER ? BWA_MODE_ROUNDS : mode;
  p.o = o->ptr;
  p.soB = o->sB; p.soH = o->sH; p.soS = o->sS;
  p.lse = lse;
  const int bf = q->dtype == BWA_BF16;
  const int BM = bwa::fwd_tile_rows(bf, p.D);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  p.groups = (int)(BH * n);
  if (mode == BWA_MODE_ROUNDS) {
    p.o_acc = (float*)workspace;
    p.tiles = ceil_div(ceil_div(q->S, n), BM);
    for (int r = 0; r < n && e == hipSuccess; ++r) {
      p.round = r;
      e = bwa::fwd_launch(p, bf, st);
    }
    if (e == hipSuccess) e = bwa::finalize_launch(p, bf, st);
  } else if (mode == BWA_MODE_ROUNDS_TRANSFER) {
    // ROUNDS with the exchange made real (device copies into receive slots)
    const size_t es = elem_size(q->dtype);
    const XferLayout L(BH, q->S, k->S, (int)q->D, es);
    char* ws = (char*)workspace;
    char* slot[2] = {ws + L.o + L.l, ws + L.o + L.l + L.slot};
    const int64_t row = q->D * (int64_t)es;  // bytes of one Q/K/V row
    const int64_t qS = q->S, kS = k->S;
    p.tiles = ceil_div(ceil_div(q->S, n), BM);
    auto copy = [&](void* dst, const void* src, size_t bytes) {
      return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st);
    };
    if (sched == BWA_SCHED_KV_STATIONARY) {
      // Q_i, O_i, L_i rotate; slot r % 2 holds every worker's received set
      for (int r = 0; r < n && e == hipSuccess; ++r) {
        char* cur = slot[r % 2];
        float* oc = (float*)(cur + L.q);
        float* lc = (float*)(cur + L.q + L.o);
        if (r > 0) {
          p.q = cur;
          p.sqS = q->D; p.sqH = qS * q->D; p.sqB = q->H * qS * q->D;
        }
        p.o_acc = oc;
        p.lse = lc;
        p.round = r;
        e = bwa::fwd_launch(p, bf, st);
        if (e != hipSuccess || r + 1 == n) break;
        char* nx = slot[(r + 1) % 2];
        if (r == 0)
          e = bwa::copy_rows_launch(q->ptr, q->sB * es, q->sH * es, q->sS * es, nx, (int)q->B,
                                    (int)q->H, qS, (int)row, st);
        else
          e = copy(nx, cur, (size_t)(BH * qS) * row);
        if (e == hipSuccess) e = copy(nx + L.q, oc, (size_t)(BH * qS * q->D) * 4);
        if (e == hipSuccess) e = copy(nx + L.q + L.o, lc, (size_t)(BH * qS) * 4);
      }
      if (e == hipSuccess) e = copy(lse, p.lse, (size_t)(BH * qS) * 4);
      if (e == hipSuccess) e = bwa::finalize_launch(p, bf, st);
    } else {
      // K_i, V_i rotate; (O, L) stay with their query block
      p.o_acc = (float*)ws;
      for (int r = 0; r < n && e == hipSuccess; ++r) {
        char* cur = slot[r % 2];
        if (r > 0) {
          p.k = cur;
          p.v = cur + L.kv;
          p.skS = p.svS = k->D;
          p.skH = p.svH = kS * k->D;
          p.skB = p.svB = k->H * kS * k->D;
        }
        p.round = r;
        e = bwa::fwd_launch(p, bf, st);
        if (e != hipSuccess || r + 1 == n) break;
        char* nx = slot[(r + 1) % 2];
        if (r == 0) {
          e = bwa::copy_rows_launch(k->ptr, k->sB * es, k->sH * es, k->sS * es, nx, (int)k->B,
                                    (int)k->H, kS, (int)row, st);
          if (e == hipSuccess)
            e = bwa::copy_rows_launch(v->ptr, v->sB * es, v->sH * es, v->sS * es, nx + L.kv,
                                      (int)v->B, (int)v->H, kS, (int)row, st);
        } else {
          e = copy(nx, cur, 2 * L.kv);
        }
      }
      if (e == hipSuccess) e = bwa::finalize_launch(p, bf, st);
    }
  } else if (mode == BWA_MODE_FUSED) {
    p.tiles = ceil_div(ceil_div(q->S, n), BM);
    e = bwa::fwd_launch(p, bf, st);
  } else {
    p.o_acc = (float*)workspace;
    p.lse_part = (float*)((char*)workspace + align256((size_t)n * BH * q->S * q->D * 4));
    p.tiles = ceil_div(q->S, BM);
    e = bwa::fwd_launch(p, bf, st);
    if (e == hipSuccess) e = bwa::split_merge_launch(p, bf, st);
  }
  if (e != hipSuccess) return hip_fail(e, "ring forward launch");
  return BWA_OK;
}

size_t bwa_ring_bwd_workspace(const bwa_tensor* q, const bwa_tensor* k, int n, bwa_mode mode) {
  if (!q || !k || q->B <= 0 || q->H <= 0 || q->S < 0 || k->S < 0 ||
      (q->D != 64 && q->D != 128) || n < 1)
    return 0;
  return bwa::bwd_workspace_bytes(q->B * q->H, q->S, k->S, (int)q->D, n, mode);
}

}  // extern "C"

namespace {

// Argument checks shared by bwa_ring_bwd and its allocation-free variant.
bwa_status check_bwd(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v,
                     const bwa_tensor* o, const float* lse, const bwa_tensor* dout, int n,
                     bwa_schedule sched, bwa_mode mode, int causal, float scale,
                     const bwa_tensor* dq, const bwa_tensor* dk, const bwa_tensor* dv) {
  bwa_status s;
  if ((s = check_qkv(q, k, v, causal)) != BWA_OK) return s;
  if ((s = check_like(o, q, q->S, "o")) != BWA_OK) return s;
  if ((s = check_like(dout, q, q->S, "dout")) != BWA_OK) return s;
  if ((s = check_like(dq, q, q->S, "dq")) != BWA_OK) return s;
  if ((s = check_like(dk, q, k->S, "dk")) != BWA_OK) return s;
  if ((s = check_like(dv, q, k->S, "dv")) != BWA_OK) return s;
  if ((s = check_scale(scale)) != BWA_OK) return s;
  if (mode == BWA_MODE_ROUNDS_TRANSFER)
    return fail(BWA_ERR_UNSUPPORTED, "ROUNDS_TRANSFER is a forward mode");
  if ((s = check_ring(q, k, n, mode)) != BWA_OK) return s;
  if ((s = check_sched(sched)) != BWA_OK) return s;
  if (causal == 2 && q->S % n != 0)
    return fail(BWA_ERR_UNSUPPORTED, "striped causal order needs n to divide S");
  if (!bwa::bwd_supported(q->dtype, (int)q->D))
    return fail(BWA_ERR_UNSUPPORTED, "backward implemented for bf16 only (D = 64 or 128)");
  if (q->S > 0 && !lse) return fail(BWA_ERR_INVALID_ARG, "lse is NULL");
  return BWA_OK;
}

bwa_status run_bwd(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v,
                   const bwa_tensor* o, const float* lse, const bwa_tensor* dout, int n,
                   bwa_schedule sched, bwa_mode mode, int causal, float scale,
                   const bwa_tensor* dq, const bwa_tensor* dk, const bwa_tensor* dv,
                   void* workspace, void* stream) {
  bwa::BwdArgs a = {};
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.dq = dq; a.dk = dk; a.dv = dv;
  a.lse = lse;
  a.n = n;
  a.sched = sched;
  a.mode = mode;
  a.causal = causal;
  a.scale = scale;
  a.workspace = workspace;
  hipError_t e = bwa::bwd_run(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "ring backward launch");
  return BWA_OK;
}

}  // namespace

extern "C" {

bwa_status bwa_ring_bwd(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v,
                        const bwa_tensor* o, const float* lse, const bwa_tensor* dout, int n,
                        bwa_schedule sched, bwa_mode mode, int causal, float scale,
                        const bwa_tensor* dq, const bwa_tensor* dk, const bwa_tensor* dv,
                        void* workspace, size_t ws_bytes, void* stream) {
  bwa_status s = check_bwd(q, k, v, o, lse, dout, n, sched, mode, causal, scale, dq, dk, dv);
  if (s != BWA_OK) return s;
  if (q->S == 0) return BWA_OK;
  const int64_t BH = q->B * q->H;
  size_t need = bwa::bwd_workspace_bytes(BH, q->S, k->S, (int)q->D, n, mode);
  if (need > 0) {
    if (!workspace || ws_bytes < need)
      return fail(BWA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
    if ((uintptr_t)workspace % 256 != 0)
      return fail(BWA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  return run_bwd(q, k, v, o, lse, dout, n, sched, mode, causal, scale, dq, dk, dv, workspace,
                 stream);
}

bwa_status bwa_ring_bwd_noalloc(const bwa_tensor* q, const bwa_tensor* k, const bwa_tensor* v,
                                const bwa_tensor* o, const float* lse, const bwa_tensor* dout,
                                int n, bwa_schedule sched, bwa_mode mode, int causal, float scale,
                                const bwa_tensor* dq, const bwa_tensor* dk, const bwa_tensor* dv,
                                void* stream) {
  bwa_status s = check_bwd(q, k, v, o, lse, dout, n, sched, mode, causal, scale, dq, dk, dv);
  if (s != BWA_OK) return s;
  if (mode == BWA_MODE_ROUNDS)
    return fail(BWA_ERR_UNSUPPORTED,
                "the allocation-free backward runs FUSED (or SPLIT, the same); ROUNDS carries "
                "fp32 dQ/dK/dV accumulators beyond its scratch array");
  if (q->S == 0) return BWA_OK;
  const size_t need =
      bwa::bwd_workspace_bytes(q->B * q->H, q->S, k->S, (int)q->D, n, BWA_MODE_FUSED);
  if (need > bwa::scratch_bytes())
    return fail(BWA_ERR_WORKSPACE,
                "scratch of %zu bytes needed (B*H*S_Q*4), the allocation-free backward has %zu",
                need, bwa::scratch_bytes());
  void* ptr = nullptr;
  hipError_t e = bwa::scratch_ptr(&ptr);
  if (e != hipSuccess) return hip_fail(e, "scratch array address");
  return run_bwd(q, k, v, o, lse, dout, n, sched, BWA_MODE_FUSED, causal, scale, dq, dk, dv, ptr,
                 stream);
}

bwa_status bwa_kv_recompute(const void* y, const void* wk_t, const void* wv_t, int64_t B,
                            int64_t S_KV, int64_t E, int64_t H, int64_t D, int32_t dtype,
                            const bwa_tensor* k, const bwa_tensor* v, void* stream) {
  if (dtype != BWA_BF16) return fail(BWA_ERR_UNSUPPORTED, "kv_recompute is bf16 only");
  if (B <= 0 || S_KV < 0 || E <= 0 || H <= 0) return fail(BWA_ERR_INVALID_ARG, "bad sizes");
  if (D != 64 && D != 128) return fail(BWA_ERR_UNSUPPORTED, "D must be 64 or 128");
  if (E % 64 != 0) return fail(BWA_ERR_UNSUPPORTED, "E must be a multiple of 64");
  if ((H * D) % 128 != 0) return fail(BWA_ERR_UNSUPPORTED, "H*D must be a multiple of 128");
  if (B * S_KV >= kMaxDim || E >= kMaxDim) return fail(BWA_ERR_UNSUPPORTED, "sizes too large");
  if ((B * S_KV) * E * 2 >= ((int64_t)1 << 32) || (H * D) * E * 2 >= ((int64_t)1 << 32))
    return fail(BWA_ERR_UNSUPPORTED, "y and each W must be smaller than 4 GiB");
  bwa_status s;
  if ((s = check_tensor(k, "k", true)) != BWA_OK) return s;
  if ((s = check_tensor(v, "v", true)) != BWA_OK) return s;
  if (k->dtype != BWA_BF16 || v->dtype != BWA_BF16 || k->B != B || v->B != B || k->H != H ||
      v->H != H || k->S != S_KV || v->S != S_KV || k->D != D || v->D != D)
    return fail(BWA_ERR_INVALID_ARG, "k / v shape or dtype does not match [B, H, S_KV, D] bf16");
  if (S_KV == 0) return BWA_OK;
  if (!y || !wk_t || !wv_t) return fail(BWA_ERR_INVALID_ARG, "NULL input pointer");
  if ((uintptr_t)y % 16 || (uintptr_t)wk_t % 16 || (uintptr_t)wv_t % 16)
    return fail(BWA_ERR_UNSUPPORTED, "y, wk_t, wv_t must be 16-byte aligned");
  hipError_t e = bwa::gemm_kv_launch(y, wk_t, wv_t, B, S_KV, E, H, D, k, v, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kv recompute launch");
  return BWA_OK;
}

bwa_status bwa_kv_recompute_bwd(const void* y, const void* wk_t, const void* wv_t,
                                const bwa_tensor* dk, const bwa_tensor* dv, int64_t B,
                                int64_t S_KV, int64_t E, int64_t H, int64_t D, float* dwk_t,
                                float* dwv_t, float* dy, int32_t accumulate, void* stream) {
  if (B <= 0 || S_KV <= 0 || E <= 0 || H <= 0) return fail(BWA_ERR_INVALID_ARG, "bad sizes");
  if (D != 64 && D != 128) return fail(BWA_ERR_UNSUPPORTED, "D must be 64 or 128");
  if (E % 256 != 0) return fail(BWA_ERR_UNSUPPORTED, "E must be a multiple of 256");
  if ((H * D) % 256 != 0) return fail(BWA_ERR_UNSUPPORTED, "H*D must be a multiple of 256");
  if (S_KV % 64 != 0) return fail(BWA_ERR_UNSUPPORTED, "S_KV must be a multiple of 64");
  if (B * S_KV >= kMaxDim || E >= kMaxDim || H * D >= kMaxDim)
    return fail(BWA_ERR_UNSUPPORTED, "sizes too large");
  bwa_status s;
  if ((s = check_tensor(dk, "dk", false)) != BWA_OK) return s;
  if ((s = check_tensor(dv, "dv", false)) != BWA_OK) return s;
  if (dk->dtype != BWA_BF16 || dv->dtype != BWA_BF16 || dk->B != B || dv->B != B ||
      dk->H != H || dv->H != H || dk->S != S_KV || dv->S != S_KV || dk->D != D || dv->D != D)
    return fail(BWA_ERR_INVALID_ARG, "dk / dv shape or dtype does not match [B, H, S_KV, D] bf16");
  if (dk->sB != dv->sB || dk->sH != dv->sH || dk->sS != dv->sS)
    return fail(BWA_ERR_UNSUPPORTED, "dk and dv must share one layout (equal strides)");
  if (!dwk_t && !dwv_t && !dy) return fail(BWA_ERR_INVALID_ARG, "no output requested");
  if (!y || !wk_t || !wv_t) return fail(BWA_ERR_INVALID_ARG, "NULL input pointer");
  if ((uintptr_t)y % 16 || (uintptr_t)wk_t % 16 || (uintptr_t)wv_t % 16)
    return fail(BWA_ERR_UNSUPPORTED, "y, wk_t, wv_t must be 16-byte aligned");
  if ((uintptr_t)dwk_t % 4 || (uintptr_t)dwv_t % 4 || (uintptr_t)dy % 4)
    return fail(BWA_ERR_UNSUPPORTED, "outputs must be 4-byte aligned");
  hipError_t e = bwa::gemm_grad_launch(y, wk_t, wv_t, dk, dv, B, S_KV, E, H, D, dwk_t, dwv_t, dy,
                                       accumulate ? 1 : 0, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kv recompute backward launch");
  return BWA_OK;
}

}  // extern "C"
