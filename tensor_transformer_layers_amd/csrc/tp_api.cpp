// C ABI of libtp: argument validation, workspace layout and kernel dispatch.
// Every check runs before the first HIP call, so a rejected call launches
// nothing (and never touches the GPU).
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <cmath>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/tp.h"
#include "tp_kernels.hpp"

namespace {

typedef uint16_t bf16_t;  // bf16 storage on the host side (pointer arithmetic only)

thread_local std::string g_err;

tp_status fail(tp_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

tp_status ok() {
  g_err.clear();
  return TP_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int64_t vec_of(tp_dtype dt) { return dt == TP_BF16 ? 8 : 4; }
size_t esize(tp_dtype dt) { return dt == TP_BF16 ? 2 : 4; }
const char* dt_name(tp_dtype dt) { return dt == TP_BF16 ? "bf16" : "f32"; }

constexpr int64_t kIntMax = 0x7fffffff;
constexpr int kMaxOverlapChunks = 64;
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool log_enabled() {
  static const bool on = [] {
    const char* e = getenv("TP_LOG");
    return e && *e && *e != '0';
  }();
  return on;
}

// ------------------------------------------------------------ kernel timing
// When enabled, each kernel launch below carries a HIP start/stop event pair
// attached to its own dispatch (hipExtLaunchKernelGGL), so the pair spans the
// kernel's execution on the launching stream and nothing else;
// tp_timing_read() resolves the pairs into per-kernel totals.  Off by
// default: no events are created or recorded.
struct PendingPair {
  std::string name;
  hipEvent_t a, b;
};
std::mutex g_tmu;
bool g_timing = false;
std::vector<PendingPair> g_pending;
std::vector<hipEvent_t> g_event_pool;
std::map<std::string, std::pair<double, int64_t>> g_totals;
std::vector<std::string> g_names;  // storage for tp_timing_read's name pointers
thread_local tp::LaunchEvents t_armed = {nullptr, nullptr};  // for the next launch on this thread

hipEvent_t pooled_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Arms an event pair for the one kernel launch inside its scope; stop()
// files the pair if the launch took it (a launch skipped for an empty
// problem leaves it armed, and the events go back to the pool).
struct KernelTimer {
  const char* name;
  hipEvent_t a = nullptr, b = nullptr;
  KernelTimer(const char* n, hipStream_t) : name(n) {
    std::lock_guard<std::mutex> g(g_tmu);
    if (!g_timing) return;
    a = pooled_event();
    b = pooled_event();
    if (!a || !b) {
      if (a) g_event_pool.push_back(a);
      if (b) g_event_pool.push_back(b);
      a = b = nullptr;
      return;
    }
    t_armed = {a, b};
  }
  void stop() {
    if (!a) return;
    const bool used = t_armed.start == nullptr;
    t_armed = {nullptr, nullptr};
    std::lock_guard<std::mutex> g(g_tmu);
    if (used) {
      g_pending.push_back({name, a, b});
    } else {
      g_event_pool.push_back(a);
      g_event_pool.push_back(b);
    }
    a = b = nullptr;
  }
};

tp_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(TP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

tp_status check_dtype(tp_dtype dt) {
  if (dt != TP_F32 && dt != TP_BF16) return fail(TP_ERR_DTYPE, "dtype %d is not TP_F32 or TP_BF16", (int)dt);
  return TP_OK;
}

// One GEMM operand: rows x cols view with leading dimension ld.
tp_status check_matrix(const char* name, const void* p, int64_t rows, int64_t cols, int64_t ld,
                       int64_t vec) {
  if (!p) return fail(TP_ERR_NULL, "%s is NULL", name);
  if (ld < cols) return fail(TP_ERR_SHAPE, "%s: leading dimension %lld < %lld columns", name, (long long)ld,
                             (long long)cols);
  if (!aligned16(p)) return fail(TP_ERR_ALIGN, "%s is not 16-byte aligned", name);
  if (ld % vec) return fail(TP_ERR_ALIGN, "%s: leading dimension %lld is not a multiple of %lld", name,
                            (long long)ld, (long long)vec);
  if (rows > kIntMax || cols > kIntMax) return fail(TP_ERR_SHAPE, "%s: dimension exceeds 2^31-1", name);
  // the kernels address a tile of up to 256 rows through one buffer resource
  // with 32-bit byte offsets
  const int64_t es = 16 / vec;
  if (ld * es * 256 >= (int64_t(1) << 32))
    return fail(TP_ERR_SHAPE, "%s: leading dimension %lld too large (256 rows of it exceed 4 GiB of offsets)", name,
                (long long)ld);
  return TP_OK;
}

#define TP_TRY(x)                 \
  do {                            \
    tp_status s_ = (x);           \
    if (s_ != TP_OK) return s_;   \
  } while (0)

tp_status check_slices(int64_t T, int n_slices, int slice) {
  if (n_slices < 1) return fail(TP_ERR_SHAPE, "n_slices %d < 1", n_slices);
  if (slice < -1 || slice >= n_slices)
    return fail(TP_ERR_SHAPE, "slice %d outside [-1, %d)", slice, n_slices);
  if (T % n_slices)
    return fail(TP_ERR_DIVISIBILITY, "T=%lld tokens do not split into %d sequence slices", (long long)T,
                n_slices);
  return TP_OK;
}

tp_status validate_reduce(tp_dtype out_dt, int n_parts, int64_t T, int64_t H, const float* P,
                          int64_t part_stride, const void* bias, const void* Y, int n_slices, int slice) {
  TP_TRY(check_dtype(out_dt));
  if (n_parts < 1 || n_parts > 1024) return fail(TP_ERR_SHAPE, "n_parts %d outside [1, 1024]", n_parts);
  if (T < 0 || H <= 0) return fail(TP_ERR_SHAPE, "T=%lld, H=%lld", (long long)T, (long long)H);
  if (H % 8) return fail(TP_ERR_ALIGN, "H=%lld is not a multiple of 8", (long long)H);
  TP_TRY(check_slices(T, n_slices, slice));
  if (T == 0) return TP_OK;  // empty input: nothing to read or write
  if (!P) return fail(TP_ERR_NULL, "P is NULL");
  if (!Y) return fail(TP_ERR_NULL, "Y is NULL");
  if (!aligned16(P) || !aligned16(Y)) return fail(TP_ERR_ALIGN, "P or Y is not 16-byte aligned");
  if (bias && !aligned16(bias)) return fail(TP_ERR_ALIGN, "bias is not 16-byte aligned");
  if (n_parts > 1 && part_stride < T * H)
    return fail(TP_ERR_SHAPE, "part_stride %lld < T*H = %lld (partials overlap)", (long long)part_stride,
                (long long)(T * H));
  if (part_stride % 4) return fail(TP_ERR_ALIGN, "part_stride %lld is not a multiple of 4", (long long)part_stride);
  return TP_OK;
}

tp_status run_reduce(hipStream_t s, tp_dtype out_dt, int n_parts, int64_t T, int64_t H, const float* P,
                     int64_t part_stride, const void* bias, void* Y, int n_slices, int slice) {
  tp::ReduceParams r{};
  r.P = P;
  r.part_stride = part_stride;
  r.n_parts = n_parts;
  r.H = H;
  r.rows = slice < 0 ? T : T / n_slices;
  r.row0 = slice < 0 ? 0 : (int64_t)slice * (T / n_slices);
  r.bias = bias;
  r.Y = Y;
  r.ldy = H;
  KernelTimer kt("reduce_partials", s);
  const hipError_t e = tp::launch_reduce(r, out_dt == TP_BF16, s);
  kt.stop();
  return hip_status(e, "reduce_partials launch");
}

tp_status validate_norm(tp_dtype dt, int n_slices, int64_t T, int64_t H, const void* X, int64_t slice_stride,
                        int64_t ldx, const void* gamma, float eps, const void* Y, int64_t ldy, int slice) {
  TP_TRY(check_dtype(dt));
  if (T < 0 || H <= 0) return fail(TP_ERR_SHAPE, "T=%lld, H=%lld", (long long)T, (long long)H);
  const int64_t vec = dt == TP_BF16 ? 8 : 4;
  if (H % vec) return fail(TP_ERR_ALIGN, "H=%lld is not a multiple of %lld", (long long)H, (long long)vec);
  const int64_t hmax = tp::rmsnorm_max_hidden(dt == TP_BF16);
  if (H > hmax) return fail(TP_ERR_SHAPE, "H=%lld exceeds the norm kernel's limit %lld", (long long)H, (long long)hmax);
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(TP_ERR_SHAPE, "eps=%g must be finite and >= 0", (double)eps);
  TP_TRY(check_slices(T, n_slices, slice));
  if (T == 0) return TP_OK;  // empty input: nothing to read or write
  const int64_t per = T / n_slices;
  TP_TRY(check_matrix("X", X, per, H, ldx, vec));
  TP_TRY(check_matrix("Y", Y, T, H, ldy, vec));
  if (!gamma) return fail(TP_ERR_NULL, "gamma is NULL");
  if (!aligned16(gamma)) return fail(TP_ERR_ALIGN, "gamma is not 16-byte aligned");
  if (slice_stride % vec)
    return fail(TP_ERR_ALIGN, "slice_stride %lld is not a multiple of %lld", (long long)slice_stride, (long long)vec);
  if (n_slices > 1 && slice_stride < (per - 1) * ldx + H)
    return fail(TP_ERR_SHAPE, "slice_stride %lld < (T/n_slices - 1)*ldx + H = %lld (slices overlap)",
                (long long)slice_stride, (long long)((per - 1) * ldx + H));
  return TP_OK;
}

tp_status validate_norm_split(const tp_norm_split_desc* d, size_t* need) {
  if (!d) return fail(TP_ERR_NULL, "descriptor is NULL");
  TP_TRY(check_dtype(d->dt));
  if (d->kind != TP_NORM_RMS && d->kind != TP_NORM_LAYER) return fail(TP_ERR_DTYPE, "norm kind %d unknown", (int)d->kind);
  if (d->T < 0 || d->H <= 0 || d->N <= 0)
    return fail(TP_ERR_SHAPE, "T=%lld H=%lld N=%d", (long long)d->T, (long long)d->H, d->N);
  if (d->H % d->N)
    return fail(TP_ERR_DIVISIBILITY, "hidden H=%lld is not divisible by N=%d shards (shard would be %lld + %lld/%d)",
                (long long)d->H, d->N, (long long)(d->H / d->N), (long long)(d->H % d->N), d->N);
  if (d->shard_begin < 0 || d->shard_count < 1 || d->shard_begin + d->shard_count > d->N)
    return fail(TP_ERR_SHAPE, "shard range [%d, %d) outside [0, %d)", d->shard_begin,
                d->shard_begin + d->shard_count, d->N);
  const int64_t vec = vec_of(d->dt), Hs = d->H / d->N;
  if (Hs % vec)
    return fail(TP_ERR_ALIGN, "shard width H/N=%lld is not a multiple of %lld (%s)", (long long)Hs, (long long)vec,
                dt_name(d->dt));
  const int64_t hmax = tp::rmsnorm_max_hidden(d->dt == TP_BF16);
  if (Hs > hmax)
    return fail(TP_ERR_SHAPE, "shard width H/N=%lld exceeds the norm kernel's limit %lld", (long long)Hs, (long long)hmax);
  if (!(d->eps >= 0.0f) || !std::isfinite(d->eps))
    return fail(TP_ERR_SHAPE, "eps=%g must be finite and >= 0", (double)d->eps);
  if (d->kind == TP_NORM_RMS && d->beta) return fail(TP_ERR_SHAPE, "RMSNorm takes no beta (must be NULL)");
  *need = 0;
  if (d->T == 0) return TP_OK;  // empty input: nothing to read or write
  TP_TRY(check_matrix("X", d->X, d->T, d->H, d->ldx, vec));
  TP_TRY(check_matrix("Y", d->Y, d->T, d->H, d->ldy, vec));
  if (!d->gamma) return fail(TP_ERR_NULL, "gamma is NULL");
  if (!aligned16(d->gamma)) return fail(TP_ERR_ALIGN, "gamma is not 16-byte aligned");
  if (d->beta && !aligned16(d->beta)) return fail(TP_ERR_ALIGN, "beta is not 16-byte aligned");
  if (d->T > kIntMax || (int64_t)d->N * d->T > kIntMax) return fail(TP_ERR_SHAPE, "N*T exceeds 2^31-1");
  *need = align256((size_t)d->N * d->T * 2 * sizeof(float));
  return TP_OK;
}

tp::GemmParams gemm(const void* A, int64_t lda, int64_t sA, const void* B, int64_t ldb, int64_t sB, void* C,
                    int64_t ldc, int64_t sC, int64_t M, int64_t N, int64_t K, int batch) {
  tp::GemmParams p{};
  p.A = A;
  p.lda = lda;
  p.sA = sA;
  p.B = B;
  p.ldb = ldb;
  p.sB = sB;
  p.C = C;
  p.ldc = ldc;
  p.sC = sC;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.batch = batch;
  return p;
}

hipError_t launch(const char* name, tp_dtype dt, const tp::GemmParams& p, tp::Epilogue e, hipStream_t s) {
  KernelTimer kt(name, s);
  const hipError_t r = dt == TP_BF16 ? tp::launch_gemm_bf16(p, e, s) : tp::launch_gemm_f32(p, e, s);
  kt.stop();
  return r;
}

// ------------------------------------------------------------------ MLP desc
struct MlpShape {
  int64_t Fs;        // intermediate per shard
  int64_t a_rows;    // rows of one shard's column weight block
  size_t p_bytes;    // fp32 partial slab (N slots)
  size_t h_offset;   // intermediate slab offset
  size_t h_bytes;
  int64_t h_ld;      // row pitch of the intermediate: Fs rounded up to 128 bytes, so
                     // that the row GEMM's operand rows start on cache-line boundaries
  size_t total;
};

tp_status validate_mlp(const tp_mlp_desc* d, MlpShape* sh) {
  if (!d) return fail(TP_ERR_NULL, "descriptor is NULL");
  TP_TRY(check_dtype(d->dt));
  if (d->act != TP_ACT_NONE && d->act != TP_ACT_GELU && d->act != TP_ACT_SWIGLU)
    return fail(TP_ERR_DTYPE, "activation %d unknown", (int)d->act);
  if (d->act == TP_ACT_SWIGLU && d->dt != TP_BF16) return fail(TP_ERR_DTYPE, "SwiGLU path is bf16-only");
  if (d->act == TP_ACT_SWIGLU && d->a) return fail(TP_ERR_SHAPE, "SwiGLU column bias must be NULL");
  if (d->T < 0 || d->H <= 0 || d->F <= 0 || d->N <= 0)
    return fail(TP_ERR_SHAPE, "T=%lld H=%lld F=%lld N=%d", (long long)d->T, (long long)d->H, (long long)d->F,
                d->N);
  if (d->F % d->N)
    return fail(TP_ERR_DIVISIBILITY,
                "intermediate F=%lld is not divisible by N=%d shards (shard would be %lld + %lld/%d columns)",
                (long long)d->F, d->N, (long long)(d->F / d->N), (long long)(d->F % d->N), d->N);
  if (d->shard_begin < 0 || d->shard_count < 1 || d->shard_begin + d->shard_count > d->N)
    return fail(TP_ERR_SHAPE, "shard range [%d, %d) outside [0, %d)", d->shard_begin,
                d->shard_begin + d->shard_count, d->N);
  TP_TRY(check_slices(d->T, d->n_slices, d->slice));
  const int64_t vec = vec_of(d->dt);
  const int64_t Fs = d->F / d->N;
  if (d->T == 0) {  // empty input: nothing to read, write or stage
    sh->Fs = Fs;
    sh->a_rows = d->act == TP_ACT_SWIGLU ? 2 * Fs : Fs;
    sh->p_bytes = sh->h_offset = sh->h_bytes = sh->total = 0;
    sh->h_ld = Fs;
    return TP_OK;
  }
  if (d->H % 8) return fail(TP_ERR_ALIGN, "hidden H=%lld is not a multiple of 8", (long long)d->H);
  if (Fs % vec)
    return fail(TP_ERR_ALIGN, "shard width F/N=%lld is not a multiple of %lld (%s)", (long long)Fs,
                (long long)vec, dt_name(d->dt));
  const int64_t a_rows = d->act == TP_ACT_SWIGLU ? 2 * Fs : Fs;
  TP_TRY(check_matrix("X", d->X, d->T, d->H, d->H, vec));
  TP_TRY(check_matrix("A", d->A, a_rows * d->N, d->H, d->H, vec));
  TP_TRY(check_matrix("B", d->B, d->H, d->F, d->F, vec));
  if (d->a && !aligned16(d->a)) return fail(TP_ERR_ALIGN, "a is not 16-byte aligned");
  if (d->b && !aligned16(d->b)) return fail(TP_ERR_ALIGN, "b is not 16-byte aligned");
  if (d->shard_count == d->N) {
    if (!d->Y) return fail(TP_ERR_NULL, "Y is NULL");
    if (!aligned16(d->Y)) return fail(TP_ERR_ALIGN, "Y is not 16-byte aligned");
  }
  if (d->Z) {
    if (d->dt != TP_BF16) return fail(TP_ERR_DTYPE, "the stored pre-activation Z is written by the bf16 path only");
    const int64_t zw = d->act == TP_ACT_SWIGLU ? 2 * d->F : d->F;  // SwiGLU: [gate | up] per shard
    TP_TRY(check_matrix("Z", d->Z, d->T, zw, zw, vec));
  }
  if (d->Hact) {
    if (d->dt != TP_BF16) return fail(TP_ERR_DTYPE, "the stored activation Hact is written by the bf16 path only");
    if (d->act == TP_ACT_NONE)
      return fail(TP_ERR_SHAPE, "Hact with no activation: the intermediate is the pre-activation (use Z)");
    TP_TRY(check_matrix("Hact", d->Hact, d->T, d->F, d->F, vec));
  }
  if (d->T > kIntMax) return fail(TP_ERR_SHAPE, "T exceeds 2^31-1");
  sh->Fs = Fs;
  sh->a_rows = a_rows;
  sh->p_bytes = align256((size_t)d->N * d->T * d->H * sizeof(float));
  sh->h_offset = sh->p_bytes;
  const int64_t line = 128 / (int64_t)esize(d->dt);
  sh->h_ld = (Fs + line - 1) / line * line;
  sh->h_bytes = align256((size_t)d->shard_count * d->T * sh->h_ld * esize(d->dt));
  sh->total = sh->h_offset + sh->h_bytes;
  return TP_OK;
}

// ------------------------------------------------------------ attention desc
struct AttnShape {
  int64_t T, hl, hd;  // tokens, local heads, local width hl*head_dim
  size_t p_bytes, qk_off, vt_off, o_off, total;
};

tp_status validate_attn(const tp_attn_desc* d, AttnShape* sh) {
  if (!d) return fail(TP_ERR_NULL, "descriptor is NULL");
  TP_TRY(check_dtype(d->dt));
  if (d->dt != TP_BF16) return fail(TP_ERR_DTYPE, "attention path is bf16-only");
  if (d->batch < 0 || d->seq < 0 || d->hidden <= 0 || d->heads <= 0 || d->N <= 0)
    return fail(TP_ERR_SHAPE, "batch=%lld seq=%lld hidden=%lld heads=%d N=%d", (long long)d->batch,
                (long long)d->seq, (long long)d->hidden, d->heads, d->N);
  if (d->head_dim != 128) return fail(TP_ERR_SHAPE, "head_dim=%d (only 128 is built)", d->head_dim);
  if ((int64_t)d->heads * d->head_dim != d->hidden)
    return fail(TP_ERR_SHAPE, "heads*head_dim=%lld != hidden=%lld", (long long)d->heads * d->head_dim,
                (long long)d->hidden);
  if (d->heads % d->N)
    return fail(TP_ERR_DIVISIBILITY, "heads=%d are not divisible by N=%d shards (whole heads per shard)",
                d->heads, d->N);
  if (d->seq % 128) return fail(TP_ERR_SHAPE, "seq=%lld is not a multiple of 128", (long long)d->seq);
  if (d->shard_begin < 0 || d->shard_count < 1 || d->shard_begin + d->shard_count > d->N)
    return fail(TP_ERR_SHAPE, "shard range [%d, %d) outside [0, %d)", d->shard_begin,
                d->shard_begin + d->shard_count, d->N);
  const int64_t T = d->batch * d->seq;
  TP_TRY(check_slices(T, d->n_slices, d->slice));
  const int64_t hl = d->heads / d->N, hd = hl * d->head_dim;
  if (T == 0) {  // empty input: nothing to read, write or stage
    sh->T = 0;
    sh->hl = hl;
    sh->hd = hd;
    sh->p_bytes = sh->qk_off = sh->vt_off = sh->o_off = sh->total = 0;
    return TP_OK;
  }
  TP_TRY(check_matrix("X", d->X, T, d->hidden, d->hidden, 8));
  TP_TRY(check_matrix("Wqkv", d->Wqkv, 3 * hd * d->N, d->hidden, d->hidden, 8));
  TP_TRY(check_matrix("Wo", d->Wo, d->hidden, d->hidden, d->hidden, 8));
  if (d->bo && !aligned16(d->bo)) return fail(TP_ERR_ALIGN, "bo is not 16-byte aligned");
  if (d->shard_count == d->N) {
    if (!d->Y) return fail(TP_ERR_NULL, "Y is NULL");
    if (!aligned16(d->Y)) return fail(TP_ERR_ALIGN, "Y is not 16-byte aligned");
  }
  if (T > kIntMax) return fail(TP_ERR_SHAPE, "batch*seq exceeds 2^31-1");
  // the staged V^T rows (T keys each) and one sequence's Q|K rows are
  // addressed with 32-bit byte offsets
  if (T * 2 * 256 >= (int64_t(1) << 32))
    return fail(TP_ERR_SHAPE, "batch*seq=%lld exceeds the %lld-token limit of the staged V^T", (long long)T,
                (long long)((int64_t(1) << 32) / 512 - 1));
  if (d->seq * 2 * hd * 2 >= (int64_t(1) << 32))
    return fail(TP_ERR_SHAPE, "seq=%lld too long for the staged Q|K rows", (long long)d->seq);
  const size_t c = (size_t)d->shard_count;
  sh->T = T;
  sh->hl = hl;
  sh->hd = hd;
  sh->p_bytes = align256((size_t)d->N * T * d->hidden * sizeof(float));
  sh->qk_off = sh->p_bytes;
  sh->vt_off = sh->qk_off + align256(c * T * 2 * hd * 2);
  sh->o_off = sh->vt_off + align256(c * hd * T * 2);
  sh->total = sh->o_off + align256(c * T * hd * 2);
  return TP_OK;
}

// ------------------------------------------------------- MLP backward desc
// Workspace (256-byte aligned pieces, bf16 unless noted), Fc = shard_count*Fs:
//   P    N x [T x H] fp32   dX partials, slot i = shard i
//   Z    [T x Fz] (ld zld)  recomputed pre-activation (Fz = Fc, or 2*Fc for
//                           SwiGLU: each shard's [gate | up] columns)
//   dZ   [T x Fz] (ld zld)
//   Hs   [T x Fc]           act(Z): SiLU(gate)*up or GELU(Z), written by the dZ
//                           kernel's epilogue (SwiGLU, the two-pass GELU kernel,
//                           and GELU on the direct path)
//   XT, dYT [H x T];  HT [Fc x T];  dZT [Fz x T];  AT [H x Fz];  BT [Fc x H]
//                           transposed operands: the transposing path only,
//                           except BT for the two-pass GELU kernel
//   CS   fp32               column-sum partials of da and db (direct path)
//   K    S x [Fz x H] fp32  split-K partials of the weight gradients
//
// The direct path (bf16, shapes the K-outer GEMM takes) reads every operand
// as stored: the GEMMs take dZ, X, dY, act(Z) and the weight rows K-outer, and
// the bias gradients are column sums.  Otherwise (fp32, or a contraction
// length not a multiple of 64) the operands are transposed first.
struct BwdShape {
  int64_t Fs, Fc, zld;
  int64_t Fz;   // columns of Z and dZ: Fc, or 2*Fc for SwiGLU ([gate | up] per shard)
  int splits;   // split-K factor of the token-axis contractions
  bool direct;  // operands read as stored (K-outer GEMM operands)
  size_t p_bytes, z_off, dz_off, h_off, xt_off, dyt_off, ht_off, dzt_off, at_off, bt_off, cs_off, csb_off, k_off,
      total;
};

// Whether the direct path takes the backward: bf16, every K-outer contraction
// length (H for dH, the shard width for dX, the token split for dA and dB) a
// multiple of 64, and every K-outer operand's span within a 32-bit buffer
// range.  Lowers *splits until each token split is a multiple of 64.
bool bwd_direct_ok(const tp_mlp_bwd_desc* d, int64_t zs, int64_t Fz, int64_t Fc, int* splits) {
  if (d->dt != TP_BF16 || d->T % 64 || d->H % 64 || zs % 64) return false;
  int S = *splits;
  while (S > 1 && (d->T / S) % 64) S /= 2;
  const int64_t kc = d->T / S;
  const int64_t lim = (int64_t)0xFFFFFFFF - 1024;
  auto fits = [&](int64_t k, int64_t ld) { return (k - 1) * ld * 2 + 512 <= lim; };
  const int64_t wide = std::max(std::max(Fz, Fc), 2 * d->F);  // widest ld of dZ / act(Z) / a stored Z
  if (!fits(d->H, d->F) || !fits(zs, d->H) || !fits(kc, d->H) || !fits(kc, wide)) return false;
  *splits = S;
  return true;
}

// Weight gradients contract over all T tokens into a small [Fc x H] output
// when the hidden size is narrow.  Split the token axis so that the launch
// fills the chip: with 256x256 tiles (one per CU, the GEMM's choice once
// there are 256 of them) when splitting up to 16 ways gets there, else with
// 128x128 tiles at ~2 workgroups per CU.  Each split keeps K >= 512 and a
// multiple of 8.
int bwd_splits(int64_t T, int64_t Fc, int64_t H) {
  const int64_t big = ((Fc + 255) / 256) * ((H + 255) / 256);
  if (big >= 256) return 1;
  int s = 1;
  while (s < 16 && big * s < 256 && T / (2 * s) >= 512) s *= 2;
  if (big * s < 256) {
    const int64_t small = ((Fc + 127) / 128) * ((H + 127) / 128);
    s = 1;
    while (s < 16 && small * s < 512 && T / (2 * s) >= 512) s *= 2;
  }
  while (s > 1 && T % (8 * s)) s /= 2;
  return s;
}

// GELU with a short contraction (H <= 2048): the recomputed pre-activation
// and dZ come from one two-pass kernel that keeps the pre-activation on chip
// (its separate round trip through HBM dominates at narrow hidden sizes).
bool bwd_fused_gelu(const tp_mlp_bwd_desc* d) {
  return d->dt == TP_BF16 && d->act == TP_ACT_GELU && d->H <= 2048 && !d->Z;
}

tp_status validate_mlp_bwd(const tp_mlp_bwd_desc* d, BwdShape* sh) {
  if (!d) return fail(TP_ERR_NULL, "descriptor is NULL");
  TP_TRY(check_dtype(d->dt));
  if (d->act != TP_ACT_GELU && d->act != TP_ACT_NONE && d->act != TP_ACT_SWIGLU)
    return fail(TP_ERR_DTYPE, "backward activation %d unknown", (int)d->act);
  if (d->act == TP_ACT_SWIGLU && d->dt != TP_BF16) return fail(TP_ERR_DTYPE, "SwiGLU backward is bf16-only");
  if (d->act == TP_ACT_SWIGLU && (d->a || d->da))
    return fail(TP_ERR_SHAPE, "SwiGLU has no column bias: a and da must be NULL");
  if (d->T < 0 || d->H <= 0 || d->F <= 0 || d->N <= 0)
    return fail(TP_ERR_SHAPE, "T=%lld H=%lld F=%lld N=%d", (long long)d->T, (long long)d->H, (long long)d->F,
                d->N);
  if (d->F % d->N)
    return fail(TP_ERR_DIVISIBILITY,
                "intermediate F=%lld is not divisible by N=%d shards (shard would be %lld + %lld/%d columns)",
                (long long)d->F, d->N, (long long)(d->F / d->N), (long long)(d->F % d->N), d->N);
  if (d->shard_begin < 0 || d->shard_count < 1 || d->shard_begin + d->shard_count > d->N)
    return fail(TP_ERR_SHAPE, "shard range [%d, %d) outside [0, %d)", d->shard_begin,
                d->shard_begin + d->shard_count, d->N);
  const int64_t Fs = d->F / d->N, Fc = Fs * d->shard_count;
  const bool swiglu = d->act == TP_ACT_SWIGLU;
  *sh = BwdShape{};
  sh->Fs = Fs;
  sh->Fc = Fc;
  sh->Fz = swiglu ? 2 * Fc : Fc;
  sh->zld = sh->Fz;
  sh->splits = 1;
  TP_TRY(check_slices(d->T, d->n_slices, d->slice));
  if (d->T == 0) return TP_OK;  // empty input: nothing to read, write or stage
  if (d->T % 8) return fail(TP_ERR_ALIGN, "T=%lld is not a multiple of 8", (long long)d->T);
  if (d->H % 8) return fail(TP_ERR_ALIGN, "hidden H=%lld is not a multiple of 8", (long long)d->H);
  if (Fs % 8) return fail(TP_ERR_ALIGN, "shard width F/N=%lld is not a multiple of 8", (long long)Fs);
  const int64_t a_rows = swiglu ? 2 * d->F : d->F;
  const int64_t vec = vec_of(d->dt);
  TP_TRY(check_matrix("X", d->X, d->T, d->H, d->H, vec));
  TP_TRY(check_matrix("A", d->A, a_rows, d->H, d->H, vec));
  TP_TRY(check_matrix("B", d->B, d->H, d->F, d->F, vec));
  TP_TRY(check_matrix("dY", d->dY, d->T, d->H, d->H, vec));
  TP_TRY(check_matrix("dA", d->dA, a_rows, d->H, d->H, 4));
  TP_TRY(check_matrix("dB", d->dB, d->H, d->F, d->F, 4));
  if (d->a && !aligned16(d->a)) return fail(TP_ERR_ALIGN, "a is not 16-byte aligned");
  if (d->da && !aligned16(d->da)) return fail(TP_ERR_ALIGN, "da is not 16-byte aligned");
  if (d->db && !aligned16(d->db)) return fail(TP_ERR_ALIGN, "db is not 16-byte aligned");
  if (d->shard_count == d->N) {
    if (!d->dX) return fail(TP_ERR_NULL, "dX is NULL");
    if (!aligned16(d->dX)) return fail(TP_ERR_ALIGN, "dX is not 16-byte aligned");
  }
  if (d->Z) {
    const int64_t zw = swiglu ? 2 * d->F : d->F;  // SwiGLU: [gate | up] per shard
    TP_TRY(check_matrix("Z", d->Z, d->T, zw, zw, vec));
  }
  if (d->Hact) {
    if (d->act != TP_ACT_GELU || !d->Z)
      return fail(TP_ERR_SHAPE, "the stored activation Hact is read with GELU and a stored Z only");
    TP_TRY(check_matrix("Hact", d->Hact, d->T, d->F, d->F, vec));
  }
  if (d->T > kIntMax || d->F > kIntMax) return fail(TP_ERR_SHAPE, "size exceeds 2^31-1");
  const size_t T = (size_t)d->T, H = (size_t)d->H, fc = (size_t)Fc, fz = (size_t)sh->Fz, es = esize(d->dt);
  sh->splits = bwd_splits(d->T, sh->Fz, d->H);
  const int64_t zs = swiglu ? 2 * Fs : Fs;
  sh->direct = bwd_direct_ok(d, zs, sh->Fz, Fc, &sh->splits);
  const bool fused = bwd_fused_gelu(d);
  const bool tr = !sh->direct;  // transposed operands in the workspace
  sh->p_bytes = align256((size_t)d->N * T * H * sizeof(float));
  sh->z_off = sh->p_bytes;
  sh->dz_off = sh->z_off + (d->Z ? 0 : align256(T * fz * es));  // no recomputed Z with a stored one
  sh->h_off = sh->dz_off + align256(T * fz * es);
  const bool hs = swiglu || fused || (sh->direct && d->act == TP_ACT_GELU);
  sh->xt_off = sh->h_off + (hs ? align256(T * fc * es) : 0);
  sh->dyt_off = sh->xt_off + (tr ? align256(H * T * es) : 0);
  sh->ht_off = sh->dyt_off + (tr ? align256(H * T * es) : 0);
  sh->dzt_off = sh->ht_off + (tr ? align256(fc * T * es) : 0);
  sh->at_off = sh->dzt_off + (tr ? align256(fz * T * es) : 0);
  sh->bt_off = sh->at_off + (tr ? align256(H * fz * es) : 0);
  sh->cs_off = sh->bt_off + (tr || fused ? align256(fc * H * es) : 0);
  sh->csb_off = sh->cs_off + (sh->direct ? align256(tp::colsum_part_floats(d->T, Fc) * sizeof(float)) : 0);
  sh->k_off = sh->csb_off + (sh->direct ? align256(tp::colsum_part_floats(d->T, d->H) * sizeof(float)) : 0);
  sh->total = sh->k_off + (sh->splits > 1 ? align256((size_t)sh->splits * fz * H * sizeof(float)) : 0);
  return TP_OK;
}

// The backward after dZ (and its transpose) exist: the input-gradient
// partials, the weight and bias gradients, and the fold of the partials.
template <class TokenGemm, class RowSum>
tp_status bwd_tail(hipStream_t s, const tp_mlp_bwd_desc* d, const BwdShape& sh, void* ws, const void* dZ,
                   const void* dZT, const void* XT, const void* dYT, const void* HT, const void* AT,
                   TokenGemm& token_gemm, RowSum& rowsum) {
  const int64_t T = d->T, H = d->H, F = d->F, Fs = sh.Fs, Fc = sh.Fc, Fz = sh.Fz;
  const int c = d->shard_count, i0 = d->shard_begin;
  const int64_t zs = d->act == TP_ACT_SWIGLU ? 2 * Fs : Fs;
  float* P = static_cast<float*>(ws);
  // dX partial of each shard into its slab slot: dZ_i A_i (K = zs)
  const tp::GemmParams xg = gemm(dZ, sh.zld, zs, AT, Fz, zs, P + (size_t)i0 * T * H, H, T * H, T, H, zs, c);
  TP_TRY(hip_status(launch("bwd_dx_gemm", d->dt, xg, tp::EPI_PARTIAL, s), "bwd_dx_gemm"));
  // dA rows of the range: dZ^T X  (M = Fz, N = H, contraction over T)
  TP_TRY(token_gemm("bwd_da_gemm", dZT, XT, Fz, H, d->dA + (size_t)i0 * zs * H, H));
  // dB columns of the range: dY^T act(Z)  (M = H, N = Fc)
  TP_TRY(token_gemm("bwd_db_gemm", dYT, HT, H, Fc, d->dB + (size_t)i0 * Fs, F));
  // bias gradients: column sums of dZ (range) and of dY (once)
  if (d->da) TP_TRY(rowsum("bwd_bias_rowsum", dZT, T, d->da + (size_t)i0 * Fs, Fc, T));
  if (d->db) TP_TRY(rowsum("bwd_bias_rowsum", dYT, T, d->db, H, T));

  if (c < d->N) return ok();
  return run_reduce(s, d->dt, d->N, T, H, P, T * H, nullptr, d->dX, d->n_slices, d->slice);
}

// The backward on the direct path: every operand read as stored.  dH = dY B_r
// takes the range's columns of B K-outer ([H x Fc], ld F); dX_i = dZ_i A_i the
// shard's rows of A K-outer ([zs x H]); dA = dZ^T X and dB = dY^T act(Z) take
// both operands K-outer over the token axis.  The bias gradients are column
// sums of dZ and dY.
tp_status bwd_direct(hipStream_t s, const tp_mlp_bwd_desc* d, const BwdShape& sh, char* base) {
  const int64_t T = d->T, H = d->H, F = d->F, Fs = sh.Fs, Fc = sh.Fc, Fz = sh.Fz;
  const int c = d->shard_count, i0 = d->shard_begin, S = sh.splits;
  const bool gelu = d->act == TP_ACT_GELU, swiglu = d->act == TP_ACT_SWIGLU;
  const int64_t zs = swiglu ? 2 * Fs : Fs;
  const size_t es = 2;
  char* Z = base + sh.z_off;
  char* dZ = base + sh.dz_off;
  char* Hs = base + sh.h_off;
  char* BT = base + sh.bt_off;
  float* CSa = reinterpret_cast<float*>(base + sh.cs_off);
  float* CSb = reinterpret_cast<float*>(base + sh.csb_off);
  float* K = reinterpret_cast<float*>(base + sh.k_off);
  float* P = reinterpret_cast<float*>(base);
  const char* A_r = static_cast<const char*>(d->A) + (size_t)i0 * zs * H * es;  // range rows of A
  const char* B_r = static_cast<const char*>(d->B) + (size_t)i0 * Fs * es;      // range columns of B
  const char* a_r = d->a ? static_cast<const char*>(d->a) + (size_t)i0 * Fs * es : nullptr;

  // act(Z), the B operand of dB: [T x Fc] at pitch hld
  const void* Hop = Hs;
  int64_t hld = Fc;
  if (bwd_fused_gelu(d)) {
    // the two-pass kernel reads its second operand K-contiguous: B_r^T once
    tp::TransposeParams t{B_r, F, BT, H, H, Fc};
    KernelTimer kt("bwd_transpose", s);
    const hipError_t e = tp::launch_transpose(t, false, false, s);
    kt.stop();
    TP_TRY(hip_status(e, "bwd_transpose"));
    tp::GemmParams fg = gemm(d->X, H, 0, A_r, H, 0, dZ, sh.zld, 0, T, Fc, H, 1);
    fg.bias = a_r;
    fg.A2 = d->dY;
    fg.B2 = BT;
    fg.C2 = Hs;
    fg.ldc2 = Fc;
    TP_TRY(hip_status(launch("bwd_fused_gemm", TP_BF16, fg, tp::EPI_GELU_FUSED, s), "bwd_fused_gemm"));
  } else {
    // Z = X A_r^T (+ a_r): the forward's stored one, or recomputed
    const void* Zp = Z;
    int64_t zld = sh.zld;
    if (d->Z) {
      Zp = static_cast<const char*>(d->Z) + (size_t)i0 * zs * es;  // SwiGLU: [gate | up] blocks
      zld = swiglu ? 2 * F : F;
    } else {
      tp::GemmParams zg = gemm(d->X, H, 0, A_r, H, 0, Z, sh.zld, 0, T, Fz, H, 1);
      zg.bias = a_r;
      TP_TRY(hip_status(launch("bwd_recompute_gemm", TP_BF16, zg, tp::EPI_STORE, s), "bwd_recompute_gemm"));
    }
    if (swiglu) {
      // per shard: dH = dY B_i; [dG | dU] and SiLU(G) U from the stored [G | U]
      tp::GemmParams dg = gemm(d->dY, H, 0, B_r, F, Fs, dZ, sh.zld, zs, T, Fs, H, c);
      dg.b_ko = 1;
      dg.aux = Zp;
      dg.ldaux = zld;
      dg.sAux = zs;
      dg.upOff = Fs;
      dg.C2 = Hs;
      dg.ldc2 = Fc;
      dg.sC2 = Fs;
      TP_TRY(hip_status(launch("bwd_dz_gemm", TP_BF16, dg, tp::EPI_SWIGLU_BWD, s), "bwd_dz_gemm"));
    } else {
      // dZ = (dY B_r) * act'(Z); GELU(Z) written beside it for dB
      tp::GemmParams dg = gemm(d->dY, H, 0, B_r, F, 0, dZ, sh.zld, 0, T, Fc, H, 1);
      dg.b_ko = 1;
      dg.aux = Zp;
      dg.ldaux = zld;
      if (gelu && d->Hact) {  // the forward's activation: dZ alone
        Hop = static_cast<const char*>(d->Hact) + (size_t)i0 * Fs * es;
        hld = F;
      } else if (gelu) {
        dg.C2 = Hs;
        dg.ldc2 = Fc;
      } else {
        Hop = Zp;
        hld = zld;
      }
      TP_TRY(hip_status(launch("bwd_dz_gemm", TP_BF16, dg, gelu ? tp::EPI_GELU_BWD : tp::EPI_STORE, s),
                        "bwd_dz_gemm"));
    }
  }
  // dX partial of each shard into its slab slot: dZ_i A_i (K = zs), A_i K-outer
  tp::GemmParams xg = gemm(dZ, sh.zld, zs, A_r, H, zs * H, P + (size_t)i0 * T * H, H, T * H, T, H, zs, c);
  xg.b_ko = 1;
  TP_TRY(hip_status(launch("bwd_dx_gemm", TP_BF16, xg, tp::EPI_PARTIAL, s), "bwd_dx_gemm"));

  // C[M x N] = Aop^T Bop over the token axis, both [T x .] K-outer; split-K
  // when the output is small, the splits' partials folded in split order
  auto token_gemm = [&](const char* name, const void* Aop, int64_t lda, const void* Bop, int64_t ldb, int64_t M,
                        int64_t N, float* C, int64_t ldc) -> tp_status {
    if (S == 1) {
      tp::GemmParams g = gemm(Aop, lda, 0, Bop, ldb, 0, C, ldc, 0, M, N, T, 1);
      g.a_ko = g.b_ko = 1;
      return hip_status(launch(name, TP_BF16, g, tp::EPI_PARTIAL, s), name);
    }
    const int64_t kc = T / S;
    tp::GemmParams g = gemm(Aop, lda, kc * lda, Bop, ldb, kc * ldb, K, N, M * N, M, N, kc, S);
    g.a_ko = g.b_ko = 1;
    g.xcd_per_problem = S % 8 == 0;  // each split's operand blocks stay in one XCD's L2
    TP_TRY(hip_status(launch(name, TP_BF16, g, tp::EPI_PARTIAL, s), name));
    tp::ReduceParams r{};
    r.P = K;
    r.part_stride = M * N;
    r.n_parts = S;
    r.rows = M;
    r.H = N;
    r.row0 = 0;
    r.bias = nullptr;
    r.Y = C;
    r.ldy = ldc;
    KernelTimer kt("bwd_splitk_reduce", s);
    const hipError_t e = tp::launch_reduce(r, false, s);
    kt.stop();
    return hip_status(e, "bwd_splitk_reduce");
  };
  // dA rows of the range: dZ^T X  (M = Fz, N = H)
  TP_TRY(token_gemm("bwd_da_gemm", dZ, sh.zld, d->X, H, Fz, H, d->dA + (size_t)i0 * zs * H, H));
  // dB columns of the range: dY^T act(Z)  (M = H, N = Fc)
  TP_TRY(token_gemm("bwd_db_gemm", d->dY, H, Hop, hld, H, Fc, d->dB + (size_t)i0 * Fs, F));
  // bias gradients: column sums of dZ (range) and of dY (once), both in the
  // same two launches
  tp::ColSumParams cps[2];
  int ncs = 0;
  if (d->da) cps[ncs++] = tp::ColSumParams{dZ, sh.zld, T, Fc, CSa, d->da + (size_t)i0 * Fs};
  if (d->db) cps[ncs++] = tp::ColSumParams{d->dY, H, T, H, CSb, d->db};
  if (ncs > 0) {
    KernelTimer kt("bwd_bias_colsum", s);
    hipError_t e = tp::launch_colsum_chunks(cps, ncs, s);
    kt.stop();
    TP_TRY(hip_status(e, "bwd_bias_colsum"));
    KernelTimer kf("bwd_bias_colsum_fold", s);
    e = tp::launch_colsum_fold(cps, ncs, s);
    kf.stop();
    TP_TRY(hip_status(e, "bwd_bias_colsum_fold"));
  }

  if (c < d->N) return ok();
  return run_reduce(s, TP_BF16, d->N, T, H, P, T * H, nullptr, d->dX, d->n_slices, d->slice);
}

// ------------------------------------------------------- vocab-parallel CE
// Workspace: the per-(token, 64-column chunk) statistics of the shard range
// written by the logits GEMM's epilogue -- three arrays (max, sum, label
// logit) of shard_count*cps*T floats each -- then the per-shard statistics
// m, s, z, each N x [T] fp32 (slot i = shard i).
struct VocabShape {
  int64_t Vp, Vs;
  int cps;  // 64-column chunks per shard
  size_t chunk_bytes, m_off, s_off, z_off, total;
};

int64_t vocab_shard_width(int64_t V, int N) {
  const int64_t vs = (V + N - 1) / N;
  return (vs + 7) / 8 * 8;
}

tp_status validate_vocab(const tp_vocab_ce_desc* d, VocabShape* sh) {
  if (!d) return fail(TP_ERR_NULL, "descriptor is NULL");
  TP_TRY(check_dtype(d->dt));
  if (d->dt != TP_BF16) return fail(TP_ERR_DTYPE, "vocab-parallel cross-entropy is bf16-only");
  if (d->T < 0 || d->H <= 0 || d->V <= 0 || d->N <= 0)
    return fail(TP_ERR_SHAPE, "T=%lld H=%lld V=%lld N=%d", (long long)d->T, (long long)d->H, (long long)d->V, d->N);
  if (d->shard_begin < 0 || d->shard_count < 1 || d->shard_begin + d->shard_count > d->N)
    return fail(TP_ERR_SHAPE, "shard range [%d, %d) outside [0, %d)", d->shard_begin,
                d->shard_begin + d->shard_count, d->N);
  *sh = VocabShape{};
  sh->Vs = vocab_shard_width(d->V, d->N);
  sh->Vp = sh->Vs * d->N;
  if (d->T == 0) return TP_OK;  // empty input: nothing to read or write
  if (d->H % 8) return fail(TP_ERR_ALIGN, "hidden H=%lld is not a multiple of 8", (long long)d->H);
  TP_TRY(check_matrix("X", d->X, d->T, d->H, d->H, 8));
  TP_TRY(check_matrix("E", d->E, sh->Vp, d->H, d->H, 8));
  if (!d->labels) return fail(TP_ERR_NULL, "labels is NULL");
  if (!aligned4(d->labels)) return fail(TP_ERR_ALIGN, "labels is not 4-byte aligned");
  if (d->shard_count == d->N) {
    if (!d->loss) return fail(TP_ERR_NULL, "loss is NULL");
    if (!aligned16(d->loss)) return fail(TP_ERR_ALIGN, "loss is not 16-byte aligned");
  }
  if (d->mean_loss && (reinterpret_cast<uintptr_t>(d->mean_loss) & 3u))
    return fail(TP_ERR_ALIGN, "mean_loss is not 4-byte aligned");
  if (d->T > kIntMax || sh->Vs > kIntMax) return fail(TP_ERR_SHAPE, "size exceeds 2^31-1");
  const size_t T = (size_t)d->T;
  sh->cps = (int)((sh->Vs + 63) / 64);
  sh->chunk_bytes = align256(3 * (size_t)d->shard_count * sh->cps * T * sizeof(float));
  sh->m_off = sh->chunk_bytes;
  sh->s_off = sh->m_off + align256((size_t)d->N * T * sizeof(float));
  sh->z_off = sh->s_off + align256((size_t)d->N * T * sizeof(float));
  sh->total = sh->z_off + align256((size_t)d->N * T * sizeof(float));
  return TP_OK;
}

tp_status validate_embed(const tp_vocab_embed_desc* d, size_t* need) {
  if (!d) return fail(TP_ERR_NULL, "descriptor is NULL");
  TP_TRY(check_dtype(d->dt));
  if (d->T < 0 || d->H <= 0 || d->V <= 0 || d->N <= 0)
    return fail(TP_ERR_SHAPE, "T=%lld H=%lld V=%lld N=%d", (long long)d->T, (long long)d->H, (long long)d->V, d->N);
  if (d->shard_begin < 0 || d->shard_count < 1 || d->shard_begin + d->shard_count > d->N)
    return fail(TP_ERR_SHAPE, "shard range [%d, %d) outside [0, %d)", d->shard_begin,
                d->shard_begin + d->shard_count, d->N);
  *need = 0;
  if (d->T == 0) return TP_OK;
  if (d->H % 8) return fail(TP_ERR_ALIGN, "hidden H=%lld is not a multiple of 8", (long long)d->H);
  const int64_t vec = vec_of(d->dt);
  TP_TRY(check_matrix("E", d->E, vocab_shard_width(d->V, d->N) * d->N, d->H, d->H, vec));
  if (!d->ids) return fail(TP_ERR_NULL, "ids is NULL");
  if (!aligned4(d->ids)) return fail(TP_ERR_ALIGN, "ids is not 4-byte aligned");
  if (d->shard_count == d->N) TP_TRY(check_matrix("Y", d->Y, d->T, d->H, d->H, vec));
  if (d->T > kIntMax) return fail(TP_ERR_SHAPE, "T exceeds 2^31-1");
  *need = align256((size_t)d->N * d->T * d->H * (d->dt == TP_F32 ? 4 : 2));
  return TP_OK;
}

tp_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return fail(TP_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned16(ws)) return fail(TP_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (ws_bytes < need) return fail(TP_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  return TP_OK;
}

}  // namespace

namespace tp {
LaunchEvents take_launch_events() {
  const LaunchEvents e = t_armed;
  t_armed = {nullptr, nullptr};
  return e;
}
}  // namespace tp

extern "C" {

tp_status tp_column_linear(void* stream, tp_dtype dt, tp_act act, int64_t T, int64_t K, int64_t Ns,
                           const void* X, int64_t ldx, const void* W_i, int64_t ldw, const void* bias_i,
                           void* Y_i, int64_t ldy) {
  TP_TRY(check_dtype(dt));
  if (act != TP_ACT_NONE && act != TP_ACT_GELU && act != TP_ACT_SWIGLU)
    return fail(TP_ERR_DTYPE, "activation %d unknown", (int)act);
  if (act == TP_ACT_SWIGLU && dt != TP_BF16) return fail(TP_ERR_DTYPE, "SwiGLU path is bf16-only");
  if (act == TP_ACT_SWIGLU && bias_i) return fail(TP_ERR_SHAPE, "SwiGLU bias must be NULL");
  if (T < 0 || K <= 0 || Ns <= 0)
    return fail(TP_ERR_SHAPE, "T=%lld K=%lld Ns=%lld", (long long)T, (long long)K, (long long)Ns);
  const int64_t vec = vec_of(dt);
  if (K % vec) return fail(TP_ERR_ALIGN, "K=%lld is not a multiple of %lld", (long long)K, (long long)vec);
  if (T == 0) return ok();  // empty input: nothing to read or write
  TP_TRY(check_matrix("X", X, T, K, ldx, vec));
  TP_TRY(check_matrix("W_i", W_i, act == TP_ACT_SWIGLU ? 2 * Ns : Ns, K, ldw, vec));
  if (!Y_i) return fail(TP_ERR_NULL, "Y_i is NULL");
  if (ldy < Ns) return fail(TP_ERR_SHAPE, "ldy %lld < Ns %lld", (long long)ldy, (long long)Ns);
  if (!aligned16(Y_i)) return fail(TP_ERR_ALIGN, "Y_i is not 16-byte aligned");
  if (ldy % vec) return fail(TP_ERR_ALIGN, "ldy %lld is not a multiple of %lld", (long long)ldy, (long long)vec);
  if (T > kIntMax || (act == TP_ACT_SWIGLU ? 2 * Ns : Ns) > kIntMax) return fail(TP_ERR_SHAPE, "size exceeds 2^31-1");
  if (T == 0) return ok();
  tp::GemmParams p = gemm(X, ldx, 0, W_i, ldw, 0, Y_i, ldy, 0, T, Ns, K, 1);
  p.bias = bias_i;
  p.upOff = Ns * ldw;
  const tp::Epilogue e = act == TP_ACT_GELU ? tp::EPI_GELU : act == TP_ACT_SWIGLU ? tp::EPI_SWIGLU : tp::EPI_STORE;
  return hip_status(launch("column_linear", dt, p, e, static_cast<hipStream_t>(stream)), "column_linear launch");
}

tp_status tp_row_linear_partial(void* stream, tp_dtype dt, int64_t T, int64_t Ks, int64_t Nout, const void* X_i,
                                int64_t ldx, const void* W_i, int64_t ldw, float* P_i, int64_t ldp) {
  TP_TRY(check_dtype(dt));
  if (T < 0 || Ks <= 0 || Nout <= 0)
    return fail(TP_ERR_SHAPE, "T=%lld Ks=%lld Nout=%lld", (long long)T, (long long)Ks, (long long)Nout);
  const int64_t vec = vec_of(dt);
  if (Ks % vec) return fail(TP_ERR_ALIGN, "Ks=%lld is not a multiple of %lld", (long long)Ks, (long long)vec);
  if (T == 0) return ok();  // empty input: nothing to read or write
  TP_TRY(check_matrix("X_i", X_i, T, Ks, ldx, vec));
  TP_TRY(check_matrix("W_i", W_i, Nout, Ks, ldw, vec));
  if (!P_i) return fail(TP_ERR_NULL, "P_i is NULL");
  if (ldp < Nout) return fail(TP_ERR_SHAPE, "ldp %lld < Nout %lld", (long long)ldp, (long long)Nout);
  if (!aligned16(P_i)) return fail(TP_ERR_ALIGN, "P_i is not 16-byte aligned");
  if (ldp % 4) return fail(TP_ERR_ALIGN, "ldp %lld is not a multiple of 4", (long long)ldp);
  if (T > kIntMax) return fail(TP_ERR_SHAPE, "T exceeds 2^31-1");
  if (T == 0) return ok();
  const tp::GemmParams p = gemm(X_i, ldx, 0, W_i, ldw, 0, P_i, ldp, 0, T, Nout, Ks, 1);
  return hip_status(launch("row_linear_partial", dt, p, tp::EPI_PARTIAL, static_cast<hipStream_t>(stream)), "row_linear_partial launch");
}

tp_status tp_reduce_partials(void* stream, tp_dtype out_dt, int n_parts, int64_t T, int64_t H, const float* P,
                             int64_t part_stride, const void* bias, void* Y, int n_slices, int slice) {
  TP_TRY(validate_reduce(out_dt, n_parts, T, H, P, part_stride, bias, Y, n_slices, slice));
  if (T == 0) return ok();
  return run_reduce(static_cast<hipStream_t>(stream), out_dt, n_parts, T, H, P, part_stride, bias, Y, n_slices,
                    slice);
}

tp_status tp_rmsnorm_gather(void* stream, tp_dtype dt, int n_slices, int64_t T, int64_t H, const void* X,
                            int64_t slice_stride, int64_t ldx, const void* gamma, float eps, void* Y, int64_t ldy,
                            int slice) {
  TP_TRY(validate_norm(dt, n_slices, T, H, X, slice_stride, ldx, gamma, eps, Y, ldy, slice));
  if (T == 0) return ok();
  const hipStream_t s = static_cast<hipStream_t>(stream);
  tp::NormParams p{};
  p.X = X;
  p.slice_stride = slice_stride;
  p.ldx = ldx;
  p.gamma = gamma;
  p.Y = Y;
  p.ldy = ldy;
  p.slice_rows = T / n_slices;
  p.rows = slice < 0 ? T : p.slice_rows;
  p.slice = slice;
  p.H = (int)H;
  p.inv_h = 1.0f / (float)H;
  p.eps = eps;
  if (log_enabled())
    fprintf(stderr, "[tp] rmsnorm_gather %s: %d slices of [%lld x %lld] -> Y[%lld x %lld]%s\n", dt_name(dt), n_slices,
            (long long)p.slice_rows, (long long)H, (long long)T, (long long)H, slice >= 0 ? " (one slice)" : "");
  KernelTimer kt("rmsnorm_gather", s);
  const hipError_t e = tp::launch_rmsnorm_gather(p, dt == TP_BF16, s);
  kt.stop();
  TP_TRY(hip_status(e, "rmsnorm_gather launch"));
  return ok();
}

tp_status tp_layernorm_gather(void* stream, tp_dtype dt, int n_slices, int64_t T, int64_t H, const void* X,
                              int64_t slice_stride, int64_t ldx, const void* gamma, const void* beta, float eps,
                              void* Y, int64_t ldy, int slice) {
  TP_TRY(validate_norm(dt, n_slices, T, H, X, slice_stride, ldx, gamma, eps, Y, ldy, slice));
  if (beta && !aligned16(beta)) return fail(TP_ERR_ALIGN, "beta is not 16-byte aligned");
  if (T == 0) return ok();
  const hipStream_t s = static_cast<hipStream_t>(stream);
  tp::NormParams p{};
  p.X = X;
  p.slice_stride = slice_stride;
  p.ldx = ldx;
  p.gamma = gamma;
  p.beta = beta;
  p.layer = 1;
  p.Y = Y;
  p.ldy = ldy;
  p.slice_rows = T / n_slices;
  p.rows = slice < 0 ? T : p.slice_rows;
  p.slice = slice;
  p.H = (int)H;
  p.inv_h = 1.0f / (float)H;
  p.eps = eps;
  if (log_enabled())
    fprintf(stderr, "[tp] layernorm_gather %s: %d slices of [%lld x %lld] -> Y[%lld x %lld]%s\n", dt_name(dt),
            n_slices, (long long)p.slice_rows, (long long)H, (long long)T, (long long)H,
            slice >= 0 ? " (one slice)" : "");
  KernelTimer kt("layernorm_gather", s);
  const hipError_t e = tp::launch_rmsnorm_gather(p, dt == TP_BF16, s);
  kt.stop();
  TP_TRY(hip_status(e, "layernorm_gather launch"));
  return ok();
}

size_t tp_norm_split_workspace_size(const tp_norm_split_desc* d) {
  size_t need = 0;
  return validate_norm_split(d, &need) == TP_OK ? need : 0;
}

tp_status tp_norm_hidden_split(void* stream, const tp_norm_split_desc* d, void* ws, size_t ws_bytes) {
  size_t need = 0;
  TP_TRY(validate_norm_split(d, &need));
  if (d->T == 0) return ok();
  TP_TRY(check_ws(ws, ws_bytes, need));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  tp::NormSplitParams p{};
  p.X = d->X;
  p.ldx = d->ldx;
  p.gamma = d->gamma;
  p.beta = d->beta;
  p.Y = d->Y;
  p.ldy = d->ldy;
  p.stats = static_cast<float*>(ws);
  p.T = d->T;
  p.Hs = (int)(d->H / d->N);
  p.N = d->N;
  p.shard0 = d->shard_begin;
  p.shards = d->shard_count;
  p.inv_hs = 1.0f / (float)p.Hs;
  p.inv_h = 1.0f / (float)d->H;
  p.eps = d->eps;
  p.layer = d->kind == TP_NORM_LAYER;
  if (log_enabled())
    fprintf(stderr, "[tp] norm_hidden_split %s %s: T=%lld H=%lld N=%d shards [%d,%d)\n", dt_name(d->dt),
            p.layer ? "layernorm" : "rmsnorm", (long long)d->T, (long long)d->H, d->N, d->shard_begin,
            d->shard_begin + d->shard_count);
  const bool bf = d->dt == TP_BF16;
  {
    KernelTimer kt("norm_split_stats", s);
    const hipError_t e = tp::launch_norm_split_stats(p, bf, s);
    kt.stop();
    TP_TRY(hip_status(e, "norm_split_stats launch"));
  }
  KernelTimer kt("norm_split_apply", s);
  const hipError_t e = tp::launch_norm_split_apply(p, bf, s);
  kt.stop();
  TP_TRY(hip_status(e, "norm_split_apply launch"));
  return ok();
}

size_t tp_mlp_workspace_size(const tp_mlp_desc* d) {
  MlpShape sh;
  return validate_mlp(d, &sh) == TP_OK ? sh.total : 0;
}

size_t tp_mlp_partials_offset(const tp_mlp_desc* d) {
  (void)d;
  return 0;
}

size_t tp_attn_workspace_size(const tp_attn_desc* d) {
  AttnShape sh;
  return validate_attn(d, &sh) == TP_OK ? sh.total : 0;
}

size_t tp_attn_partials_offset(const tp_attn_desc* d) {
  (void)d;
  return 0;
}

}  // extern "C"

namespace {

// The shard products of token rows [row0, row0 + rows) for every shard in the
// descriptor's range: their partial rows land at the same rows of each
// shard's slab slot (and of the intermediate), so row blocks computed in any
// order fill the slab exactly as one call over all rows does.
tp_status mlp_rows(hipStream_t s, const tp_mlp_desc* d, const MlpShape& sh, void* ws, int64_t row0, int64_t rows) {
  const int64_t T = d->T, H = d->H, Fs = sh.Fs;
  const int c = d->shard_count, i0 = d->shard_begin;
  char* base = static_cast<char*>(ws);
  float* P = reinterpret_cast<float*>(base) + (size_t)row0 * H;
  const size_t es = esize(d->dt);
  void* Hs = base + sh.h_offset + (size_t)row0 * sh.h_ld * es;
  const void* X = static_cast<const char*>(d->X) + (size_t)row0 * H * es;

  // Narrow hidden sizes: one kernel per shard range computes the column
  // product, the activation and the row partial with the intermediate kept
  // on chip (it never needs to leave the shard).
  if (d->dt == TP_BF16 && d->act != TP_ACT_SWIGLU && !d->Z && !d->Hact && tp::mlp_fused_supported(H, Fs)) {
    tp::FusedMlpParams f{};
    f.X = X;
    f.ldx = H;
    f.A = static_cast<const char*>(d->A) + (size_t)i0 * Fs * H * es;
    f.lda = H;
    f.sA = Fs * H;
    f.bias = d->a ? static_cast<const char*>(d->a) + (size_t)i0 * Fs * es : nullptr;
    f.sBias = Fs;
    f.B = static_cast<const char*>(d->B) + (size_t)i0 * Fs * es;
    f.ldb = d->F;
    f.sB = Fs;
    f.P = P + (size_t)i0 * T * H;
    f.ldp = H;
    f.sP = T * H;
    f.T = (int)rows;
    f.H = (int)H;
    f.Fs = (int)Fs;
    f.shards = c;
    f.act = d->act == TP_ACT_GELU ? tp::FUSED_GELU : tp::FUSED_NONE;
    KernelTimer kt("mlp_fused", s);
    const hipError_t e = tp::launch_mlp_fused(f, s);
    kt.stop();
    return hip_status(e, "mlp fused launch");
  }

  // The stored pre-activation's rows of this block, the range's columns:
  // without an activation it is the intermediate itself (written there, read
  // from there), with GELU a second output of the column GEMM.
  const bool swiglu = d->act == TP_ACT_SWIGLU;
  const int64_t zw = swiglu ? 2 * d->F : d->F, zs = swiglu ? 2 * Fs : Fs;  // Z row width, shard block width
  void* Zr = d->Z ? static_cast<char*>(d->Z) + ((size_t)row0 * zw + (size_t)i0 * zs) * es : nullptr;
  // the intermediate: the stored Z itself without an activation, the
  // caller's Hact when given (row block, range columns), else the workspace
  void* Ha = d->Hact ? static_cast<char*>(d->Hact) + ((size_t)row0 * d->F + (size_t)i0 * Fs) * es : nullptr;
  const bool z_is_h = Zr && d->act == TP_ACT_NONE;
  void* Hc = z_is_h ? Zr : Ha ? Ha : Hs;
  const bool h_in_f = z_is_h || Ha;  // [T x F] layout, shard i at columns i*Fs
  const int64_t hld = h_in_f ? d->F : sh.h_ld, hstride = h_in_f ? Fs : T * sh.h_ld;

  // column GEMM + activation for every shard in range (X shared, one launch)
  tp::GemmParams col = gemm(X, H, 0, static_cast<const char*>(d->A) + (size_t)i0 * sh.a_rows * H * es, H,
                            sh.a_rows * H, Hc, hld, hstride, rows, Fs, H, c);
  if (d->a) {
    col.bias = static_cast<const char*>(d->a) + (size_t)i0 * Fs * es;
    col.sBias = Fs;
  }
  col.upOff = Fs * H;
  tp::Epilogue ce = d->act == TP_ACT_SWIGLU ? tp::EPI_SWIGLU : d->act == TP_ACT_GELU ? tp::EPI_GELU : tp::EPI_STORE;
  if (Zr && d->act != TP_ACT_NONE) {  // GELU or SwiGLU: the pre-activation is a second output
    ce = swiglu ? tp::EPI_SWIGLU_Z : tp::EPI_GELU_Z;
    col.C2 = Zr;
    col.ldc2 = zw;
    col.sC2 = zs;
  }
  TP_TRY(hip_status(launch("mlp_column_gemm", d->dt, col, ce, s), "mlp column launch"));

  // row partial of every shard into its slot of the fp32 slab
  const tp::GemmParams row = gemm(Hc, hld, hstride, static_cast<const char*>(d->B) + (size_t)i0 * Fs * es, d->F,
                                  Fs, P + (size_t)i0 * T * H, H, T * H, rows, H, Fs, c);
  return hip_status(launch("mlp_row_gemm", d->dt, row, tp::EPI_PARTIAL, s), "mlp row launch");
}

// Events that order the overlapped forward's two streams, reused call to call
// by the calling thread (a wait takes the event's state at the time it is
// enqueued, so re-recording later is safe); each thread has its own, so calls
// from different threads never share an event.
thread_local std::vector<hipEvent_t> t_overlap_events;

tp_status overlap_events(int n, hipEvent_t* out) {
  while ((int)t_overlap_events.size() < n) {
    hipEvent_t e = nullptr;
    const hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
    if (r != hipSuccess) return hip_status(r, "overlap event create");
    t_overlap_events.push_back(e);
  }
  for (int i = 0; i < n; ++i) out[i] = t_overlap_events[i];
  return TP_OK;
}

}  // namespace

extern "C" {

tp_status tp_mlp_forward(void* stream, const tp_mlp_desc* d, void* ws, size_t ws_bytes) {
  MlpShape sh;
  TP_TRY(validate_mlp(d, &sh));
  if (d->T == 0) return ok();
  TP_TRY(check_ws(ws, ws_bytes, sh.total));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t T = d->T, H = d->H, Fs = sh.Fs;
  const int c = d->shard_count, i0 = d->shard_begin;
  if (log_enabled())
    fprintf(stderr,
            "[tp] mlp %s act=%d N=%d shards [%d,%d): X[%lld x %lld] A_i[%lld x %lld] -> H_i[%lld x %lld] ; "
            "B_i[%lld x %lld] -> P_i[%lld x %lld] fp32%s\n",
            dt_name(d->dt), (int)d->act, d->N, i0, i0 + c, (long long)T, (long long)H, (long long)sh.a_rows,
            (long long)H, (long long)T, (long long)Fs, (long long)H, (long long)Fs, (long long)T, (long long)H,
            c == d->N ? " ; reduce" : "");
  TP_TRY(mlp_rows(s, d, sh, ws, 0, T));
  if (c < d->N) return ok();
  return run_reduce(s, d->dt, d->N, T, H, reinterpret_cast<float*>(ws), T * H, d->b, d->Y, d->n_slices, d->slice);
}

tp_status tp_mlp_forward_overlap(void* stream, void* stream2, const tp_mlp_desc* d, int chunks, void* ws,
                                 size_t ws_bytes) {
  MlpShape sh;
  TP_TRY(validate_mlp(d, &sh));
  if (d->shard_count != d->N) return fail(TP_ERR_SHAPE, "the overlapped forward needs the whole shard range");
  if (d->slice != -1) return fail(TP_ERR_SHAPE, "the overlapped forward writes every row (slice must be -1)");
  if (chunks < 1 || chunks > kMaxOverlapChunks)
    return fail(TP_ERR_SHAPE, "chunks=%d outside [1, %d]", chunks, kMaxOverlapChunks);
  if (d->T % chunks)
    return fail(TP_ERR_DIVISIBILITY, "T=%lld tokens do not split into %d chunks", (long long)d->T, chunks);
  if (d->T == 0) return ok();
  if (stream2 == stream) return fail(TP_ERR_SHAPE, "stream2 must differ from stream");
  TP_TRY(check_ws(ws, ws_bytes, sh.total));
  const hipStream_t s = static_cast<hipStream_t>(stream), s2 = static_cast<hipStream_t>(stream2);
  hipEvent_t ev[kMaxOverlapChunks + 1];
  TP_TRY(overlap_events(chunks + 1, ev));
  const int64_t T = d->T, H = d->H, rows = T / chunks;
  const size_t es = esize(d->dt);
  for (int k = 0; k < chunks; ++k) {
    TP_TRY(mlp_rows(s, d, sh, ws, k * rows, rows));
    TP_TRY(hip_status(hipEventRecord(ev[k], s), "overlap event record"));
    TP_TRY(hip_status(hipStreamWaitEvent(s2, ev[k], 0), "overlap stream wait"));
    // rows of block k of the fold, as slice k of `chunks` slices
    void* Yk = static_cast<char*>(d->Y) + (size_t)k * rows * H * es;
    TP_TRY(run_reduce(s2, d->dt, d->N, T, H, reinterpret_cast<float*>(ws), T * H, d->b, Yk, chunks, k));
  }
  TP_TRY(hip_status(hipEventRecord(ev[chunks], s2), "overlap event record"));
  TP_TRY(hip_status(hipStreamWaitEvent(s, ev[chunks], 0), "overlap stream wait"));
  return ok();
}

}  // extern "C"

namespace {

// Workspace of tp_mlp_forward_noalloc: a file-scope device array, one copy
// per GPU.  Host code never passes the array's name to a kernel (on the host
// it names a stand-in, not the device copy): each device's address comes
// from hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) char scratch[TP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

tp_status noalloc_scratch(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "noalloc: device of the stream");
  if (dev < 0 || dev >= kMaxDevices) return fail(TP_ERR_HIP, "noalloc: device %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    TP_TRY(hip_status(hipGetDevice(&cur), "noalloc: current device"));
    if (cur != dev) TP_TRY(hip_status(hipSetDevice(dev), "noalloc: select the stream's device"));
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess && r != hipSuccess) e = r;
    }
    if (e != hipSuccess) return hip_status(e, "noalloc: hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(TP_ERR_HIP, "noalloc: hipGetSymbolAddress(scratch) gave NULL on device %d", dev);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return TP_OK;
}

}  // namespace

extern "C" {

tp_status tp_mlp_forward_noalloc(void* stream, const tp_mlp_desc* d) {
  MlpShape sh;
  TP_TRY(validate_mlp(d, &sh));
  if (d->shard_count != d->N)
    return fail(TP_ERR_SHAPE, "the allocation-free forward needs the whole shard range (shard_count %d != N %d)",
                d->shard_count, d->N);
  if (d->T == 0) return ok();
  if (sh.total > TP_NOALLOC_SCRATCH_BYTES)
    return fail(TP_ERR_WORKSPACE,
                "the allocation-free forward needs %zu bytes of workspace, more than its %zu-byte static scratch "
                "(T=%lld H=%lld F=%lld N=%d); use tp_mlp_forward with a caller workspace",
                sh.total, (size_t)TP_NOALLOC_SCRATCH_BYTES, (long long)d->T, (long long)d->H, (long long)d->F,
                d->N);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  TP_TRY(noalloc_scratch(s, &ws));
  TP_TRY(mlp_rows(s, d, sh, ws, 0, d->T));
  return run_reduce(s, d->dt, d->N, d->T, d->H, reinterpret_cast<float*>(ws), d->T * d->H, d->b, d->Y, d->n_slices,
                    d->slice);
}

size_t tp_mlp_backward_workspace_size(const tp_mlp_bwd_desc* d) {
  BwdShape sh;
  return validate_mlp_bwd(d, &sh) == TP_OK ? sh.total : 0;
}

tp_status tp_mlp_backward(void* stream, const tp_mlp_bwd_desc* d, void* ws, size_t ws_bytes) {
  BwdShape sh;
  TP_TRY(validate_mlp_bwd(d, &sh));
  if (d->T == 0) return ok();
  TP_TRY(check_ws(ws, ws_bytes, sh.total));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t T = d->T, H = d->H, F = d->F, Fs = sh.Fs, Fc = sh.Fc, Fz = sh.Fz;
  const int c = d->shard_count, i0 = d->shard_begin, S = sh.splits;
  const bool gelu = d->act == TP_ACT_GELU, swiglu = d->act == TP_ACT_SWIGLU;
  const int64_t zs = swiglu ? 2 * Fs : Fs;  // Z / dZ / A columns per shard
  const tp_dtype dt = d->dt;
  const bool f32 = dt == TP_F32;
  const size_t es = esize(dt);
  if (log_enabled())
    fprintf(stderr, "[tp] mlp backward %s act=%d N=%d shards [%d,%d): T=%lld H=%lld Fs=%lld, split-K %d, %s%s%s\n",
            dt_name(dt), (int)d->act, d->N, i0, i0 + c, (long long)T, (long long)H, (long long)Fs, S,
            sh.direct ? "operands as stored" : "transposed operands",
            d->Z ? (d->Hact ? ", stored Z and H" : ", stored Z") : ", Z recomputed", c == d->N ? " ; reduce dX" : "");
  if (sh.direct) return bwd_direct(s, d, sh, static_cast<char*>(ws));
  char* base = static_cast<char*>(ws);
  char* Z = base + sh.z_off;
  char* dZ = base + sh.dz_off;
  char* Hs = base + sh.h_off;
  char* XT = base + sh.xt_off;
  char* dYT = base + sh.dyt_off;
  char* HT = base + sh.ht_off;
  char* dZT = base + sh.dzt_off;
  char* AT = base + sh.at_off;
  char* BT = base + sh.bt_off;
  float* K = reinterpret_cast<float*>(base + sh.k_off);
  const char* A_r = static_cast<const char*>(d->A) + (size_t)i0 * zs * H * es;  // range rows of A
  const char* B_r = static_cast<const char*>(d->B) + (size_t)i0 * Fs * es;      // range columns of B
  const char* a_r = d->a ? static_cast<const char*>(d->a) + (size_t)i0 * Fs * es : nullptr;

  auto transpose = [&](const char* name, const void* in, int64_t ld_in, void* out, int64_t ld_out, int64_t R,
                       int64_t C, bool act) -> tp_status {
    tp::TransposeParams t{in, ld_in, out, ld_out, R, C};
    KernelTimer kt(name, s);
    const hipError_t e = tp::launch_transpose(t, act, f32, s);
    kt.stop();
    return hip_status(e, name);
  };
  auto rowsum = [&](const char* name, const void* in, int64_t ld, float* out, int64_t R, int64_t C) -> tp_status {
    tp::RowSumParams r{in, ld, out, R, C};
    KernelTimer kt(name, s);
    const hipError_t e = tp::launch_rowsum(r, f32, s);
    kt.stop();
    return hip_status(e, name);
  };
  // C[M x N] = A[M x T] B[N x T]^T over the token axis, split-K when the
  // output is small; the splits' partials fold in split order.
  auto token_gemm = [&](const char* name, const void* Aop, const void* Bop, int64_t M, int64_t N, float* C,
                        int64_t ldc) -> tp_status {
    if (S == 1) {
      const tp::GemmParams g = gemm(Aop, T, 0, Bop, T, 0, C, ldc, 0, M, N, T, 1);
      return hip_status(launch(name, dt, g, tp::EPI_PARTIAL, s), name);
    }
    const int64_t kc = T / S;
    tp::GemmParams g = gemm(Aop, T, kc, Bop, T, kc, K, N, M * N, M, N, kc, S);
    g.xcd_per_problem = S % 8 == 0;  // each split's operand blocks stay in one XCD's L2
    TP_TRY(hip_status(launch(name, dt, g, tp::EPI_PARTIAL, s), name));
    tp::ReduceParams r{};
    r.P = K;
    r.part_stride = M * N;
    r.n_parts = S;
    r.rows = M;
    r.H = N;
    r.row0 = 0;
    r.bias = nullptr;
    r.Y = C;
    r.ldy = ldc;
    KernelTimer kt("bwd_splitk_reduce", s);
    const hipError_t e = tp::launch_reduce(r, false, s);
    kt.stop();
    return hip_status(e, "bwd_splitk_reduce");
  };

  // operands contiguous along each contraction
  TP_TRY(transpose("bwd_transpose", d->X, H, XT, T, T, H, false));    // XT  [H x T]
  TP_TRY(transpose("bwd_transpose", d->dY, H, dYT, T, T, H, false));  // dYT [H x T]
  TP_TRY(transpose("bwd_transpose", A_r, H, AT, Fz, Fz, H, false));   // AT  [H x Fz]
  TP_TRY(transpose("bwd_transpose", B_r, F, BT, H, H, Fc, false));    // BT  [Fc x H]

  if (bwd_fused_gelu(d)) {
    // dZ = (dY B_r) * GELU'(X A_r^T + a_r) and H = GELU(X A_r^T + a_r) in one kernel
    tp::GemmParams fg = gemm(d->X, H, 0, A_r, H, 0, dZ, sh.zld, 0, T, Fc, H, 1);
    fg.bias = a_r;
    fg.A2 = d->dY;
    fg.B2 = BT;
    fg.C2 = Hs;
    fg.ldc2 = Fc;
    TP_TRY(hip_status(launch("bwd_fused_gemm", TP_BF16, fg, tp::EPI_GELU_FUSED, s), "bwd_fused_gemm"));
    TP_TRY(transpose("bwd_transpose", Hs, Fc, HT, T, T, Fc, false));
    TP_TRY(transpose("bwd_transpose", dZ, sh.zld, dZT, T, T, Fz, false));  // dZT [Fz x T]
    return bwd_tail(s, d, sh, ws, dZ, dZT, XT, dYT, HT, AT, token_gemm, rowsum);
  }
  // Z = X A_r^T (+ a_r), the range's pre-activation (all shards side by side):
  // the forward's stored one, or recomputed
  const void* Zp = Z;
  int64_t zld = sh.zld;
  if (d->Z) {
    Zp = static_cast<const char*>(d->Z) + (size_t)i0 * zs * es;  // SwiGLU: [gate | up] blocks
    zld = swiglu ? 2 * F : F;
  } else {
    tp::GemmParams zg = gemm(d->X, H, 0, A_r, H, 0, Z, sh.zld, 0, T, Fz, H, 1);
    zg.bias = a_r;
    TP_TRY(hip_status(launch("bwd_recompute_gemm", dt, zg, tp::EPI_STORE, s), "bwd_recompute_gemm"));
  }
  if (swiglu) {
    // per shard: dH = dY B_i; [dG | dU] and H = SiLU(G) U from the stored [G | U]
    tp::GemmParams dg = gemm(d->dY, H, 0, BT, H, Fs * H, dZ, sh.zld, zs, T, Fs, H, c);
    dg.aux = Zp;
    dg.ldaux = zld;
    dg.sAux = zs;
    dg.upOff = Fs;
    dg.C2 = Hs;
    dg.ldc2 = Fc;
    dg.sC2 = Fs;
    TP_TRY(hip_status(launch("bwd_dz_gemm", TP_BF16, dg, tp::EPI_SWIGLU_BWD, s), "bwd_dz_gemm"));
    TP_TRY(transpose("bwd_transpose", Hs, Fc, HT, T, T, Fc, false));
  } else {
    // dZ = (dY B_r) * act'(Z)
    tp::GemmParams dg = gemm(d->dY, H, 0, BT, H, 0, dZ, sh.zld, 0, T, Fc, H, 1);
    dg.aux = Zp;
    dg.ldaux = zld;
    TP_TRY(hip_status(launch("bwd_dz_gemm", dt, dg, gelu ? tp::EPI_GELU_BWD : tp::EPI_STORE, s), "bwd_dz_gemm"));
    if (d->Hact)  // HT = H^T, the forward's activation
      TP_TRY(transpose("bwd_transpose", static_cast<const char*>(d->Hact) + (size_t)i0 * Fs * es, F, HT, T, T, Fc,
                       false));
    else
      TP_TRY(transpose("bwd_transpose", Zp, zld, HT, T, T, Fc, gelu));  // HT = act(Z)^T
  }
  TP_TRY(transpose("bwd_transpose", dZ, sh.zld, dZT, T, T, Fz, false));  // dZT [Fz x T]
  return bwd_tail(s, d, sh, ws, dZ, dZT, XT, dYT, HT, AT, token_gemm, rowsum);
}

int64_t tp_vocab_padded(int64_t V, int N) {
  if (V < 1 || N < 1) return 0;
  return vocab_shard_width(V, N) * N;
}

size_t tp_vocab_ce_workspace_size(const tp_vocab_ce_desc* d) {
  VocabShape sh;
  return validate_vocab(d, &sh) == TP_OK ? sh.total : 0;
}

tp_status tp_vocab_ce_forward(void* stream, const tp_vocab_ce_desc* d, void* ws, size_t ws_bytes) {
  VocabShape sh;
  TP_TRY(validate_vocab(d, &sh));
  if (d->T == 0) return ok();
  TP_TRY(check_ws(ws, ws_bytes, sh.total));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t T = d->T, H = d->H, Vs = sh.Vs;
  const int c = d->shard_count, i0 = d->shard_begin;
  if (log_enabled())
    fprintf(stderr, "[tp] vocab ce bf16 N=%d shards [%d,%d): X[%lld x %lld] E_i[%lld x %lld] V=%lld (padded %lld)%s\n",
            d->N, i0, i0 + c, (long long)T, (long long)H, (long long)Vs, (long long)H, (long long)d->V,
            (long long)sh.Vp, c == d->N ? " ; combine" : "");
  char* base = static_cast<char*>(ws);
  float* chunks = reinterpret_cast<float*>(base);
  const int64_t astride = (int64_t)c * sh.cps * T;
  float* m = reinterpret_cast<float*>(base + sh.m_off);
  float* sm = reinterpret_cast<float*>(base + sh.s_off);
  float* z = reinterpret_cast<float*>(base + sh.z_off);

  // logits of every shard in range (X shared: one launch), reduced in the
  // epilogue to per-chunk statistics; no logit is stored
  tp::GemmParams g = gemm(d->X, H, 0, static_cast<const bf16_t*>(d->E) + (size_t)i0 * Vs * H, H, Vs * H, nullptr,
                          Vs, 0, T, Vs, H, c);
  g.ce.labels = d->labels;
  g.ce.stats = chunks;
  g.ce.astride = astride;
  g.ce.V = d->V;
  g.ce.shard0 = i0;
  g.ce.cps = sh.cps;
  TP_TRY(hip_status(launch("vocab_logits_gemm", TP_BF16, g, tp::EPI_CE_STATS, s), "vocab_logits_gemm"));

  tp::CeFoldParams fp{};
  fp.stats = chunks;
  fp.astride = astride;
  fp.T = T;
  fp.m = m;
  fp.s = sm;
  fp.z = z;
  fp.shard0 = i0;
  fp.shards = c;
  fp.cps = sh.cps;
  {
    KernelTimer kt("vocab_ce_fold", s);
    const hipError_t e = tp::launch_ce_fold(fp, s);
    kt.stop();
    TP_TRY(hip_status(e, "vocab_ce_fold"));
  }
  if (c < d->N) return ok();

  tp::CeCombineParams cb{};
  cb.m = m;
  cb.s = sm;
  cb.z = z;
  cb.loss = d->loss;
  cb.T = T;
  cb.N = d->N;
  {
    KernelTimer kt("vocab_ce_combine", s);
    const hipError_t e = tp::launch_ce_combine(cb, s);
    kt.stop();
    TP_TRY(hip_status(e, "vocab_ce_combine"));
  }
  if (d->mean_loss) {
    KernelTimer kt("vocab_ce_mean", s);
    const hipError_t e = tp::launch_ce_mean(d->loss, T, d->mean_loss, s);
    kt.stop();
    TP_TRY(hip_status(e, "vocab_ce_mean"));
  }
  return ok();
}

size_t tp_vocab_embed_workspace_size(const tp_vocab_embed_desc* d) {
  size_t need = 0;
  return validate_embed(d, &need) == TP_OK ? need : 0;
}

tp_status tp_vocab_embed_forward(void* stream, const tp_vocab_embed_desc* d, void* ws, size_t ws_bytes) {
  size_t need = 0;
  TP_TRY(validate_embed(d, &need));
  if (d->T == 0) return ok();
  TP_TRY(check_ws(ws, ws_bytes, need));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t T = d->T, H = d->H;
  const bool f32 = d->dt == TP_F32;
  char* const P = static_cast<char*>(ws);
  tp::EmbedParams e{};
  e.ids = d->ids;
  e.E = d->E;
  e.P = P + (size_t)d->shard_begin * T * H * (f32 ? 4 : 2);
  e.sP = T * H;
  e.T = T;
  e.H = H;
  e.V = d->V;
  e.Vs = vocab_shard_width(d->V, d->N);
  e.shard0 = d->shard_begin;
  e.shards = d->shard_count;
  {
    KernelTimer kt("vocab_embed_partial", s);
    const hipError_t r = tp::launch_embed_partial(e, f32, s);
    kt.stop();
    TP_TRY(hip_status(r, "vocab_embed_partial"));
  }
  if (d->shard_count < d->N) return ok();
  tp::EmbedFoldParams f{};
  f.P = P;
  f.sP = T * H;
  f.n = T * H;
  f.N = d->N;
  f.Y = d->Y;
  KernelTimer kt("vocab_embed_fold", s);
  const hipError_t r = tp::launch_embed_fold(f, f32, s);
  kt.stop();
  TP_TRY(hip_status(r, "vocab_embed_fold"));
  return ok();
}

tp_status tp_attn_forward(void* stream, const tp_attn_desc* d, void* ws, size_t ws_bytes) {
  AttnShape sh;
  TP_TRY(validate_attn(d, &sh));
  if (sh.T == 0) return ok();
  TP_TRY(check_ws(ws, ws_bytes, sh.total));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t T = sh.T, Hd = d->hidden, hd = sh.hd;
  const int c = d->shard_count, i0 = d->shard_begin;
  if (log_enabled())
    fprintf(stderr,
            "[tp] attn N=%d shards [%d,%d): heads/shard=%lld X[%lld x %lld] Wqkv_i[%lld x %lld] -> Q,K[%lld x %lld] "
            "V^T[%lld x %lld] -> O_i[%lld x %lld] ; Wo_i[%lld x %lld] -> P_i[%lld x %lld] fp32%s\n",
            d->N, i0, i0 + c, (long long)sh.hl, (long long)T, (long long)Hd, (long long)(3 * hd), (long long)Hd,
            (long long)T, (long long)hd, (long long)hd, (long long)T, (long long)T, (long long)hd, (long long)Hd,
            (long long)hd, (long long)T, (long long)Hd, c == d->N ? " ; reduce" : "");
  if (T == 0) return ok();
  char* base = static_cast<char*>(ws);
  float* P = reinterpret_cast<float*>(base);
  void* QK = base + sh.qk_off;
  void* Vt = base + sh.vt_off;
  void* Ob = base + sh.o_off;
  const char* W0 = static_cast<const char*>(d->Wqkv) + (size_t)i0 * 3 * hd * Hd * 2;

  // Q and K of the shard's heads: [T x 2hd] = X [T x hidden] * (Q,K rows)^T
  const tp::GemmParams qk = gemm(d->X, Hd, 0, W0, Hd, 3 * hd * Hd, QK, 2 * hd, T * 2 * hd, T, 2 * hd, Hd, c);
  TP_TRY(hip_status(launch("attn_qk_gemm", TP_BF16, qk, tp::EPI_STORE, s), "attn qk launch"));
  // V^T of the shard's heads: [hd x T] = (V rows) [hd x hidden] * X^T
  const tp::GemmParams vt =
      gemm(W0 + (size_t)2 * hd * Hd * 2, Hd, 3 * hd * Hd, d->X, Hd, 0, Vt, T, hd * T, hd, T, Hd, c);
  TP_TRY(hip_status(launch("attn_vt_gemm", TP_BF16, vt, tp::EPI_STORE, s), "attn v launch"));

  tp::AttnParams a{};
  a.QK = QK;
  a.ldqk = 2 * hd;
  a.sQK = T * 2 * hd;
  a.kcol0 = hd;
  a.Vt = Vt;
  a.ldvt = T;
  a.sVt = hd * T;
  a.O = Ob;
  a.ldo = hd;
  a.sO = T * hd;
  a.batch = (int)d->batch;
  a.seq = (int)d->seq;
  a.heads = (int)sh.hl;
  a.nshards = c;
  a.scale_log2e = (float)(1.4426950408889634 / 11.313708498984761);  // log2(e) / sqrt(128)
  {
    KernelTimer kt("attn_core", s);
    const hipError_t e = tp::launch_attention(a, s);
    kt.stop();
    TP_TRY(hip_status(e, "attn launch"));
  }

  // output projection, row-parallel: P_i = O_i [T x hd] * (Wo columns of shard i)^T
  const tp::GemmParams op = gemm(Ob, hd, T * hd, static_cast<const char*>(d->Wo) + (size_t)i0 * hd * 2, Hd, hd,
                                 P + (size_t)i0 * T * Hd, Hd, T * Hd, T, Hd, hd, c);
  TP_TRY(hip_status(launch("attn_out_gemm", TP_BF16, op, tp::EPI_PARTIAL, s), "attn out-proj launch"));

  if (c < d->N) return ok();
  return run_reduce(s, TP_BF16, d->N, T, Hd, P, T * Hd, d->bo, d->Y, d->n_slices, d->slice);
}

tp_status tp_attn_local(void* stream, int64_t batch, int64_t seq, int heads, int head_dim, const void* QK,
                        int64_t ldqk, int64_t k_col0, const void* Vt, int64_t ldvt, void* O, int64_t ldo) {
  if (batch < 0 || seq < 0 || heads <= 0) return fail(TP_ERR_SHAPE, "batch=%lld seq=%lld heads=%d", (long long)batch, (long long)seq, heads);
  if (head_dim != 128) return fail(TP_ERR_SHAPE, "head_dim=%d (only 128 is built)", head_dim);
  if (seq % 128) return fail(TP_ERR_SHAPE, "seq=%lld is not a multiple of 128", (long long)seq);
  const int64_t T = batch * seq, hd = (int64_t)heads * head_dim;
  if (k_col0 < hd || k_col0 % 8)
    return fail(TP_ERR_SHAPE, "k_col0=%lld must be a multiple of 8 at or after the query columns [0, %lld)",
                (long long)k_col0, (long long)hd);
  TP_TRY(check_matrix("QK", QK, T, k_col0 + hd, ldqk, 8));
  TP_TRY(check_matrix("Vt", Vt, hd, T, ldvt, 8));
  TP_TRY(check_matrix("O", O, T, hd, ldo, 8));
  if (T > kIntMax) return fail(TP_ERR_SHAPE, "batch*seq exceeds 2^31-1");
  // one sequence's keys and one head's V^T rows are addressed with 32-bit byte offsets
  if (seq * ldqk * 2 >= (int64_t(1) << 32))
    return fail(TP_ERR_SHAPE, "seq=%lld x ldqk=%lld exceeds 4 GiB of offsets", (long long)seq, (long long)ldqk);
  if (T == 0) return ok();
  tp::AttnParams a{};
  a.QK = QK;
  a.ldqk = ldqk;
  a.kcol0 = k_col0;
  a.Vt = Vt;
  a.ldvt = ldvt;
  a.O = O;
  a.ldo = ldo;
  a.batch = (int)batch;
  a.seq = (int)seq;
  a.heads = heads;
  a.nshards = 1;
  a.scale_log2e = (float)(1.4426950408889634 / 11.313708498984761);
  KernelTimer kt("attn_core", static_cast<hipStream_t>(stream));
  const hipError_t e = tp::launch_attention(a, static_cast<hipStream_t>(stream));
  kt.stop();
  return hip_status(e, "attn_local launch");
}

tp_status tp_timing_enable(int on) {
  std::lock_guard<std::mutex> g(g_tmu);
  g_timing = on != 0;
  return ok();
}

void tp_timing_reset(void) {
  std::lock_guard<std::mutex> g(g_tmu);
  for (auto& p : g_pending) {
    (void)hipEventSynchronize(p.b);
    g_event_pool.push_back(p.a);
    g_event_pool.push_back(p.b);
  }
  g_pending.clear();
  g_totals.clear();
}

int tp_timing_read(int max, const char** names, double* total_ms, int64_t* launches) {
  std::lock_guard<std::mutex> g(g_tmu);
  for (auto& p : g_pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(p.b) == hipSuccess && hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
      auto& t = g_totals[p.name];
      t.first += ms;
      t.second += 1;
    }
    g_event_pool.push_back(p.a);
    g_event_pool.push_back(p.b);
  }
  g_pending.clear();
  g_names.clear();
  for (auto& kv : g_totals) g_names.push_back(kv.first);
  int i = 0;
  for (auto& kv : g_totals) {
    if (i >= max) break;
    if (names) names[i] = g_names[i].c_str();
    if (total_ms) total_ms[i] = kv.second.first;
    if (launches) launches[i] = kv.second.second;
    ++i;
  }
  return (int)g_totals.size();
}

const char* tp_status_string(tp_status s) {
  switch (s) {
    case TP_OK: return "TP_OK";
    case TP_ERR_NULL: return "TP_ERR_NULL";
    case TP_ERR_SHAPE: return "TP_ERR_SHAPE";
    case TP_ERR_DIVISIBILITY: return "TP_ERR_DIVISIBILITY";
    case TP_ERR_DTYPE: return "TP_ERR_DTYPE";
    case TP_ERR_ALIGN: return "TP_ERR_ALIGN";
    case TP_ERR_WORKSPACE: return "TP_ERR_WORKSPACE";
    case TP_ERR_HIP: return "TP_ERR_HIP";
  }
  return "TP_ERR_UNKNOWN";
}

const char* tp_last_error(void) { return g_err.c_str(); }

const char* tp_version(void) { return "libtp 0.1 (gfx950)"; }

}  // extern "C"
