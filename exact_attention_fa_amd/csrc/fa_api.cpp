// C-ABI entry points: argument validation, workspace layout and dispatch to the HIP
// launchers.  Every check happens before anything is enqueued, so a rejected call has no
// side effect ("FlashAttention for Tesla P100", section "What it supports": unsupported
// requests raise instead of degrading quietly).
#include "../../include/fa.h"

#include <math.h>
#include <stdint.h>

#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kVersion = 10100;  // 1.1.0
constexpr int kMaxParts = 64;    // key-range pieces / merge parts per call

size_t round_up(size_t x) { return (x + 255u) & ~(size_t)255u; }

int check_dims(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0) return FA_ERR_BAD_SHAPE;
  if (D != 64 && D != 128) return FA_ERR_HEAD_DIM;
  if (Hq % Hkv != 0) return FA_ERR_GQA;
  const int64_t lim = INT32_MAX;
  // The kernels index heads, rows and grid blocks with 32-bit integers.
  if (N > lim / D || B > lim / Hq || B * Hq > lim / N) return FA_ERR_TOO_LARGE;
  return FA_OK;
}

int check_dtype(int dtype) {
  return (dtype == FA_FP16 || dtype == FA_BF16 || dtype == FA_FP32) ? FA_OK : FA_ERR_DTYPE;
}
int check_dtype16(int dtype) { return (dtype == FA_FP16 || dtype == FA_BF16) ? FA_OK : FA_ERR_DTYPE; }
size_t elem_size(int dtype) { return dtype == FA_FP32 ? 4 : 2; }

int check_scale(float s) { return isfinite(s) ? FA_OK : FA_ERR_SCALE; }

int check_ptr(const void* p, uintptr_t align) {
  if (p == nullptr) return FA_ERR_NULL_POINTER;
  if (reinterpret_cast<uintptr_t>(p) % align != 0) return FA_ERR_ALIGNMENT;
  return FA_OK;
}

struct Range {
  const void* p;
  size_t bytes;
  bool output;
};

// Outputs may not overlap any other buffer of the call.
int check_alias(const Range* r, int n) {
  for (int i = 0; i < n; ++i) {
    if (!r[i].output || r[i].p == nullptr) continue;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(r[i].p), a1 = a0 + r[i].bytes;
    for (int j = 0; j < n; ++j) {
      if (j == i || r[j].p == nullptr) continue;
      const uintptr_t b0 = reinterpret_cast<uintptr_t>(r[j].p), b1 = b0 + r[j].bytes;
      if (a0 < b1 && b0 < a1) return FA_ERR_ALIAS;
    }
  }
  return FA_OK;
}

#define FA_TRY(expr)              \
  do {                            \
    const int _rc = (expr);       \
    if (_rc != FA_OK) return _rc; \
  } while (0)

int status_of(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

}  // namespace

BwdWorkspace bwd_workspace_layout(long long B, long long Hq, long long Hkv, long long N, long long D) {
  BwdWorkspace w{};
  const size_t rows = (size_t)B * (size_t)Hq * (size_t)N;
  w.n_qp = bwd_query_pieces(B, Hq, Hkv, N, D);
  w.n_kp = bwd_key_pieces(B, Hq, N, D);
  w.partial_dkdv = Hq != Hkv || w.n_qp > 1;
  size_t off = 0;
  w.delta = off;
  off += round_up(rows * 4);
  w.lse2 = off;
  off += round_up(rows * 4);
  if (w.partial_dkdv) {
    w.dk_part = off;
    off += round_up(rows * (size_t)w.n_qp * (size_t)D * 4);
    w.dv_part = off;
    off += round_up(rows * (size_t)w.n_qp * (size_t)D * 4);
  }
  if (w.n_kp > 1) {
    w.dq_part = off;
    off += round_up(rows * (size_t)w.n_kp * (size_t)D * 4);
  }
  w.total = off;
  return w;
}

}  // namespace fa

using namespace fa;

namespace {

// Validation common to the backward entry points; pointers are checked by the callers.
int check_bwd_common(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D, int dtype,
                     const void* ws, size_t ws_bytes) {
  FA_TRY(check_dtype(dtype));
  FA_TRY(check_dims(B, Hq, Hkv, N, D));
  FA_TRY(check_ptr(ws, 16));
  if (ws_bytes < bwd_workspace_layout(B, Hq, Hkv, N, D).total) return FA_ERR_WORKSPACE;
  return FA_OK;
}

// fa_bwd's order: the dQ pass first, forming the row values itself, where the dK/dV pass writes
// dk and dv directly (16-bit tensors); otherwise the preprocess first.
bool bwd_rows_first(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D, int dtype) {
  return dtype != FA_FP32 && !bwd_workspace_layout(B, Hq, Hkv, N, D).partial_dkdv;
}

BwdArgs make_bwd_args(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, void* ws, int64_t B, int64_t Hq,
                      int64_t Hkv, int64_t N, int64_t D, float scale, int causal, int dtype, void* stream) {
  BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, static_cast<char*>(ws), B, Hq, Hkv, N, D, scale,
            causal != 0, dtype == FA_BF16, static_cast<hipStream_t>(stream)};
  a.f32 = dtype == FA_FP32;
  return a;
}

}  // namespace

extern "C" {

int fa_version(void) { return kVersion; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case FA_ERR_BAD_SHAPE: return "B, Hq, Hkv and N must be positive";
    case FA_ERR_HEAD_DIM: return "head dim D must be 64 or 128";
    case FA_ERR_GQA: return "Hq must be a multiple of Hkv";
    case FA_ERR_DTYPE: return "dtype must be FA_FP16 or FA_BF16 (or FA_FP32 for fa_fwd, fa_bwd and its stages)";
    case FA_ERR_SCALE: return "softmax_scale must be finite";
    case FA_ERR_ALIGNMENT: return "buffers must be 16-byte aligned (lse: 4-byte)";
    case FA_ERR_WORKSPACE: return "workspace is smaller than fa_bwd_workspace_size()";
    case FA_ERR_HIP: return "the HIP runtime rejected a kernel launch";
    case FA_ERR_TOO_LARGE: return "problem size exceeds the 32-bit index range of the kernels";
    case FA_ERR_ALIAS: return "an output buffer overlaps another buffer of the call";
    case FA_ERR_SPLIT: return "split / part count out of range (1..64, or 0 for the library's choice)";
    case FA_ERR_SCRATCH: return "fa_bwd_noalloc: the call needs more workspace than the 80 MiB static scratch";
    default: return "unknown status";
  }
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
           int64_t Hkv, int64_t N, int64_t D, float softmax_scale, int causal, int dtype, void* stream) {
  FA_TRY(check_dtype(dtype));
  FA_TRY(check_dims(B, Hq, Hkv, N, D));
  FA_TRY(check_scale(softmax_scale));
  FA_TRY(check_ptr(q, 16));
  FA_TRY(check_ptr(k, 16));
  FA_TRY(check_ptr(v, 16));
  FA_TRY(check_ptr(o, 16));
  FA_TRY(check_ptr(lse, 4));
  const size_t qb = (size_t)(B * Hq * N * D) * elem_size(dtype), kb = (size_t)(B * Hkv * N * D) * elem_size(dtype);
  const Range r[] = {{q, qb, false}, {k, kb, false}, {v, kb, false}, {o, qb, true},
                     {lse, (size_t)(B * Hq * N) * 4, true}};
  FA_TRY(check_alias(r, 5));
  FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, D, softmax_scale, causal != 0, dtype == FA_BF16,
            static_cast<hipStream_t>(stream)};
  a.f32 = dtype == FA_FP32;
  return status_of(launch_fwd(a));
}

int fa_fwd_splitkv_parts(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D, int causal) {
  if (check_dims(B, Hq, Hkv, N, D) != FA_OK) return 0;
  return fwd_auto_parts(B, Hq, N, D, causal != 0);
}

size_t fa_fwd_splitkv_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D, int n_split) {
  if (check_dims(B, Hq, Hkv, N, D) != FA_OK || n_split < 1 || n_split > kMaxParts) return 0;
  if (n_split == 1) return 0;
  const size_t rows = (size_t)B * (size_t)Hq * (size_t)N;
  return round_up((size_t)n_split * rows * (size_t)D * 4) + round_up((size_t)n_split * rows * 4);
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                   size_t workspace_bytes, int n_split, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D,
                   float softmax_scale, int causal, int dtype, void* stream) {
  FA_TRY(check_dtype(dtype));
  FA_TRY(check_dims(B, Hq, Hkv, N, D));
  FA_TRY(check_scale(softmax_scale));
  if (n_split < 0 || n_split > kMaxParts) return FA_ERR_SPLIT;
  // the fp32 path has no pieces: any count resolves to fa_fwd
  const int n = dtype == FA_FP32 ? 1 : (n_split == 0 ? fwd_auto_parts(B, Hq, N, D, causal != 0) : n_split);
  if (n == 1) return fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, D, softmax_scale, causal, dtype, stream);
  FA_TRY(check_ptr(q, 16));
  FA_TRY(check_ptr(k, 16));
  FA_TRY(check_ptr(v, 16));
  FA_TRY(check_ptr(o, 16));
  FA_TRY(check_ptr(lse, 4));
  FA_TRY(check_ptr(workspace, 256));
  const size_t need = fa_fwd_splitkv_workspace_size(B, Hq, Hkv, N, D, n);
  if (workspace_bytes < need) return FA_ERR_WORKSPACE;
  const size_t rows = (size_t)(B * Hq * N);
  const size_t qb = rows * (size_t)D * 2, kb = (size_t)(B * Hkv * N * D) * 2;  // 16-bit here
  const Range r[] = {{q, qb, false}, {k, kb, false}, {v, kb, false}, {o, qb, true}, {lse, rows * 4, true},
                     {workspace, need, true}};
  FA_TRY(check_alias(r, 6));
  float* const op = static_cast<float*>(workspace);
  float* const lp = reinterpret_cast<float*>(static_cast<char*>(workspace) + round_up((size_t)n * rows * D * 4));
  FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, D, softmax_scale, causal != 0, dtype == FA_BF16,
            static_cast<hipStream_t>(stream), false, n, op, lp};
  FA_TRY(status_of(launch_fwd(a)));
  const MergeArgs m{op, lp, n, (long long)rows, D, o, lse, dtype == FA_BF16, static_cast<hipStream_t>(stream)};
  return status_of(launch_merge(m));
}

int fa_merge_partials(const float* o_parts, const float* lse_parts, int n_parts, void* o, float* lse, int64_t rows,
                      int64_t D, int dtype, void* stream) {
  FA_TRY(check_dtype16(dtype));
  if (rows <= 0) return FA_ERR_BAD_SHAPE;
  if (D != 64 && D != 128) return FA_ERR_HEAD_DIM;
  if (n_parts < 1 || n_parts > kMaxParts) return FA_ERR_SPLIT;
  if (rows > (int64_t)INT32_MAX * 8 / D) return FA_ERR_TOO_LARGE;
  FA_TRY(check_ptr(o_parts, 16));
  FA_TRY(check_ptr(lse_parts, 4));
  FA_TRY(check_ptr(o, 16));
  FA_TRY(check_ptr(lse, 4));
  const size_t pr = (size_t)n_parts * (size_t)rows;
  const Range r[] = {{o_parts, pr * (size_t)D * 4, false}, {lse_parts, pr * 4, false},
                     {o, (size_t)rows * (size_t)D * 2, true}, {lse, (size_t)rows * 4, true}};
  FA_TRY(check_alias(r, 4));
  const MergeArgs m{o_parts, lse_parts, n_parts, rows, D, o, lse, dtype == FA_BF16, static_cast<hipStream_t>(stream)};
  return status_of(launch_merge(m));
}

size_t fa_bwd_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D) {
  if (check_dims(B, Hq, Hkv, N, D) != FA_OK) return 0;
  return bwd_workspace_layout(B, Hq, Hkv, N, D).total;
}


int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
           void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int64_t B, int64_t Hq,
           int64_t Hkv, int64_t N, int64_t D, float softmax_scale, int causal, int dtype, void* stream) {
  FA_TRY(check_bwd_common(B, Hq, Hkv, N, D, dtype, workspace, workspace_bytes));
  FA_TRY(check_scale(softmax_scale));
  const void* p16[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* p : p16) FA_TRY(check_ptr(p, 16));
  FA_TRY(check_ptr(lse, 4));
  const size_t qb = (size_t)(B * Hq * N * D) * elem_size(dtype), kb = (size_t)(B * Hkv * N * D) * elem_size(dtype);
  const Range r[] = {{q, qb, false},  {k, kb, false},  {v, kb, false},  {o, qb, false},
                     {dout, qb, false}, {lse, (size_t)(B * Hq * N) * 4, false},
                     {dq, qb, true},  {dk, kb, true},  {dv, kb, true},
                     {workspace, bwd_workspace_layout(B, Hq, Hkv, N, D).total, true}};
  FA_TRY(check_alias(r, 10));
  const BwdArgs a = make_bwd_args(q, k, v, o, dout, lse, dq, dk, dv, workspace, B, Hq, Hkv, N, D, softmax_scale,
                                  causal, dtype, stream);
  // Without dK/dV partials the dQ pass runs first and forms the row values the dK/dV pass reads
  // (one launch fewer); otherwise the preprocess runs first and the dQ pass follows the dK/dV
  // pass, whose partials it sums.
  if (bwd_rows_first(B, Hq, Hkv, N, D, dtype)) {
    FA_TRY(status_of(launch_bwd_dq_rows(a)));
    return status_of(launch_bwd_dkdv(a));
  }
  FA_TRY(status_of(launch_bwd_preprocess(a)));
  FA_TRY(status_of(launch_bwd_dkdv(a)));
  return status_of(launch_bwd_dq_post(a));
}

int fa_bwd_preprocess(const void* o, const void* dout, const float* lse, void* workspace, size_t workspace_bytes,
                      int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D, int dtype, void* stream) {
  FA_TRY(check_bwd_common(B, Hq, Hkv, N, D, dtype, workspace, workspace_bytes));
  FA_TRY(check_ptr(o, 16));
  FA_TRY(check_ptr(dout, 16));
  FA_TRY(check_ptr(lse, 4));
  const size_t qb = (size_t)(B * Hq * N * D) * elem_size(dtype);
  const Range r[] = {{o, qb, false}, {dout, qb, false}, {lse, (size_t)(B * Hq * N) * 4, false},
                     {workspace, bwd_workspace_layout(B, Hq, Hkv, N, D).total, true}};
  FA_TRY(check_alias(r, 4));
  const BwdArgs a = make_bwd_args(nullptr, nullptr, nullptr, o, dout, lse, nullptr, nullptr, nullptr, workspace,
                                  B, Hq, Hkv, N, D, 1.f, 0, dtype, stream);
  return status_of(launch_bwd_preprocess(a));
}

int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dv, void* workspace,
                size_t workspace_bytes, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D,
                float softmax_scale, int causal, int dtype, void* stream) {
  FA_TRY(check_bwd_common(B, Hq, Hkv, N, D, dtype, workspace, workspace_bytes));
  FA_TRY(check_scale(softmax_scale));
  const void* p16[] = {q, k, v, dout};
  for (const void* p : p16) FA_TRY(check_ptr(p, 16));
  // the fp32 path writes dk/dv directly; the 16-bit path writes partials for GQA and pieces
  const bool direct = dtype == FA_FP32 || !bwd_workspace_layout(B, Hq, Hkv, N, D).partial_dkdv;
  if (direct) {
    FA_TRY(check_ptr(dk, 16));
    FA_TRY(check_ptr(dv, 16));
  }
  const size_t qb = (size_t)(B * Hq * N * D) * elem_size(dtype), kb = (size_t)(B * Hkv * N * D) * elem_size(dtype);
  const Range r[] = {{q, qb, false}, {k, kb, false}, {v, kb, false}, {dout, qb, false},
                     {direct ? dk : nullptr, kb, true}, {direct ? dv : nullptr, kb, true},
                     {workspace, bwd_workspace_layout(B, Hq, Hkv, N, D).total, !direct}};
  FA_TRY(check_alias(r, 7));
  const BwdArgs a = make_bwd_args(q, k, v, nullptr, dout, nullptr, nullptr, dk, dv, workspace, B, Hq, Hkv, N, D,
                                  softmax_scale, causal, dtype, stream);
  return status_of(launch_bwd_dkdv(a));
}

int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout, void* dq, void* workspace,
              size_t workspace_bytes, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D,
              float softmax_scale, int causal, int dtype, void* stream) {
  FA_TRY(check_bwd_common(B, Hq, Hkv, N, D, dtype, workspace, workspace_bytes));
  FA_TRY(check_scale(softmax_scale));
  const void* p16[] = {q, k, v, dout, dq};
  for (const void* p : p16) FA_TRY(check_ptr(p, 16));
  const size_t qb = (size_t)(B * Hq * N * D) * elem_size(dtype), kb = (size_t)(B * Hkv * N * D) * elem_size(dtype);
  const BwdWorkspace w = bwd_workspace_layout(B, Hq, Hkv, N, D);
  const Range r[] = {{q, qb, false}, {k, kb, false}, {v, kb, false}, {dout, qb, false}, {dq, qb, true},
                     {workspace, w.total, w.n_kp > 1 && dtype != FA_FP32}};
  FA_TRY(check_alias(r, 6));
  const BwdArgs a = make_bwd_args(q, k, v, nullptr, dout, nullptr, dq, nullptr, nullptr, workspace, B, Hq, Hkv, N, D,
                                  softmax_scale, causal, dtype, stream);
  return status_of(launch_bwd_dq(a));
}

int fa_bwd_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D, int dtype) {
  const int e = check_dtype(dtype) != FA_OK ? check_dtype(dtype) : check_dims(B, Hq, Hkv, N, D);
  if (e != FA_OK) return -e;
  return bwd_rows_first(B, Hq, Hkv, N, D, dtype) ? FA_BWD_PLAN_ROWS : FA_BWD_PLAN_STAGES;
}

int fa_bwd_dq_rows(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* workspace, size_t workspace_bytes, int64_t B, int64_t Hq, int64_t Hkv,
                   int64_t N, int64_t D, float softmax_scale, int causal, int dtype, void* stream) {
  FA_TRY(check_bwd_common(B, Hq, Hkv, N, D, dtype, workspace, workspace_bytes));
  FA_TRY(check_scale(softmax_scale));
  const void* p16[] = {q, k, v, o, dout, dq};
  for (const void* p : p16) FA_TRY(check_ptr(p, 16));
  FA_TRY(check_ptr(lse, 4));
  const size_t qb = (size_t)(B * Hq * N * D) * elem_size(dtype), kb = (size_t)(B * Hkv * N * D) * elem_size(dtype);
  const Range r[] = {{q, qb, false},    {k, kb, false},  {v, kb, false},
                     {o, qb, false},    {dout, qb, false}, {lse, (size_t)(B * Hq * N) * 4, false},
                     {dq, qb, true},    {workspace, bwd_workspace_layout(B, Hq, Hkv, N, D).total, true}};
  FA_TRY(check_alias(r, 8));
  const BwdArgs a = make_bwd_args(q, k, v, o, dout, lse, dq, nullptr, nullptr, workspace, B, Hq, Hkv, N, D,
                                  softmax_scale, causal, dtype, stream);
  if (a.f32) {  // the fp32 path has no combined pass: the two stages
    FA_TRY(status_of(launch_bwd_preprocess(a)));
    return status_of(launch_bwd_dq(a));
  }
  return status_of(launch_bwd_dq_rows(a));
}

int fa_bwd_postprocess(void* dk, void* dv, void* workspace, size_t workspace_bytes, int64_t B, int64_t Hq,
                       int64_t Hkv, int64_t N, int64_t D, int dtype, void* stream) {
  FA_TRY(check_bwd_common(B, Hq, Hkv, N, D, dtype, workspace, workspace_bytes));
  FA_TRY(check_ptr(dk, 16));
  FA_TRY(check_ptr(dv, 16));
  const size_t kb = (size_t)(B * Hkv * N * D) * elem_size(dtype);
  const Range r[] = {{dk, kb, true}, {dv, kb, true},
                     {workspace, bwd_workspace_layout(B, Hq, Hkv, N, D).total, false}};
  FA_TRY(check_alias(r, 3));
  const BwdArgs a = make_bwd_args(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, dk, dv, workspace,
                                  B, Hq, Hkv, N, D, 1.f, 0, dtype, stream);
  return status_of(launch_bwd_postprocess(a));
}

}  // extern "C"
