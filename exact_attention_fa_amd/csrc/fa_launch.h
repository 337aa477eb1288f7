// Internal interface between the C-ABI layer (fa_api.cpp) and the kernel launchers.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  long long B, Hq, Hkv, N, D;
  float scale;
  bool causal;
  bool bf16;
  hipStream_t stream;
  bool f32 = false;          // float32 tensors (the fp32 verification path; bf16 is ignored)
  int n_part = 1;            // > 1: key-range pieces written as fp32 partials (o_part, lse_part)
  float* o_part = nullptr;   // (n_part, B, Hq, N, D)
  float* lse_part = nullptr; // (n_part, B, Hq, N)
};

// Merge of fp32 partial results over disjoint key sets (see fa_merge_partials).
struct MergeArgs {
  const float* o_part;   // (n_part, rows, D)
  const float* lse_part; // (n_part, rows)
  int n_part;
  long long rows, D;
  void* o;
  float* lse;
  bool bf16;
  hipStream_t stream;
};

// Workspace carve-up used by the backward stages (byte offsets from the base).
struct BwdWorkspace {
  size_t delta;    // fp32 (B, Hq, N): -D = -rowsum(dO * O)
  size_t lse2;     // fp32 (B, Hq, N): LSE * log2(e)
  size_t dk_part;  // fp32 (B, Hq, n_qp, N, D): dK partials per query head and query-range piece
  size_t dv_part;  // fp32 (B, Hq, n_qp, N, D): dV partials (both only when partial_dkdv)
  size_t dq_part;  // fp32 (B, Hq, n_kp, N, D): dQ partials per key-range piece (only when n_kp > 1)
  int n_qp;        // query-range pieces of the dK/dV pass
  int n_kp;        // key-range pieces of the dQ pass
  bool partial_dkdv;  // the dK/dV pass writes partials (Hq > Hkv or n_qp > 1)
  size_t total;
};
// Pieces for grids too small to occupy every CU (depend on the shape only).
int bwd_query_pieces(long long B, long long Hq, long long Hkv, long long N, long long D);
int bwd_key_pieces(long long B, long long Hq, long long N, long long D);
BwdWorkspace bwd_workspace_layout(long long B, long long Hq, long long Hkv, long long N, long long D);

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  char* ws;
  long long B, Hq, Hkv, N, D;
  float scale;
  bool causal;
  bool bf16;
  hipStream_t stream;
  bool f32 = false;  // float32 tensors (the fp32 verification path)
};

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_merge(const MergeArgs& a);
int fwd_auto_parts(long long B, long long Hq, long long N, long long D, bool causal);
hipError_t launch_bwd_preprocess(const BwdArgs& a);
hipError_t launch_bwd_dkdv(const BwdArgs& a);
hipError_t launch_bwd_dq(const BwdArgs& a);
// The dQ pass followed by the postprocess, with the grouped-query dK/dV partial sums run inside
// the dQ pass where its grid allows: the same results as launch_bwd_dq, launch_bwd_postprocess.
hipError_t launch_bwd_dq_post(const BwdArgs& a);
// The dQ pass forming and storing the row values (-D, LSE*log2(e)) itself, in place of the
// preprocess launch before it: 16-bit tensors, and only where the dK/dV pass that follows
// writes no partials.  The same results as launch_bwd_preprocess, launch_bwd_dq.
hipError_t launch_bwd_dq_rows(const BwdArgs& a);
hipError_t launch_bwd_postprocess(const BwdArgs& a);
// The fp32 verification path (fa_f32.hip); launch_fwd and the launch_bwd_* stages dispatch to
// these when FwdArgs::f32 / BwdArgs::f32 is set.
hipError_t launch_fwd_f32(const FwdArgs& a);
hipError_t launch_bwd_preprocess_f32(const BwdArgs& a);
hipError_t launch_bwd_dkdv_f32(const BwdArgs& a);
hipError_t launch_bwd_dq_f32(const BwdArgs& a);

}  // namespace fa
