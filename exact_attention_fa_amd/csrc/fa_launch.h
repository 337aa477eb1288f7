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
  size_t delta;    // fp32 (B, Hq, N): D = rowsum(dO * O)
  size_t lse2;     // fp32 (B, Hq, N): LSE * log2(e)
  size_t dk_part;  // fp32 (B, Hq, N, D): per-query-head dK partials (only when Hq > Hkv)
  size_t dv_part;  // fp32 (B, Hq, N, D): per-query-head dV partials (only when Hq > Hkv)
  size_t total;
};
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
};

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_merge(const MergeArgs& a);
int fwd_auto_parts(long long B, long long Hq, long long N, long long D, bool causal);
hipError_t launch_bwd_preprocess(const BwdArgs& a);
hipError_t launch_bwd_dkdv(const BwdArgs& a);
hipError_t launch_bwd_dq(const BwdArgs& a);
hipError_t launch_bwd_postprocess(const BwdArgs& a);

}  // namespace fa
