/*
 * fa.h - C ABI of a fused, tiled, exact scaled-dot-product attention library for
 * AMD MI355X (gfx950).
 *
 * The operation ("From-scratch CUDA attention kernel reaches 94.4% of FlashAttention-4
 * on NVIDIA B200", section "How the kernel partitions its work"; "FlashAttention for
 * Tesla P100", sections "What it supports" and "Documentation"):
 *
 *   S   = scale * Q K^T                         per (batch, query head)
 *   P   = softmax over the visible keys of each row of S
 *   O   = P V
 *   LSE = log-sum-exp (natural log) of each row of S over its visible keys
 *
 * and its gradient for an upstream dO, with D = rowsum(dO * O):
 *
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q
 *
 * where P is recomputed from the saved LSE.  The N x N matrices S and P are never
 * stored.
 *
 * Conventions shared by every entry point
 *   Layout     Q, O, dO, dQ: (B, Hq, N, D); K, V, dK, dV: (B, Hkv, N, D); LSE: (B, Hq, N).
 *              All contiguous row-major, D innermost, no strides.  Sequence length N is
 *              the same for queries and keys (self-attention).
 *   dtype      FA_FP16 or FA_BF16 for every 16-bit tensor of a call; LSE, the backward
 *              workspace and all accumulation are fp32.  Outputs are rounded to nearest
 *              even.  FA_FP32 selects the float32 verification path for fa_fwd, fa_bwd and
 *              the fa_bwd stages: every tensor float32, products and sums in fp32 FMAs
 *              ("FlashAttention for Tesla P100", section "What it supports": fp32
 *              accumulation; "FlashNystrom", section "Scope": an fp32 path kept for
 *              gradient checking).  It is plain and correct rather than fast (no matrix
 *              cores), for checking the 16-bit results against.  fa_fwd_splitkv runs it
 *              as fa_fwd; fa_merge_partials does not take it.
 *   Heads      Hq must be a multiple of Hkv; query head h reads KV head h / (Hq / Hkv)
 *              (MHA, GQA and MQA).
 *   Causal     causal != 0: key j is visible to query i iff j <= i (square, top-left).
 *              Blocks above the diagonal are skipped, not computed and masked.
 *   Scale      softmax_scale: any finite value.  0 gives uniform attention; a negative scale
 *              is exact too (the kernels run |scale| on the negated Q, or K, operand).
 *   D          64 or 128.  N >= 1, arbitrary (ragged tails need no padding).
 *   Pointers   device pointers, 16-byte aligned, not aliasing one another.  The caller
 *              owns every buffer; inputs are only read, outputs are fully overwritten.
 *   Stream     a hipStream_t passed as void*; NULL is the default stream.  Work is only
 *              enqueued: nothing synchronises, allocates or frees device memory, and the
 *              library keeps no mutable global state (apart from fa_bwd_noalloc's static
 *              scratch array, see there).
 *   Errors     every argument is checked before anything is enqueued; on a non-zero
 *              status nothing was launched and no output was touched.  FA_ERR_HIP means a
 *              launch was rejected by the runtime.  Faults inside a kernel surface at the
 *              caller's next synchronisation, as for any stream library.
 *   Not offered (rejected by construction rather than silently degraded): dropout,
 *              attention bias, arbitrary or padding masks, sliding windows, block
 *              sparsity, KV-cache decoding, Nq != Nk, other head dims.
 */
#ifndef FA_MI355X_FA_H
#define FA_MI355X_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fa_dtype {
  FA_FP16 = 0,
  FA_BF16 = 1,
  FA_FP32 = 2  /* float32 verification path: fa_fwd, fa_bwd and its stages only */
};

enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL_POINTER = 1, /* a required pointer is NULL */
  FA_ERR_BAD_SHAPE = 2,    /* B, Hq, Hkv or N <= 0 */
  FA_ERR_HEAD_DIM = 3,     /* D is not 64 or 128 */
  FA_ERR_GQA = 4,          /* Hq is not a multiple of Hkv */
  FA_ERR_DTYPE = 5,        /* dtype is not FA_FP16 / FA_BF16 (/ FA_FP32 where accepted) */
  FA_ERR_SCALE = 6,        /* softmax_scale is NaN or infinite */
  FA_ERR_ALIGNMENT = 7,    /* a pointer is not 16-byte aligned */
  FA_ERR_WORKSPACE = 8,    /* workspace_bytes < fa_bwd_workspace_size(...) */
  FA_ERR_HIP = 9,          /* the HIP runtime rejected a launch */
  FA_ERR_TOO_LARGE = 10,   /* a size exceeds the 32-bit index range the kernels use */
  FA_ERR_ALIAS = 11,       /* an output buffer overlaps another buffer of the call */
  FA_ERR_SPLIT = 12,       /* a split / part count is out of range */
  FA_ERR_SCRATCH = 13      /* fa_bwd_noalloc: the call needs more than FA_NOALLOC_SCRATCH_BYTES */
};

/* Library version as major*10000 + minor*100 + patch. */
int fa_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char* fa_status_string(int status);

/*
 * Forward.  Reads q (B,Hq,N,D), k and v (B,Hkv,N,D); writes o (B,Hq,N,D, same dtype)
 * and lse (B,Hq,N, fp32, natural-log units of the scaled scores).  One kernel launch.
 * Bitwise deterministic.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D,
           float softmax_scale, int causal, int dtype, void* stream);

/*
 * Forward with the key range of every query tile cut into n_split contiguous pieces, for
 * grids too small to fill the GPU (few batch x head x query tiles, long sequences: the
 * per-GPU share of a head-sharded problem).  Each piece writes its normalised output and
 * log-sum-exp as fp32 partials into the workspace, and a merge pass (fa_merge_partials)
 * combines them through the LSEs ("FlashNystrom", section "Latency": splitting the work of
 * one output over several workgroups keeps a low batch x head grid busy).  Same inputs,
 * outputs and conventions as fa_fwd; the result equals fa_fwd's up to the rounding order
 * and is bitwise deterministic for a given n_split.
 *   n_split    1..64 pieces, or 0 for fa_fwd_splitkv_parts(...) (the library's choice).
 *              A resolved count of 1 is exactly fa_fwd, and the workspace may then be NULL.
 *   workspace  caller-owned device memory of at least
 *              fa_fwd_splitkv_workspace_size(B, Hq, Hkv, N, D, n) bytes for the resolved n:
 *              n x (B, Hq, N, D) fp32 outputs and n x (B, Hq, N) fp32 LSEs, 256-byte aligned.
 * Errors as fa_fwd, plus FA_ERR_SPLIT (n_split outside 0..64) and FA_ERR_WORKSPACE.
 */
int fa_fwd_splitkv_parts(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D, int causal);
size_t fa_fwd_splitkv_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D, int n_split);
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                   size_t workspace_bytes, int n_split, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                   int64_t D, float softmax_scale, int causal, int dtype, void* stream);

/*
 * Merge of attention results over disjoint key sets (the merge step of fa_fwd_splitkv, and
 * the step a sequence-parallel port would use to combine per-block results).  For each of
 * `rows` rows, part s holds the output over its key set, normalised, o_parts[(s*rows + r)*D + d]
 * (fp32), and its natural-log log-sum-exp lse_parts[s*rows + r] (-inf for an empty set).
 * With m = max_s LSE_s and w_s = exp(LSE_s - m):
 *   lse[r] = m + log(sum_s w_s),   o[r] = sum_s (w_s / sum_s w_s) o_s[r]   (rounded to dtype)
 * A row whose parts are all empty gets o = 0 and lse = -inf.  Parts are summed in index order
 * (deterministic).  n_parts 1..64; D 64 or 128; o and o_parts 16-byte aligned, lse and
 * lse_parts 4-byte aligned.
 */
int fa_merge_partials(const float* o_parts, const float* lse_parts, int n_parts, void* o, float* lse,
                      int64_t rows, int64_t D, int dtype, void* stream);

/*
 * Bytes of device workspace fa_bwd needs: the fp32 D = rowsum(dO * O) and LSE * log2(e)
 * vectors; fp32 dK/dV partials per query head and query-range piece when Hq > Hkv or the
 * grid is cut into query-range pieces; fp32 dQ partials per key-range piece when the dQ
 * pass's grid is cut into such pieces (grids too small to fill the GPU).  Returns 0 for
 * invalid shapes.
 */
size_t fa_bwd_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D);

/*
 * Backward.  Inputs q, k, v, o (from fa_fwd), dout (dO, shape of q), lse (from fa_fwd);
 * outputs dq (shape of q), dk and dv (shape of k); all 16-bit tensors in `dtype`.
 * workspace: caller-owned device memory of at least fa_bwd_workspace_size(...) bytes,
 * contents undefined before and after.  Enqueues the stages below in the order
 * fa_bwd_plan(...) names; where it runs fa_bwd_dq after fa_bwd_dkdv, the dQ pass also
 * performs fa_bwd_postprocess's sums if its grid has no key-range pieces (one launch
 * fewer, the same bits).  No atomics: every output element is reduced in a fixed order, so
 * the result is bitwise deterministic.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
           int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D,
           float softmax_scale, int causal, int dtype, void* stream);

/*
 * The stages of fa_bwd, exported so a caller (or a profiler harness) can place events
 * between them.  Running them on one stream with the same workspace, in the order
 * fa_bwd_plan(...) gives, enqueues exactly fa_bwd's kernels (apart from the postprocess
 * fa_bwd folds into its dQ pass) and gives its bits; the order fa_bwd_preprocess,
 * fa_bwd_dkdv, fa_bwd_dq, fa_bwd_postprocess gives the same bits for every problem
 * (fa_bwd_dkdv and fa_bwd_dq only depend on the row values and may run in either order).
 *   fa_bwd_preprocess:  -D = -rowsum(dout * o) and LSE * log2(e) into the workspace (fp32).
 *   fa_bwd_dkdv:        key-stationary pass: recomputes P from the workspace's LSE and
 *                       writes dk = scale * dS^T Q and dv = P^T dO, or fp32 partials into the
 *                       workspace (Hq > Hkv, or grids cut into query-range pieces).
 *   fa_bwd_dq:          query-stationary pass: recomputes P and dS and writes
 *                       dq = scale * dS K.
 *   fa_bwd_dq_rows:     fa_bwd_preprocess and fa_bwd_dq as one pass: each query row's -D and
 *                       LSE * log2(e) are formed from o, dout and lse where the dQ pass holds
 *                       the row, stored into the workspace with the bits fa_bwd_preprocess
 *                       stores, and used there; then dq is written.  It may take the place of
 *                       the two in any order above (for FA_FP32 it enqueues the two).
 *   fa_bwd_postprocess: sums the dK/dV partials (over each query-head group and query-range
 *                       piece) into dk/dv; where fa_bwd_dkdv wrote dk/dv it enqueues nothing.
 */
enum fa_bwd_plan_kind {
  FA_BWD_PLAN_STAGES = 0, /* fa_bwd_preprocess, fa_bwd_dkdv, fa_bwd_dq, fa_bwd_postprocess */
  FA_BWD_PLAN_ROWS = 1    /* fa_bwd_dq_rows, fa_bwd_dkdv */
};
/*
 * The order fa_bwd enqueues for a problem: FA_BWD_PLAN_ROWS for 16-bit tensors whose dK/dV
 * pass writes dk and dv directly (the dQ pass goes first and forms the row values, one launch
 * fewer), else FA_BWD_PLAN_STAGES.  For arguments fa_bwd would reject, the negated status.
 */
int fa_bwd_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D, int dtype);
int fa_bwd_preprocess(const void* o, const void* dout, const float* lse, void* workspace,
                      size_t workspace_bytes, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D,
                      int dtype, void* stream);
int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dv,
                void* workspace, size_t workspace_bytes, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                int64_t D, float softmax_scale, int causal, int dtype, void* stream);
int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout, void* dq,
              void* workspace, size_t workspace_bytes, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
              int64_t D, float softmax_scale, int causal, int dtype, void* stream);
int fa_bwd_dq_rows(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* workspace, size_t workspace_bytes, int64_t B,
                   int64_t Hq, int64_t Hkv, int64_t N, int64_t D, float softmax_scale, int causal,
                   int dtype, void* stream);
int fa_bwd_postprocess(void* dk, void* dv, void* workspace, size_t workspace_bytes,
                       int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D, int dtype,
                       void* stream);

/*
 * Backward that allocates nothing and takes no workspace: for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, outputs, errors and kernels as fa_bwd, whose workspace here is
 * a device array inside the library: FA_NOALLOC_SCRATCH_BYTES (80 MiB) on each GPU the library
 * runs on, held until the process ends.  Its address is resolved on the first call on a device
 * (the stream's device, or the current one for a NULL stream); a failure to resolve it is
 * FA_ERR_HIP.  A call whose fa_bwd_workspace_size(...) exceeds the array returns FA_ERR_SCRATCH
 * and enqueues nothing.  Every call on one GPU shares that GPU's array, and the kernels write
 * every part of it they read before reading it (no part needs to start at zero): calls that may
 * overlap on one GPU (different streams, or graphs replayed concurrently) race and must be
 * ordered by the caller.
 */
#define FA_NOALLOC_SCRATCH_BYTES (80u * 1024u * 1024u)
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                   int64_t N, int64_t D, float softmax_scale, int causal, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_FA_H */
