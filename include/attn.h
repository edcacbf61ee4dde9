/*
 * attn.h - C ABI of the MI355X (gfx950) fused scaled-dot-product attention
 * library: forward and backward, dense [B,H,N,D] and packed-THD varlen.
 *
 * What is computed follows the NVIDIA NeMo-Automodel API pages:
 *  - "ffpa_attention" page, API entries of the dense forward/backward and the
 *    varlen forward/backward wrappers: the forward returns out (query rows,
 *    value head dim) and an fp32 log-sum-exp, handles GQA inside; the backward
 *    takes the caller's out/lse (so a ring can feed a globally merged pair) and
 *    returns dq, dk, dv with dk/dv reduced to the Hkv heads.
 *  - "fa4" page, module overview (document-causal bullets): the causal mask is
 *    aligned to the bottom-right corner of each segment, so query i of a
 *    segment with lq queries and lk keys sees keys j <= i + (lk - lq);
 *    zero-query segments are allowed and let key segments tile the keys.
 *  - "gemma4_moe cp_attention" page, -inf-safe merge entry: two partial
 *    results of the same queries combine as lse = logaddexp(lse_a, lse_b),
 *    out = weighted mean with weights exp(lse_x - lse); a row where both are
 *    -inf keeps out 0.
 *
 * Conventions shared by every entry point
 *  - dtype: the element type of q, k, v, out, dout, dq, dk, dv: ATTN_BF16 or
 *    ATTN_F16 (the "ffpa_attention" page's module overview routes both), the
 *    same for every tensor of a call. Products accumulate in fp32; outputs are
 *    rounded to nearest even. lse is always fp32.
 *  - lse is the natural log of the sum of exp over the *scaled* scores
 *    (scale * q.k). A query row with no visible key gets out = 0 and
 *    lse = -inf; the backward treats lse = -inf as "row attends nothing".
 *  - scale must be finite and non-zero (ATTN_E_INVALID otherwise).
 *  - GQA: Hq must be a multiple of Hkv; q-head h reads kv-head h / (Hq/Hkv).
 *  - Head dims: (Dqk, Dv) must be one of the pairs attn_is_supported()
 *    accepts: (64,64), (128,128), (192,128), (256,256), (512,512).
 *  - Strides are in elements; the innermost (head-dim) stride must be 1, every
 *    other stride a multiple of 8, and every tensor pointer 16-byte aligned.
 *  - Every output element is written (callers need not pre-zero): empty rows
 *    get out 0 / lse -inf; keys no query sees get dk = dv = 0.
 *  - Ownership: the caller allocates every buffer (inputs, outputs and the
 *    workspace). The library allocates no device memory and keeps no state
 *    between calls. Calls enqueue work on `stream` (a hipStream_t; NULL is
 *    the default stream) and return; buffers must stay valid until the
 *    stream reaches that point. Results are deterministic: the same inputs
 *    give bitwise-identical outputs (no floating-point atomics).
 *  - Workspace: a call with workspace == NULL and workspace_bytes != NULL is a
 *    size query: the required size is written to *workspace_bytes and nothing
 *    is launched. Otherwise a call that needs workspace must get a 16-byte
 *    aligned buffer with *workspace_bytes >= the required size, else
 *    ATTN_E_WORKSPACE. The workspace holds no result and may be reused once
 *    the stream has passed the call.
 *  - Errors: problems visible on the host return a negative status before any
 *    launch, and attn_last_error() describes the last one on this thread.
 *    Malformed cu_seqlens contents (not monotone, not ending at T) give
 *    unspecified values but every access stays inside [0, T); setting the
 *    environment variable ATTN_VALIDATE=1 makes the varlen calls copy
 *    cu_seqlens to the host (synchronously) and reject them as ATTN_E_INVALID.
 */
#ifndef VCA_ATTN_H
#define VCA_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ATTN_OK = 0,
  ATTN_E_INVALID = -1,     /* bad argument (NULL, size, stride, alignment, GQA) */
  ATTN_E_UNSUPPORTED = -2, /* valid but not compiled: dtype or head-dim pair */
  ATTN_E_WORKSPACE = -3,   /* workspace smaller than required */
  ATTN_E_HIP = -4          /* a HIP runtime call failed; text has hipGetErrorString */
};

enum { ATTN_BF16 = 0, ATTN_F32 = 1, ATTN_F16 = 2 };

/* Backward flags. ATTN_DQ_ACCUMULATE: dq += this call's dq (the sum is taken
 * in fp32 and rounded once to bf16), so per-chunk backward passes of one
 * query shard sum their dq in place, as a ring's local dq sum does
 * ("gemma4_moe cp_attention" page, FFPA ring backward entries). */
enum { ATTN_DQ_ACCUMULATE = 1 };

/* Text of the last non-zero status returned on the calling thread ("" if none). */
const char* attn_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int attn_version(void);

/* 1 if (dtype, Dqk, Dv) is compiled in, else 0. Analogue of the readiness
 * probes on the "ffpa_attention" page (varlen/low-level "ready" functions). */
int attn_is_supported(int dtype, int dqk, int dv);

/* Dense forward ("ffpa_attention" page, dense forward entry).
 *  q   [B, Hq,  Nq, Dqk]   k [B, Hkv, Nk, Dqk]   v [B, Hkv, Nk, Dv]
 *  out [B, Hq,  Nq, Dv]  (written)    lse [B, Hq, Nq] fp32 contiguous (written)
 *  strides[12] = element strides (b, h, n) of q, k, v, out, in that order
 *  (so both BHND- and BSHD-contiguous storage work). Nq may differ from Nk;
 *  with causal = 1 the mask is bottom-right aligned (query i sees keys
 *  j <= i + Nk - Nq). Needs a small workspace (the call's list of query
 *  tiles, segment by segment with each one's heaviest tile first); query
 *  its size with workspace = NULL. */
int attn_fwd_dense(int dtype, const void* q, const void* k, const void* v, void* out,
                   float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int Dqk, int Dv,
                   const int64_t* strides, float scale, int causal, void* workspace,
                   size_t* workspace_bytes, hipStream_t stream);

/* Varlen forward on packed THD tensors ("ffpa_attention" page, varlen forward
 * entry, returning out[T,Hq,D] and lse[Hq,T]).
 *  q [Tq, Hq, Dqk]  k [Tk, Hkv, Dqk]  v [Tk, Hkv, Dv]  out [Tq, Hq, Dv]
 *  lse [Hq, Tq] fp32 contiguous.
 *  cu_q, cu_k: device int32 [num_segments + 1]; segment s pairs query rows
 *  cu_q[s]..cu_q[s+1] with key rows cu_k[s]..cu_k[s+1]. Required:
 *  cu_q[0] = cu_k[0] = 0, non-decreasing, cu_q[S] = Tq, cu_k[S] = Tk.
 *  Zero-query and zero-key segments are allowed.
 *  max_q, max_k: host upper bounds of the per-segment lengths.
 *  strides[8] = element strides (t, h) of q, k, v, out.
 *  Needs a workspace (the heavy-first work list built on the device from
 *  cu_seqlens); query its size with workspace = NULL. */
int attn_fwd_varlen(int dtype, const void* q, const void* k, const void* v, void* out,
                    float* lse, const int32_t* cu_q, const int32_t* cu_k, int num_segments,
                    int max_q, int max_k, int Tq, int Tk, int Hq, int Hkv, int Dqk, int Dv,
                    const int64_t* strides, float scale, int causal, void* workspace,
                    size_t* workspace_bytes, hipStream_t stream);

/* The varlen forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): same arguments, results and errors as attn_fwd_varlen, without
 * a workspace. The work list lives in a static device array of
 * 256 + 8 * ATTN_NOALLOC_MAX_ITEMS bytes (4 MiB) that the library holds on
 * every GPU it runs on until the process ends; the call allocates nothing.
 * It needs ceil(Tq / 32) + num_segments <= ATTN_NOALLOC_MAX_ITEMS, else
 * ATTN_E_WORKSPACE before any launch. Every call on one GPU shares that
 * GPU's array and the array keeps the last call's contents: calls that
 * overlap on one GPU (e.g. on two streams without ordering) race and give
 * wrong results; calls ordered on one stream are safe. */
#define ATTN_NOALLOC_MAX_ITEMS 524256
int attn_fwd_varlen_noalloc(int dtype, const void* q, const void* k, const void* v, void* out,
                            float* lse, const int32_t* cu_q, const int32_t* cu_k,
                            int num_segments, int max_q, int max_k, int Tq, int Tk, int Hq,
                            int Hkv, int Dqk, int Dv, const int64_t* strides, float scale,
                            int causal, hipStream_t stream);

/* Dense backward from the caller's out/lse ("ffpa_attention" page, dense
 * backward entry). dout, out [B,Hq,Nq,Dv]; lse [B,Hq,Nq] fp32 contiguous;
 * dq [B,Hq,Nq,Dqk]; dk [B,Hkv,Nk,Dqk]; dv [B,Hkv,Nk,Dv] (dk/dv summed over the
 * q-heads of each GQA group).
 * strides[24] = (b, h, n) strides of q, k, v, out, dout, dq, dk, dv.
 * Needs a workspace (query it with workspace = NULL). flags: ATTN_DQ_*.
 * Head dims 128 and 192/128: the workspace also holds the dS blocks of the
 * q-heads of one launch pair (the dK/dV pass stores them, the dQ pass
 * multiplies them by K instead of recomputing S and dP), at most
 * ATTN_BWD_DS_MIB MiB (environment variable, default 8192; 0 turns the store
 * off); when one GQA group's blocks exceed it, the dQ pass recomputes.
 * Head dims 256 and 512 (two-phase backward): the workspace holds the bf16 P
 * and dS blocks of as many 256-query row slots as fit in ATTN_BWD_TILES_MIB
 * MiB (environment variable, default 8192; at least one slot, whose size
 * grows with the key length only); more slots run as consecutive chunks,
 * and the workspace then also holds fp32 dK/dV accumulators (4 bytes x key
 * rows x Hkv x (Dqk + Dv)). The workspace size query reports the total. */
int attn_bwd_dense(int dtype, const void* dout, const void* q, const void* k, const void* v,
                   const void* out, const float* lse, void* dq, void* dk, void* dv, int B,
                   int Hq, int Hkv, int Nq, int Nk, int Dqk, int Dv, const int64_t* strides,
                   float scale, int causal, int flags, void* workspace,
                   size_t* workspace_bytes, hipStream_t stream);

/* Varlen backward from the caller's out/lse ("ffpa_attention" page, varlen
 * backward entry, returning (dq, dk, dv)). Shapes as in attn_fwd_varlen, with
 * dq [Tq,Hq,Dqk], dk [Tk,Hkv,Dqk], dv [Tk,Hkv,Dv].
 * strides[16] = (t, h) strides of q, k, v, out, dout, dq, dk, dv. */
int attn_bwd_varlen(int dtype, const void* dout, const void* q, const void* k, const void* v,
                    const void* out, const float* lse, void* dq, void* dk, void* dv,
                    const int32_t* cu_q, const int32_t* cu_k, int num_segments, int max_q,
                    int max_k, int Tq, int Tk, int Hq, int Hkv, int Dqk, int Dv,
                    const int64_t* strides, float scale, int causal, int flags,
                    void* workspace, size_t* workspace_bytes, hipStream_t stream);

/* Left sliding window and logit softcap: the four calls above with one more
 * argument, ext (the "attention utils" page, window argument of its
 * mask helpers: a positive left window counts the keys a query sees, its own
 * position included; the "ffpa_attention" page, softcap argument of the
 * forward entries, which that page pins off).
 *  ext->window: 0 = none. W > 0 (only with causal = 1, else ATTN_E_INVALID):
 *  query i of a segment with lq queries and lk keys sees keys j with
 *  i + (lk - lq) - W < j <= i + (lk - lq), its W most recent keys.
 *  ext->softcap: 0 = none. c > 0: every scaled score x = scale * q.k is
 *  replaced by c * tanh(x / c) before the softmax; lse is taken over the
 *  capped scores, and the backward applies the chain factor
 *  1 - tanh^2(x / c) to dS.
 *  Negative window, negative or non-finite softcap: ATTN_E_INVALID. ext =
 *  NULL (or both fields 0) is exactly the plain call. The backward of a
 *  problem must get the ext its forward got (its lse depends on it). With ext
 *  set, the backward takes the generic dK/dV kernel at every head dim (the
 *  software-pipelined ones are compiled without the options); the workspace
 *  size is that of the plain call. */
typedef struct attn_ext {
  int window;
  float softcap;
} attn_ext;
int attn_fwd_dense_ex(int dtype, const void* q, const void* k, const void* v, void* out,
                      float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int Dqk, int Dv,
                      const int64_t* strides, float scale, int causal, const attn_ext* ext,
                      void* workspace, size_t* workspace_bytes, hipStream_t stream);
int attn_fwd_varlen_ex(int dtype, const void* q, const void* k, const void* v, void* out,
                       float* lse, const int32_t* cu_q, const int32_t* cu_k, int num_segments,
                       int max_q, int max_k, int Tq, int Tk, int Hq, int Hkv, int Dqk, int Dv,
                       const int64_t* strides, float scale, int causal, const attn_ext* ext,
                       void* workspace, size_t* workspace_bytes, hipStream_t stream);
int attn_bwd_dense_ex(int dtype, const void* dout, const void* q, const void* k, const void* v,
                      const void* out, const float* lse, void* dq, void* dk, void* dv, int B,
                      int Hq, int Hkv, int Nq, int Nk, int Dqk, int Dv, const int64_t* strides,
                      float scale, int causal, const attn_ext* ext, int flags, void* workspace,
                      size_t* workspace_bytes, hipStream_t stream);
int attn_bwd_varlen_ex(int dtype, const void* dout, const void* q, const void* k, const void* v,
                       const void* out, const float* lse, void* dq, void* dk, void* dv,
                       const int32_t* cu_q, const int32_t* cu_k, int num_segments, int max_q,
                       int max_k, int Tq, int Tk, int Hq, int Hkv, int Dqk, int Dv,
                       const int64_t* strides, float scale, int causal, const attn_ext* ext,
                       int flags, void* workspace, size_t* workspace_bytes, hipStream_t stream);

/* Online-softmax merge of two partial results of the same query rows
 * ("gemma4_moe cp_attention" page, -inf-safe merge entry).
 *  out_a, out_b: [rows, H, Dv] contiguous, element type dtype_a / dtype_b
 *  (ATTN_BF16, ATTN_F32 or ATTN_F16); lse_a, lse_b: [H, rows] fp32.
 *  out: [rows, H, Dv] fp32 (written); lse: [H, rows] fp32 (written);
 *  out_copy: optional (may be NULL) copy of out in copy_dtype (ATTN_BF16 or
 *  ATTN_F16), RNE, for feeding the backward. out may alias out_a when dtype_a
 *  is ATTN_F32, and lse may alias lse_a (running-accumulator use). Rows where
 *  both lse are -inf get out 0 and lse -inf. No workspace. */
int attn_merge(const void* out_a, int dtype_a, const float* lse_a, const void* out_b,
               int dtype_b, const float* lse_b, float* out, float* lse, void* out_copy,
               int copy_dtype, int rows, int H, int Dv, hipStream_t stream);

/* Document-causal segment layout ("fa4" page, module overview and the
 * _varlen_segments / _varlen_layout entries). Host-only, no GPU work.
 *  doc_ids: host int32 [B, S] document ids of each row (1-based, 0 = padding).
 *  Queries are the positions [q_start, q_start + q_len) of every row; keys
 *  are the positions [k_start, k_start + k_len).
 *  mode 0 (causal, keys cover the queries: k_start <= q_start and
 *  q_start + q_len <= k_start + k_len): every run of equal ids is split at the
 *  query-shard end; a piece that overlaps the shard pairs its queries with all
 *  of its keys (bottom-right causal gives "query at p sees its document's keys
 *  up to p"); pieces without queries become zero-query segments. Padding
 *  (id 0) pieces become a query-only segment followed by a key-only segment,
 *  so padding neither attends nor is attended.
 *  mode 1 (cross, keys entirely before the queries: k_start + k_len <=
 *  q_start; run the result with causal = 0): one segment per run in order of
 *  position, pairing a document's queries with its keys in the key range;
 *  unshared runs get zero queries or zero keys.
 *  Outputs (host int32): seg_q[max_segments], seg_k[max_segments] lengths in
 *  flattened row-major order; *num_segments receives the count. Segment
 *  query lengths tile the B*q_len queries and key lengths the B*k_len keys.
 *  Returns ATTN_E_INVALID on bad ranges or when max_segments is too small
 *  (then *num_segments holds the count needed). */
int attn_doc_segments(const int32_t* doc_ids, int B, int S, int q_start, int q_len,
                      int k_start, int k_len, int mode, int32_t* seg_q, int32_t* seg_k,
                      int max_segments, int* num_segments);

/* The attn_doc_segments layout as cumulative offsets, ready for the varlen
 * calls (host-only, no GPU work): cu_q, cu_k (host int32, room for
 * max_segments + 1 entries) receive cu_x[0] = 0 and cu_x[s + 1] = cu_x[s] +
 * the length of segment s; *num_segments the segment count; *max_q / *max_k
 * the longest query / key segment (the max_q / max_k arguments of the varlen
 * calls). Same arguments, modes and errors as attn_doc_segments. */
int attn_doc_cu_seqlens(const int32_t* doc_ids, int B, int S, int q_start, int q_len,
                        int k_start, int k_len, int mode, int32_t* cu_q, int32_t* cu_k,
                        int max_segments, int* num_segments, int* max_q, int* max_k);

/* Dense routing of one ring chunk ("gemma4_moe cp_attention" page: the
 * dense-routing flags of the packed ring segments and the per-chunk dense
 * eligibility entry). Host-only, no GPU work. Same doc_ids, ranges and modes
 * as attn_doc_segments. *eligible receives 1 when the chunk can run on the
 * dense kernels over the raw [B, H, S, D] rows (queries = positions
 * [q_start, q_start + q_len), keys = [k_start, k_start + k_len); causal for
 * mode 0, non-causal for mode 1) and give the document-causal result on every
 * non-padding query:
 *  mode 0: the key range ends where the query range ends, and every row's
 *  keys are one document with padding (id 0) only as a suffix;
 *  mode 1: every row's keys are exactly one document without padding, and
 *  the row's queries are that document with padding only as a suffix (or all
 *  padding).
 * pad_rows (optional, host uint8 [B, q_len]) receives 1 for padding queries:
 * after a dense run their out rows must be zeroed and lse set to -inf
 * (attn_zero_rows), which the backward then treats as attending nothing.
 * Returns ATTN_E_INVALID on bad ranges (the attn_doc_segments conditions). */
int attn_dense_route(const int32_t* doc_ids, int B, int S, int q_start, int q_len, int k_start,
                     int k_len, int mode, uint8_t* pad_rows, int* eligible);

/* Zero the rows a dense ring chunk must not produce: for every (b, i) with
 * rows[b * S + i] != 0 (device uint8 [B, S]), out[b, h, i, :] = 0 (ATTN_BF16,
 * ATTN_F16 or ATTN_F32 per dtype) and lse[b*lse_sb + h*lse_sh + i] = -inf for
 * all H heads. out is a [B, H, S, D] view with element strides (ob, oh, on)
 * and unit innermost stride; lse may be NULL. Enqueued on stream; no
 * workspace. */
int attn_zero_rows(void* out, int dtype, int64_t ob, int64_t oh, int64_t on, float* lse,
                   int64_t lse_sb, int64_t lse_sh, const uint8_t* rows, int B, int H, int S, int D,
                   hipStream_t stream);

/* ---- Packed ring layout ("gemma4_moe cp_attention" page: per-document
 * varlen segments with flat gather indices, the [B, H, S, D] <-> packed
 * [T, H, D] row moves and their lse counterparts, the gradient scatter-add,
 * the in-place live-row merge and the in-place-versus-scatter predicate). */

/* Segments shared by a query shard and one KV chunk (host-only, no GPU work).
 *  q_ids: host int32 [B, Sq] document ids of the query shard; k_ids: [B, Sk]
 *  of the key chunk (1-based, 0 = padding). Every id > 0 found in row b of
 *  both becomes one segment: its query positions p (in order) as flat indices
 *  b*Sq + p and its key positions as b*Sk + p. Rows in order; within a row,
 *  documents in the order they first occur among the queries; ids in only one
 *  of the two, and padding, form no segment.
 *  q_index (room for B*Sq), k_index (room for B*Sk): host int32 gather
 *  indices; cu_q, cu_k (room for max_segments + 1): cumulative offsets into
 *  them (cu_q[i] pairs cu_k[i]). *num_segments (0: no shared document),
 *  *Tq / *Tk (live tokens), *max_q / *max_k receive the layout's sizes.
 *  Run the local (causal) chunk with causal = 1 (a document's keys then end
 *  where its queries end, so bottom-right alignment is position causality
 *  when q_ids == k_ids) and a cross chunk of earlier keys with causal = 0.
 *  ATTN_E_INVALID on bad arguments or when max_segments is too small (then
 *  *num_segments holds the count needed). */
int attn_ring_segments(const int32_t* q_ids, int Sq, const int32_t* k_ids, int Sk, int B,
                       int32_t* q_index, int32_t* k_index, int32_t* cu_q, int32_t* cu_k,
                       int max_segments, int* num_segments, int* Tq, int* Tk, int* max_q,
                       int* max_k);

/* 1 when merging a chunk's live_rows packed rows in place (attn_merge_rows)
 * moves fewer HBM bytes than scattering them into a [B, H, S, D] tensor and
 * merging every row (attn_scatter_rows + attn_merge); dtype is the chunk
 * output's type. The pages give no threshold: this is the byte count of the
 * two routes with this library's kernels. Host-only. */
int attn_ring_inplace_preferred(int64_t live_rows, int64_t B, int64_t S, int H, int D, int dtype);

/* dst[t, h, :] = src[b, h, s, :] for index[t] = b*S + s (device int32 [T]):
 * src a [B, H, S, D] view with element strides (sb, sh, sn) and unit innermost
 * stride, dst contiguous [T, H, D]; dtype ATTN_BF16, ATTN_F16 or ATTN_F32;
 * dst_dtype = dtype, or ATTN_BF16 / ATTN_F16 for fp32 src (rounded to nearest
 * even, D a multiple of 8: e.g. the merged fp32 out for a chunk's backward);
 * D * element size a multiple of 16, pointers 16-byte aligned. Indices must
 * lie in [0, B*S) (the kernel does not clamp them). */
int attn_gather_rows(int dtype, const void* src, int64_t sb, int64_t sh, int64_t sn,
                     const int32_t* index, int B, int H, int S, int D, int T, void* dst,
                     int dst_dtype, hipStream_t stream);

/* The inverse move: dst view [B, H, S, D] rows index[t] receive src[t, h, :]
 * (ATTN_ROWS_ASSIGN), or every row is zeroed first (ATTN_ROWS_ASSIGN_ZERO_REST:
 * rows no index names end as 0), or src is added to them in fp32 and rounded
 * once (ATTN_ROWS_ADD: the gradient scatter-add; the indices must be distinct,
 * which attn_ring_segments guarantees). Same layout rules as
 * attn_gather_rows. */
enum { ATTN_ROWS_ASSIGN = 0, ATTN_ROWS_ASSIGN_ZERO_REST = 1, ATTN_ROWS_ADD = 2 };
int attn_scatter_rows(int dtype, const void* src, const int32_t* index, int T, int H, int D,
                      void* dst, int64_t sb, int64_t sh, int64_t sn, int B, int S, int mode,
                      hipStream_t stream);

/* lse_packed[h, t] = lse_dense[b, h, s] (both fp32 contiguous, [H, T] and
 * [B, H, S]) for index[t] = b*S + s; attn_scatter_lse writes the other way,
 * first setting every dense entry to -inf when fill_rest != 0 (rows no
 * segment covers are then "attends nothing"). */
int attn_gather_lse(const float* lse_dense, const int32_t* index, int B, int H, int S, int T,
                    float* lse_packed, hipStream_t stream);
int attn_scatter_lse(const float* lse_packed, const int32_t* index, int T, int H, float* lse_dense,
                     int B, int S, int fill_rest, hipStream_t stream);

/* In-place online-softmax merge of one chunk at its live rows: for every t
 * and head h, with (b, s) from index[t], the running fp32 accumulators
 * out_acc[b, h, s, :] (a [B, H, S, D] view, element strides sb, sh, sn) and
 * lse_acc[b, h, s] (contiguous [B, H, S]) are combined with out_b[t, h, :]
 * ([T, H, D] contiguous, dtype_b) and lse_b[h, t] ([H, T]) exactly as
 * attn_merge combines two results (both -inf: out 0, lse -inf). Rows not
 * named are untouched; indices must be distinct. */
int attn_merge_rows(float* out_acc, int64_t sb, int64_t sh, int64_t sn, float* lse_acc, int B,
                    int S, const void* out_b, int dtype_b, const float* lse_b,
                    const int32_t* index, int T, int H, int D, hipStream_t stream);

/* Opt-in kernel timing, for profiling on the caller's own streams. While
 * enabled (per calling thread), every kernel this library launches from that
 * thread is bracketed by two HIP events recorded on its stream. Returns the
 * previous setting. Disabled by default; adds two event records per launch. */
int attn_timing_enable(int enable);

/* Waits for and reads the recorded launches (in launch order) of the calling
 * thread, then clears the record. Up to max_records entries: names receives
 * NUL-terminated kernel labels in slots of name_len bytes ("attn_schedule",
 * "attn_fwd", "attn_bwd_dq", "attn_bwd_dkdv", "attn_bwd_dq_ds" (dQ from stored dS);
 * for head dims 256 and 512
 * "attn_bwd_delta", "attn_bwd_scores", "attn_bwd_dkdv_tiles",
 * "attn_bwd_dq_tiles"; "attn_merge", "attn_zero_rows", "attn_ring_rows",
 * "attn_ring_fill", "attn_ring_lse", "attn_merge_rows"), ms the elapsed
 * milliseconds; *count receives the total number recorded. Returns
 * ATTN_E_HIP if an event could not be read. */
int attn_timing_read(int max_records, char* names, int name_len, float* ms, int* count);

#ifdef __cplusplus
}
#endif

#endif /* VCA_ATTN_H */
