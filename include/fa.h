/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library libfa_mi355x.so.
 *
 * What it computes. For every batch b and head h, with Q, K, V of shape [N, d]:
 *   S = scale * Q K^T, with S_ij = -inf where key j is not visible to query i,
 *   P = softmax(S) row by row, O = P V, LSE_i = ln sum_j exp(S_ij),
 * and the gradient of L = sum(dO * O) with respect to Q, K and V.
 * "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness"
 * (summary of arXiv 2205.14135), Problem and motivation, defines S, P and O; its FAQ
 * states that the tiled method returns this same exact result; its Key ideas section
 * fixes what the backward pass gets from the forward pass (O and the softmax
 * statistics, here folded into LSE). "[Review] From Online Softmax to Flash
 * Attention", sections FlashAttention and Algorithm FlashAttention (Tiling), gives
 * the online-softmax recurrence the forward kernel runs.
 *
 * Visibility. Key j is visible to query i iff (causal == 0 || j <= i) and
 * (kv_len == NULL || j < kv_len[b]). The causal rule is the lower-triangular mask
 * tril(ones, 0) of "Fewer matrix multiplications, same results" (flash-attention
 * issue #941), diagonal included, top-left aligned; keys at or past kv_len[b] are
 * scored -inf like the out-of-range keys of the review's Triton listings.
 *
 * Layout. q, k, v, dout, o, dq, dk, dv are dense row-major [B, H, N, d] (the
 * [batch, heads, seq, head_dim] order of the issue's listing); lse is [B, H, N].
 * q, k, v and dout share one element type (dtype); o, lse, dq, dk, dv are float32.
 *
 * Pointers. Every tensor pointer is device memory owned by the caller; the library
 * keeps no pointer after a call returns. kv_len, when not NULL, is a device array
 * of B int32 values, each in [1, N] (not checked on the host: reading it would need
 * a copy). Tensor pointers must be 16-byte aligned, lse and kv_len 4-byte aligned.
 * Outputs must not overlap inputs or each other (checked). The library allocates
 * nothing and keeps no state between calls; calls are thread-safe.
 *
 * Streams. `stream` is a hipStream_t (NULL: the null stream). Every entry point
 * only validates on the host and enqueues; it returns before the GPU work ends, and
 * a device fault shows up at the caller's next synchronisation.
 *
 * Errors. Entry points return FA_OK or an error code; on error nothing has been
 * enqueued and fa_last_error() (thread-local) says why.
 *
 * Limits. d in {64, 128}; scale finite and > 0; B, H, N >= 0 (a zero size makes
 * the call a no-op); B*H*N*d < 2^40; N <= 2^22. bf16/f16 inputs are read exactly;
 * internally P and dS are rounded to fp16 for the matrix cores, and bf16 operands
 * they multiply are converted to fp16, which is exact when every |x| of V, dO, Q and
 * K lies in [2^-14, 65504] or is 0 (smaller magnitudes lose low bits).
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define FA_API __attribute__((visibility("default")))
#else
#define FA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and dout. */
enum fa_dtype { FA_F32 = 0, FA_BF16 = 1, FA_F16 = 2 };

/* Status codes. */
enum fa_status {
  FA_OK = 0,
  FA_EINVAL = 1,        /* null pointer, bad size, misalignment, overlap, bad scale */
  FA_EUNSUPPORTED = 2,  /* head_dim or dtype the library has no kernel for */
  FA_EWORKSPACE = 3,    /* backward workspace missing or too small */
  FA_EHIP = 4           /* the HIP runtime reported an error at launch */
};

/*
 * Forward pass. Writes o [B,H,N,d] float32 (O = P V) and lse [B,H,N] float32
 * (natural-log log-sum-exp of the scaled, masked scores of each query row).
 * The N x N score matrix never leaves the chip: each workgroup keeps a block of
 * query rows and streams key/value tiles through the online-softmax recurrence
 * (running row maximum, running denominator, rescaled output accumulator).
 */
FA_API int fa_fwd(const void* q, const void* k, const void* v, float* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, int dtype,
           const int32_t* kv_len, void* stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes: the per-row
 * D_i = sum_k dO_ik O_ik (float32 [B,H,N]) and then the largest |dO| of every group of
 * 32 query rows (float32 [B,H,ceil(N/32)]), each region rounded up to 256 bytes.
 */
FA_API size_t fa_bwd_workspace_size(int B, int H, int N, int d);

/*
 * Backward pass of L = sum(dout * O). Inputs: q, k, v, dout (dtype), o and lse
 * exactly as fa_fwd wrote them for the same q, k, v, scale, causal and kv_len.
 * Outputs (float32, overwritten): dq, dk, dv [B,H,N,d]. The scores and
 * probabilities are recomputed on chip from q, k and lse, tile by tile.
 * workspace: device memory of at least fa_bwd_workspace_size(B,H,N,d) bytes,
 * 256-byte aligned, owned by the caller, contents on entry irrelevant.
 * Two kernels run in order on `stream`: dq (queries outer), which also forms
 * D = rowsum(dout*o) for its rows and the 32-row maxima of |dout| and writes them into
 * the workspace, then dk/dv (keys outer), which reads them; each output is written
 * exactly once, so results are deterministic. dtype FA_BF16, FA_F16 or FA_F32.
 * Precision (FA_F32): every product runs on the fp32 matrix cores in fp32, P and dS
 * included; the result matches the definition to fp32 rounding.
 * Precision (FA_BF16, FA_F16): the matrix-core products run on fp16 operands with fp32
 * accumulation.
 * dout is multiplied by a power of two (per query row in the dq kernel, per workgroup
 * from the 32-row maxima in the dk/dv kernel) that brings its largest magnitude into
 * [1, 2) before rounding, and the gradients are divided by it exactly at the end, so
 * the relative precision does not depend on the magnitude of dout. q, k and v are
 * rounded to fp16 as they are: their magnitudes must stay within the fp16 range
 * (|x| <= 65504; values below 2^-14 lose relative precision).
 */
FA_API int fa_bwd(const void* q, const void* k, const void* v, const float* o,
           const void* dout, const float* lse, float* dq, float* dk, float* dv,
           int B, int H, int N, int d, float scale, int causal, int dtype,
           const int32_t* kv_len, void* workspace, size_t workspace_bytes,
           void* stream);

/*
 * Split-KV (key axis cut into ranges, partials merged afterwards).
 * "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness"
 * (summary of arXiv 2205.14135), Method, incremental softmax tracking: the softmax
 * statistics of a vector split into parts combine as m = max(m1, m2),
 * l = e^{m1-m} l1 + e^{m2-m} l2, and the block outputs are rescaled by the same
 * factors. Computing each key range's block on its own and merging with this rule
 * gives the unsplit result (up to rounding): more workgroups for few query rows and
 * long key sequences, and the per-shard half of a sequence-parallel layout.
 *
 * fa_split_count: number of key ranges of split_len keys covering N keys,
 * ceil(N / split_len); -1 when split_len is not a positive multiple of 64.
 */
FA_API int fa_split_count(int N, int split_len);

/*
 * fa_split_hint: the split_len for which fa_fwd_partial + fa_merge is expected to beat
 * fa_fwd on this device for a problem of this shape, or 0 when fa_fwd should run
 * unsplit (the split itself is the combination rule above; when to split is not on
 * the pages: the rule below is measured on the MI355X). Counting query-block
 * workgroups of 256 rows at head_dim 128 and of the forward's own size at 64, a split
 * is recommended when they are at most half the compute units (two splits) or, under
 * the causal mask, at most one per compute unit (four splits), halving the count until
 * every split holds at least 2048 keys (1024 under the causal mask); f32 and N < 2048
 * always give 0. Host only: reads the current device's compute-unit count once per
 * process (256 if none is visible) and launches nothing. Arguments as fa_fwd (scale not
 * taken); B, H, N, d or dtype that fa_fwd would reject give the negated status
 * (-FA_EINVAL or -FA_EUNSUPPORTED; fa_last_error says which).
 */
FA_API int fa_split_hint(int B, int H, int N, int d, int causal, int dtype);

/*
 * The forward pass with the split chosen for it: fa_fwd when fa_split_hint gives 0 (or
 * workspace is NULL), otherwise fa_fwd_partial with that split_len into the workspace
 * followed by fa_merge into o and lse, which gives fa_fwd's O and LSE up to rounding (the
 * combination rule above). fa_fwd_workspace_size: the bytes the split needs, the
 * partials of n_splits = fa_split_count(N, split_len) ranges (0 when there is no split;
 * also 0 for arguments fa_fwd would reject). The workspace is caller-owned device
 * memory, 256-byte aligned, not overlapping any input or output; smaller than
 * fa_fwd_workspace_size gives FA_EINVAL. Other arguments, limits and errors as fa_fwd,
 * fa_fwd_partial and fa_merge; both kernels go to `stream` in that order.
 */
FA_API size_t fa_fwd_workspace_size(int B, int H, int N, int d, int causal, int dtype);
FA_API int fa_fwd_auto(const void* q, const void* k, const void* v, float* o, float* lse,
                int B, int H, int N, int d, float scale, int causal, int dtype,
                const int32_t* kv_len, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * Partial forward pass over key ranges. Range p holds keys
 * [p*split_len, min(N, (p+1)*split_len)); visibility inside it is the usual one
 * (causal, kv_len). For each range p and query row, writes the normalised partial
 * output o_part[p] = P_p V over the range's visible keys and lse_part[p] = ln of the
 * sum of exp over them; a row that sees no key of the range gets o_part = 0 and
 * lse_part = -inf. o_part is float32 [n_splits, B, H, N, d], lse_part float32
 * [n_splits, B, H, N], n_splits = fa_split_count(N, split_len); both caller-owned,
 * 16- and 4-byte aligned, not overlapping the inputs or each other. split_len must
 * be a positive multiple of 64 (FA_EINVAL otherwise). dtype FA_BF16 or FA_F16
 * (FA_F32: FA_EUNSUPPORTED). Other arguments, limits and errors as fa_fwd.
 */
FA_API int fa_fwd_partial(const void* q, const void* k, const void* v, float* o_part,
                   float* lse_part, int B, int H, int N, int d, float scale, int causal,
                   int dtype, const int32_t* kv_len, int split_len, void* stream);

/*
 * Merge of n_splits partials (o_part [n_splits,B,H,N,d], lse_part [n_splits,B,H,N],
 * float32, as fa_fwd_partial writes them) into o [B,H,N,d] and lse [B,H,N]:
 *   m = max_p lse_part[p], lse = m + ln sum_p e^{lse_part[p] - m},
 *   o = sum_p e^{lse_part[p] - lse} o_part[p];
 * a row whose every lse_part is -inf gets o = 0, lse = -inf. Any partials with this
 * meaning may be merged (for instance partials of key shards computed elsewhere).
 * n_splits in [1, 65536]; d in {64, 128}; o_part/o 16-byte aligned, lse_part/lse
 * 4-byte aligned; outputs must not overlap inputs or each other. Errors as fa_fwd.
 */
FA_API int fa_merge(const float* o_part, const float* lse_part, float* o, float* lse,
             int n_splits, int B, int H, int N, int d, void* stream);

/*
 * Block-sparse attention.
 * "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness"
 * (summary of arXiv 2205.14135), Extension: Block-Sparse FlashAttention: with a fixed
 * sparsity mask M in {0,1}^{(N/Br) x (N/Bc)} only the nonzero blocks are evaluated, and
 * the HBM traffic falls with the fraction s of nonzero blocks. Here Br = Bc =
 * FA_SPARSE_BLOCK and block_mask is a device array of ceil(N/128)^2 bytes, row-major
 * [query block][key block], shared by every batch and head; a zero entry hides every
 * key of that key block from every query of that query block, on top of the causal and
 * kv_len rules. The result equals dense attention with those scores set to -inf; a
 * query row that sees no key at all gets o = 0 and lse = -inf (and zero gradients).
 * Zero blocks are skipped: their K/V (forward, dq) or Q/dO (dk/dv) tiles are neither
 * loaded nor multiplied. N <= FA_SPARSE_MAX_N; dtype FA_BF16 or FA_F16; other
 * arguments, layouts and errors as fa_fwd / fa_bwd (o and lse passed to fa_bwd_sparse
 * come from fa_fwd_sparse with the same mask).
 */
#define FA_SPARSE_BLOCK 128
#define FA_SPARSE_MAX_N (1 << 18)

FA_API int fa_fwd_sparse(const void* q, const void* k, const void* v, float* o, float* lse,
                  int B, int H, int N, int d, float scale, int causal, int dtype,
                  const int32_t* kv_len, const uint8_t* block_mask, void* stream);

FA_API int fa_bwd_sparse(const void* q, const void* k, const void* v, const float* o,
                  const void* dout, const float* lse, float* dq, float* dk, float* dv,
                  int B, int H, int N, int d, float scale, int causal, int dtype,
                  const int32_t* kv_len, const uint8_t* block_mask, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * fa_bwd without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * The scratch fa_bwd keeps in the workspace (D and the 32-row maxima of |dout|) lives in
 * a statically allocated device array of FA_NOALLOC_SCRATCH_BYTES on every GPU the
 * library runs on, held until the process ends; the call allocates and frees nothing.
 * Sizes whose fa_bwd_workspace_size exceeds FA_NOALLOC_SCRATCH_BYTES are rejected with
 * FA_EWORKSPACE (B*H*N up to about 8.1 million rows fit). Every call on one GPU shares
 * that GPU's array, whose contents need no clearing (each call writes every element it
 * reads before reading it): calls that overlap in time on one GPU (two streams, two host
 * threads) race on it and must be serialised by the caller. Other arguments, outputs,
 * errors and results are those of fa_bwd, bit for bit.
 */
#define FA_NOALLOC_SCRATCH_BYTES (32 << 20)
FA_API int fa_bwd_noalloc(const void* q, const void* k, const void* v, const float* o,
                   const void* dout, const float* lse, float* dq, float* dk, float* dv,
                   int B, int H, int N, int d, float scale, int causal, int dtype,
                   const int32_t* kv_len, void* stream);

/*
 * One stage of the backward pass, into caller-allocated outputs: stage 0 writes
 * D = rowsum(dout * o) and the 32-row maxima of |dout| into the workspace; stage 1
 * writes dk and dv (reads both); stage 2 writes dq (it forms D for its own rows from
 * dout and o, and reads nothing from the workspace); stage 3 is stage 2 that also writes
 * D and the maxima into the workspace. fa_bwd is
 * stage 3 then stage 1 on one stream; stages 0, 1, 2 in that order give the same
 * results bit for bit (both ways of forming D sum in the same order). After stage 0,
 * stages 1 and 2 are independent and may run on two streams. Arguments, checks and
 * errors are those of fa_bwd (every pointer is validated even where the stage does not
 * touch it); stage outside 0..3 is FA_EINVAL.
 */
FA_API int fa_bwd_stage(int stage, const void* q, const void* k, const void* v,
                 const float* o, const void* dout, const float* lse, float* dq, float* dk,
                 float* dv, int B, int H, int N, int d, float scale, int causal, int dtype,
                 const int32_t* kv_len, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * Attention with dropout on the probabilities.
 * "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness"
 * (summary of arXiv 2205.14135): Key ideas (kernel fusion) fuses dropout into the one
 * attention kernel, and the FAQ on recomputation has the backward pass regenerate the
 * dropout mask on chip from the stored state of the random generator instead of reading
 * it from HBM. The pages name no generator; this library uses Philox4x32-10 (Salmon,
 * Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC11) under the key
 * (seed mod 2^32, seed >> 32). Keys fall in groups of 32: for element (batch b, head h,
 * query i, key j = 32 g + u) the random byte is byte 8*(u/16) + u%8 (little-endian over
 * the four 32-bit output words) of the block at counter (i, 2g + (u/8)%2, b*H + h,
 * offset). With t = fa_dropout_threshold(p) an element is kept iff its byte >= t, and
 * kept probabilities are scaled by 256 / (256 - t):
 *   o = (P * Z * 256/(256 - t)) v, lse = log-sum-exp of the undropped scaled scores.
 * fa_bwd_dropout computes the gradients of that o with the same mask (same p, seed and
 * offset; o and lse from fa_fwd_dropout). p must lie in [0, 1) (else FA_EINVAL); p = 0
 * gives t = 0 and exactly fa_fwd / fa_bwd. dtype FA_BF16 or FA_F16 (FA_F32 is
 * FA_EUNSUPPORTED); other arguments, layouts and errors as fa_fwd / fa_bwd. The mask is
 * a pure function of (seed, offset, b*H + h, i, j): calls with the same key reproduce it,
 * whatever the launch order.
 */
/*
 * The byte threshold t of dropout probability p: the t in [0, 255] whose keep probability
 * (256 - t)/256 lies nearest to 1 - p on the 1/256 grid (t = floor(256 p + 1/2) evaluated
 * in double precision from the float p, capped at 255), or -1 when p is not in [0, 1).
 * Host-only and pure; the dropout entry points derive their mask threshold with it.
 */
FA_API int fa_dropout_threshold(float p);

FA_API int fa_fwd_dropout(const void* q, const void* k, const void* v, float* o, float* lse,
                   int B, int H, int N, int d, float scale, int causal, int dtype,
                   const int32_t* kv_len, float p, uint64_t seed, uint32_t offset,
                   void* stream);

FA_API int fa_bwd_dropout(const void* q, const void* k, const void* v, const float* o,
                   const void* dout, const float* lse, float* dq, float* dk, float* dv,
                   int B, int H, int N, int d, float scale, int causal, int dtype,
                   const int32_t* kv_len, float p, uint64_t seed, uint32_t offset,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward pass with the P V product deferred to the end of the key row (an ablation).
 * "Fewer matrix multiplications, same results, should we consider adopting it?"
 * (flash-attention issue thread): per query block the numerator blocks of the whole key
 * row are kept on chip (earlier blocks rescaled when the running maximum rises) and the
 * output is one product with V at the end, instead of an output update per key block.
 * The thread's objection is the on-chip room for a query block's whole numerator row:
 * here it lives in registers, so N <= FA_DEFERRED_MAX_N. The result is the same exact
 * attention as fa_fwd: same arguments, layouts, outputs and errors, dtype FA_BF16 or
 * FA_F16 (FA_F32 is FA_EUNSUPPORTED), N > FA_DEFERRED_MAX_N is FA_EINVAL.
 */
#define FA_DEFERRED_MAX_N 512

FA_API int fa_fwd_deferred(const void* q, const void* k, const void* v, float* o, float* lse,
                    int B, int H, int N, int d, float scale, int causal, int dtype,
                    const int32_t* kv_len, void* stream);

/* Static description of a status code. */
FA_API const char* fa_status_str(int status);

/* Detail of the last error returned on this thread ("" when none). */
FA_API const char* fa_last_error(void);

/* Library version: major*10000 + minor*100 + patch. */
FA_API int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
