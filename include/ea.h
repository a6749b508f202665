/*
 * ea.h -- C ABI of libea.so: hybrid-head prefill attention (Elastic Attention)
 * for AMD Instinct MI355X (gfx950).
 *
 * One layer of causal prefill attention in which every KV head of every
 * sequence runs in the mode an external router assigned to it:
 *   FA  = full causal softmax attention (Eq. 1 of the Elastic Attention
 *         paper-reading notes, "02 . Background"),
 *   SSA = streaming sparse attention: attention sink plus sliding window
 *         (glossary of the notes; Table 8 gives sink/local 128/2048),
 *   XA  = block-sparse attention over blocks chosen by antidiagonal scoring
 *         and a cumulative-mass threshold (glossary; Table 8 threshold 0.9).
 * The layer output is the head-wise concatenation of the per-head outputs
 * (Eq. 3).  The mode array plays the role of the routing metadata that the
 * notes' deployment section passes to a single fused kernel launch.
 *
 * Conventions for every entry point
 *   - Tensors are packed variable-length batches: q, o [T, Hq, d];
 *     k, v [T, Hkv, d]; d contiguous, bfloat16.  lse [Hq, T] float32.
 *     Sequence b owns tokens [cu_seqlens[b], cu_seqlens[b+1]).
 *     GQA: query head h reads KV head h / (Hq / Hkv).
 *   - q, k, v and o must be 16-byte aligned (EA_ERR_INVALID_ARG otherwise).
 *   - Every pointer is owned by the caller.  "_dev" pointers are device
 *     memory on the current HIP device; "_host" pointers are host memory.
 *     The library allocates nothing, keeps no global state and is reentrant
 *     as long as concurrent calls use different workspaces; the one exception
 *     is ea_hybrid_attn_decode_noalloc, whose scratch is a device array the
 *     library owns (see there).
 *   - All arguments that the host can see are checked before any launch;
 *     on failure an ea_status other than EA_OK is returned and nothing is
 *     written.  Device-side data (cu_seqlens, modes) cannot be checked
 *     without a host synchronisation, so the kernels sanitise it instead:
 *     lengths are clamped to [0, max_seqlen] and to the token range, mode
 *     bytes other than 0/1/2 run as FA.  No input can make a kernel access
 *     memory outside the documented buffers.
 *   - Device work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) without any host synchronisation.  A launch failure returns
 *     EA_ERR_HIP.
 */
#ifndef EA_H
#define EA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  EA_OK = 0,
  EA_ERR_INVALID_ARG = 1, /* null pointer, bad size or parameter */
  EA_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim, block, stride */
  EA_ERR_WORKSPACE = 3,   /* workspace pointer null or too small */
  EA_ERR_HIP = 4          /* a HIP launch failed */
} ea_status;

typedef enum { EA_MODE_FA = 0, EA_MODE_SSA = 1, EA_MODE_XA = 2 } ea_mode;

/* Largest total_tokens (and so max_seqlen) the kernels accept: 2^31 - 2^16.
 * Token indices are 32-bit inside the kernels; the headroom keeps a token
 * index plus a tile's or a decode split's offset (at most 4,096) below 2^31.
 * A larger descriptor gets EA_ERR_UNSUPPORTED from every call that takes
 * one, and ea_workspace_bytes returns 0 for it. */
#define EA_MAX_TOKENS 0x7fff0000

typedef struct {
  int32_t num_seqs;      /* >= 0 */
  int32_t total_tokens;  /* T = cu_seqlens[num_seqs], 0 <= T <= EA_MAX_TOKENS */
  int32_t max_seqlen;    /* upper bound of every sequence length */
  int32_t num_q_heads;   /* Hq >= 1 */
  int32_t num_kv_heads;  /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;      /* d: 64 or 128 */
  int32_t block;         /* B: 64 or 128; kernel tile and XA block size */
  float softmax_scale;   /* c > 0, usually 1/sqrt(d) */
  int32_t ssa_sink;      /* s >= 0: keys j < s are always kept by SSA */
  int32_t ssa_window;    /* W >= 1: SSA keeps keys with i - j < W */
  int32_t xa_stride;     /* S: divides B with B/S in {4, 8, 16, 32} */
  int32_t xa_tau_num;    /* tau = num/den, 0 < tau <= 1, den <= 2^20 */
  int32_t xa_tau_den;
  int32_t xa_group;      /* 0: one XA mask per q-head; 1: one per KV head, scored
                            with the mean of its q-heads' antidiagonal scores
                            (needs Hq / Hkv in {1, 2, 4}) */
  int32_t xa_norm;       /* 0: softmax per reduced query row, pooled into
                            blocks (default); 1: softmax over each block row of
                            the raw block sums of s^ (for comparison) */
} ea_attn_desc;

/* Operation codes for ea_workspace_bytes. */
#define EA_OP_XA_SELECT 0
#define EA_OP_PREFILL 1
#define EA_OP_DECODE 2
#define EA_OP_PREFILL_SERIAL 3

/*
 * Workspace bytes that `op` needs for `desc`: an upper bound computed from
 * the descriptor alone (total_tokens, num_seqs, max_seqlen, heads, block).
 * Returns 0 if the descriptor is invalid or unsupported.
 */
size_t ea_workspace_bytes(const ea_attn_desc* desc, int op);

/*
 * Mask geometry shared by ea_xa_block_select and ea_hybrid_attn_prefill.
 * Mask rows are indexed by (global q-block, q-head): row = (P_b + I) * Hq + h,
 * where P_b = sum_{b' < b} ceil(L_b' / B) and I is the q-block within
 * sequence b.  Each row holds ea_mask_words(desc) uint32 words; bit J of the
 * row (word J / 32, bit J % 32) set means KV block J is attended.
 * ea_mask_rows(desc) = (T / B + num_seqs) * Hq is the row count the caller
 * allocates (an upper bound of the rows that exist).  Both return 0 for an
 * invalid descriptor.
 */
int64_t ea_mask_rows(const ea_attn_desc* desc);
int32_t ea_mask_words(const ea_attn_desc* desc);

/*
 * XA block selection (scoring + selector) for every XA (sequence, q-head).
 *
 * Defines XA's "which blocks" step (glossary of the Elastic Attention notes:
 * antidiagonal scoring; Table 8: block / stride / threshold):
 *   score   s^[a, b'] = c * sum_{t<S} <q_{aS+t}, k_{b'S+S-1-t}>  for b' <= a
 *           (a, b' index groups of S tokens inside the sequence),
 *   p[a, .] = softmax over b' <= a of s^[a, .],
 *   P[I, J] = (1 / (B/S)) * sum of p over the (a, b') pairs of block (I, J)
 *             (xa_norm = 1 instead: P[I, .] = softmax over J <= I of the sums
 *             of s^ over the causal (a, b') pairs of block (I, J)),
 *   w_J     = max(1, floor(P[I, J] * 2^24 + 1/2)),
 *   select  the shortest prefix of J sorted by (w desc, J asc) whose integer
 *           mass reaches tau * sum_J w_J, then add J = 0 and J = I.
 * Each q-head scores and selects its own mask (xa_group = 0), or every KV
 * head scores once with s^ averaged over its q-heads and all of them get that
 * mask (xa_group = 1: one reading of per-KV-head selection).  XA scores
 * sequences whose length is a multiple of B; on an XA head of a sequence
 * with L % B != 0 (no whole last block row to score) every causal block is
 * selected, which is what tau = 1 selects and makes XA equal to FA
 * (row_count = I + 1 on every such row).
 *
 * A row's masses and weights are held in LDS, so max_seqlen may span at most
 * 12,288 blocks (1,572,864 tokens at B = 128); a longer descriptor gets
 * EA_ERR_UNSUPPORTED.
 *
 * Inputs  q [T,Hq,d] bf16, k [T,Hkv,d] bf16, cu_seqlens_dev int32[num_seqs+1],
 *         modes_dev uint8[num_seqs * Hkv] (row-major [seq][kv head]).
 * Outputs (device; all ea_mask_rows rows are written)
 *   mask_out_dev       uint32[ea_mask_rows][ea_mask_words]; rows of non-XA
 *                      heads, and the rows past the batch's last q-block
 *                      (ea_mask_rows is a bound), are written as all-zero.
 *   row_count_out_dev  int32[ea_mask_rows]: selected blocks per row (0 for
 *                      non-XA heads and for the rows past the last q-block).
 *   xa_pairs_out_dev   int64[num_seqs * Hq]: attended (i, j) pairs per
 *                      (sequence, q-head); 0 for non-XA heads.
 *   block_mass_out_dev float32[ea_mask_rows][ceil(max_seqlen / B)] or NULL:
 *                      P[I, J] of XA rows for J <= I, zero for J > I; rows
 *                      of other heads are not touched.
 * Workspace: ea_workspace_bytes(desc, EA_OP_XA_SELECT) bytes, device memory.
 */
ea_status ea_xa_block_select(const ea_attn_desc* desc, const void* q_dev, const void* k_dev,
                             const int32_t* cu_seqlens_dev, const uint8_t* modes_dev,
                             uint32_t* mask_out_dev, int32_t* row_count_out_dev,
                             int64_t* xa_pairs_out_dev, float* block_mass_out_dev,
                             void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * Fused hybrid-head prefill attention (Eqs. 1-3 of the notes; one launch of
 * the attention kernel serves FA, SSA and XA heads together).
 *
 * For query i of sequence b (local index) and q-head h with KV head g:
 *   A(i) = { j <= i }                                   if mode FA
 *        = { j <= i : j < ssa_sink or i - j < ssa_window }   if mode SSA
 *        = { j <= i : mask bit (I = i / B, J = j / B) set }  if mode XA
 *   o_i  = sum_{j in A(i)} softmax_j(c <q_i, k_j>) v_j,
 *   lse_i = ln sum_{j in A(i)} exp(c <q_i, k_j>).
 * Outputs  o_out_dev [T,Hq,d] bf16 (round to nearest even from fp32) and
 *          lse_out_dev [Hq,T] float32.  Every token of every head is written.
 *          A query whose key set is empty (possible only with a caller-made
 *          XA mask that lacks its diagonal block) gets o = 0, lse = -inf.
 * xa_mask_dev: the mask written by ea_xa_block_select for the same inputs.
 *          If NULL, XA heads attend every causal block.
 * Workspace: ea_workspace_bytes(desc, EA_OP_PREFILL) bytes, device memory.
 */
ea_status ea_hybrid_attn_prefill(const ea_attn_desc* desc, const void* q_dev, const void* k_dev,
                                 const void* v_dev, const int32_t* cu_seqlens_dev,
                                 const uint8_t* modes_dev, const uint32_t* xa_mask_dev,
                                 void* o_out_dev, float* lse_out_dev, void* workspace_dev,
                                 size_t workspace_bytes, void* stream);

/*
 * The same prefill in two calls, for callers that schedule or time the
 * attention launch on its own.  ea_hybrid_attn_prefill is exactly
 * ea_hybrid_attn_plan followed by ea_hybrid_attn_run.
 *
 * ea_hybrid_attn_plan: validates the arguments, then writes into the
 *   workspace the per-sequence metadata, the work list (cost-sorted rows and
 *   their flagged kv tiles) and the packed K / V^T tiles.  Arguments mean
 *   what they mean for ea_hybrid_attn_prefill; q, o and lse are not used.
 * ea_hybrid_attn_run: launches the attention kernel over that plan.  It must
 *   follow a successful plan call on the same stream with the same
 *   descriptor, modes_dev and workspace, and k, v, cu_seqlens and the mask
 *   unchanged since; the library cannot check that pairing and reads
 *   whatever the workspace holds.  Writes o_out_dev and lse_out_dev as
 *   ea_hybrid_attn_prefill does.
 * Both return EA_ERR_* on invalid arguments before any launch, and
 * EA_ERR_HIP if a launch fails.
 */
ea_status ea_hybrid_attn_plan(const ea_attn_desc* desc, const void* k_dev, const void* v_dev,
                              const int32_t* cu_seqlens_dev, const uint8_t* modes_dev,
                              const uint32_t* xa_mask_dev, void* workspace_dev,
                              size_t workspace_bytes, void* stream);
ea_status ea_hybrid_attn_run(const ea_attn_desc* desc, const void* q_dev,
                             const uint8_t* modes_dev, void* o_out_dev, float* lse_out_dev,
                             void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * The same layer by serial dispatch: the baseline that the fused kernel is
 * measured against (English paper-reading notes, 04 Deployment, Algorithm 1
 * (a) and Figure 4; Chinese notes, 05 Deployment).  The heads are split by
 * mode into a full group (FA) and a sparse group (SSA) with explicit copies
 * of q, k and v, each group runs as its own single-mode layer
 * (ea_hybrid_attn_prefill with every head in that mode), and both outputs are
 * copied back into o_out_dev / lse_out_dev.  The result is bit-identical to
 * ea_hybrid_attn_prefill with the same modes: the same kernels compute every
 * row in the same order.
 * layer_modes_host: uint8[num_kv_heads], host memory, one mode per KV head
 *   for every sequence of the batch (the split needs the group sizes on the
 *   host); FA or SSA (XA returns EA_ERR_UNSUPPORTED).
 * Other arguments as for ea_hybrid_attn_prefill (no XA mask); num_q_heads
 * <= 256.  Workspace: ea_workspace_bytes(desc, EA_OP_PREFILL_SERIAL) bytes of
 * device memory (the split copies plus one inner prefill workspace).
 */
ea_status ea_hybrid_attn_prefill_serial(const ea_attn_desc* desc, const void* q_dev,
                                        const void* k_dev, const void* v_dev,
                                        const int32_t* cu_seqlens_dev,
                                        const uint8_t* layer_modes_host, void* o_out_dev,
                                        float* lse_out_dev, void* workspace_dev,
                                        size_t workspace_bytes, void* stream);

/*
 * Model and effective sparsity ratios (Eq. 4 and Eq. 5 of the Chinese
 * paper-reading notes, section on the two sparsity ratios), computed on the
 * host, synchronously.  One layer; the average runs over the KV heads of a
 * sequence, and the batch value is the mean over sequences.
 *   Omega_MSR(b) = mean_g [modes[b,g] == sparse_mode]
 *   rho(b,g)     = 1 - kept pairs of the G q-heads of g / (G * L_b (L_b+1) / 2)
 *                  (0 for FA; SSA counted from its key set; XA from xa_pairs)
 *   Omega_ESR(b) = mean_g rho(b, g)
 * Inputs (host): cu_seqlens_host int32[num_seqs+1] (nondecreasing, from 0),
 *   modes_host uint8[num_seqs*Hkv] (values 0..2), sparse_mode 0..2 names the
 *   "sparse" slot of the {retrieval}-{sparse} mode set, xa_pairs_host
 *   int64[num_seqs*Hq] as written by ea_xa_block_select (may be NULL only if
 *   no head is XA).
 * Outputs (host): msr_out and esr_out double[num_seqs+1] (per sequence, then
 *   the batch mean), rho_out double[num_seqs*Hkv], esr_pair_weighted_out
 *   double[1] or NULL (1 - total kept / total causal pairs).
 */
ea_status ea_sparsity_ratios(const ea_attn_desc* desc, const int32_t* cu_seqlens_host,
                             const uint8_t* modes_host, uint8_t sparse_mode,
                             const int64_t* xa_pairs_host, double* msr_out, double* esr_out,
                             double* rho_out, double* esr_pair_weighted_out);

/*
 * One decode step of the hybrid-head layer (routing is decided once per
 * request at prefill and reused for every generated token: English
 * paper-reading notes, 08 Commentary, the authors' stated limits, item 3).
 * The k / v cache already holds the current token: sequence b owns cache rows
 * [cu_seqlens[b], cu_seqlens[b+1]) of length L_b, and its new query (index
 * L_b - 1) attends, for q-head h of KV head g:
 *   A = { j <= L_b - 1 }                                         FA and XA
 *     = { j <= L_b - 1 : j < ssa_sink or L_b - 1 - j < ssa_window }   SSA
 *   o = sum_{j in A} softmax_j(c <q, k_j>) v_j,  lse = ln sum_{j in A} exp(c <q, k_j>).
 * XA heads attend every cached key: block selection needs blocks of query
 * rows, and a decode step has a single query.  An empty sequence gets o = 0
 * and lse = -inf.
 * Inputs  q_dev [num_seqs, Hq, d] bf16 (one new query per sequence),
 *         k_dev / v_dev [T, Hkv, d] bf16 (the packed cache, T = total_tokens),
 *         cu_seqlens_dev int32 [num_seqs + 1], modes_dev uint8 [num_seqs * Hkv]
 *         (sanitised on the device as for the prefill).
 * Outputs o_out_dev [num_seqs, Hq, d] bf16, lse_out_dev [num_seqs, Hq] fp32.
 * The descriptor's block / xa fields must be valid but are unused; Hq / Hkv
 * <= 16, num_seqs and Hkv <= 65535, and at most 2^31 - 1 decode
 * workgroups (num_seqs * Hkv * q-head groups * ceil(max_seqlen / (4 *
 * split)) for the shortest key split the descriptor allows; a workgroup
 * takes four splits) (EA_ERR_UNSUPPORTED otherwise).
 * Workspace: ea_workspace_bytes(desc, EA_OP_DECODE) bytes of device memory
 * (the step's split plan and workgroup list, and one fp32 partial result
 * per workgroup and q-head).  The step runs in stream order; concurrent
 * calls need separate workspaces.
 */
ea_status ea_hybrid_attn_decode(const ea_attn_desc* desc, const void* q_dev, const void* k_dev,
                                const void* v_dev, const int32_t* cu_seqlens_dev,
                                const uint8_t* modes_dev, void* o_out_dev, float* lse_out_dev,
                                void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * Decode over a cache in which SSA heads keep only their sink and window
 * keys.  Routing is decided once per request and reused for every generated
 * token (English paper-reading notes, 08 Commentary, the authors' stated
 * limits, item 3), and an SSA head attends only its first ssa_sink keys and
 * its last ssa_window keys (glossary: attention sink plus sliding window), so
 * its older keys are never read again and need no storage.
 *
 * Layout: a head-major pool of cache_rows rows of head_dim bf16 for k and
 * one for v.  (Sequence b, KV head g) owns rows [seg_off[u], seg_off[u + 1])
 * of both pools, u = b * Hkv + g.  An FA or XA segment stores key j in row
 * j.  An SSA segment is a ring of ssa_sink + ssa_window rows: key j < sink in
 * row j, key j >= sink in row sink + (j - sink) mod ssa_window, so it holds
 * exactly the keys a decode step of that head reads.
 * The modes, sink and window used to build the layout must be the ones the
 * cache is filled and read with (the library cannot check that).  Device
 * data is sanitised as elsewhere: segment bounds are clamped into the pool,
 * writes past a segment's end are dropped and reads clamped to its rows, so
 * no table content makes a kernel touch memory outside the pools.
 */

/*
 * Host: segment offsets for capacity_host[b] tokens per sequence (the length
 * the sequence may reach).  FA / XA segments get capacity rows, SSA segments
 * min(capacity, ssa_sink + ssa_window).  modes_host uint8[num_seqs * Hkv],
 * capacity_host int32[num_seqs] (>= 0), seg_off_host int64[num_seqs * Hkv +
 * 1] written (seg_off_host[num_seqs * Hkv] is the pool's row count).
 * Synchronous; EA_ERR_INVALID_ARG on a null pointer, a mode > 2 or a negative
 * capacity.
 */
ea_status ea_decode_cache_layout(const ea_attn_desc* desc, const uint8_t* modes_host,
                                 const int32_t* capacity_host, int64_t* seg_off_host);

/*
 * Fill the segmented cache from a packed cache k_dev / v_dev [T, Hkv, d]
 * (e.g. the keys and values of a prefill): for every (sequence, KV head), the
 * keys its mode keeps for decoding the sequence's last token (desc and
 * cu_seqlens_dev describe the packed cache).  k_cache_dev / v_cache_dev
 * [cache_rows, d] bf16, seg_off_dev int64[num_seqs * Hkv + 1] (device copies
 * of the layout), modes_dev uint8[num_seqs * Hkv].  num_seqs * Hkv <= 65535.
 * Asynchronous on `stream`.
 */
ea_status ea_decode_cache_fill(const ea_attn_desc* desc, const void* k_dev, const void* v_dev,
                               const int32_t* cu_seqlens_dev, const uint8_t* modes_dev,
                               const int64_t* seg_off_dev, int64_t cache_rows, void* k_cache_dev,
                               void* v_cache_dev, void* stream);

/*
 * Append one token per sequence: k_new_dev / v_new_dev [num_seqs, Hkv, d]
 * are written as key L_b - 1 of each segment, where cu_seqlens_dev gives the
 * lengths L_b after the append (an empty sequence appends nothing).  An SSA
 * ring overwrites the slot of the key that just left the window.
 * As for ea_hybrid_attn_decode_cached, desc.total_tokens and max_seqlen may
 * be upper bounds of the lengths.
 */
ea_status ea_decode_cache_append(const ea_attn_desc* desc, const void* k_new_dev,
                                 const void* v_new_dev, const int32_t* cu_seqlens_dev,
                                 const uint8_t* modes_dev, const int64_t* seg_off_dev,
                                 int64_t cache_rows, void* k_cache_dev, void* v_cache_dev,
                                 void* stream);

/*
 * One decode step over the segmented cache: the same step, split plan and
 * key order as ea_hybrid_attn_decode over the packed cache that holds the
 * same keys, so the outputs are bit-identical.  cu_seqlens_dev gives the
 * cached lengths L_b (the current token is cached); q, o, lse, modes,
 * workspace (EA_OP_DECODE) and limits as for ea_hybrid_attn_decode.
 * desc.total_tokens and desc.max_seqlen may be upper bounds of the sum and
 * the longest of the L_b (for example the capacity the layout was built
 * for): then one descriptor, one workspace and one captured graph serve
 * every step of a decode loop whose lengths grow in cu_seqlens_dev.  (The
 * split, and so the rounding, follows the descriptor: equal descriptors give
 * bit-identical results.)
 */
ea_status ea_hybrid_attn_decode_cached(const ea_attn_desc* desc, const void* q_dev,
                                       const void* k_cache_dev, const void* v_cache_dev,
                                       const int64_t* seg_off_dev, int64_t cache_rows,
                                       const int32_t* cu_seqlens_dev, const uint8_t* modes_dev,
                                       void* o_out_dev, float* lse_out_dev, void* workspace_dev,
                                       size_t workspace_bytes, void* stream);

/*
 * ea_hybrid_attn_decode without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Arguments, outputs, checks and results
 * are those of ea_hybrid_attn_decode (the same kernels run); the step's
 * scratch (split plan, workgroup list, fp32 partials) lives instead in a
 * device array of EA_DECODE_NOALLOC_SCRATCH_BYTES that the library owns, one
 * per GPU, held from the first call on that GPU until the process ends.
 * The call allocates nothing: no hipMalloc / hipFree and no allocating
 * library routine.
 * Limit: a step whose ea_workspace_bytes(desc, EA_OP_DECODE) exceeds
 * EA_DECODE_NOALLOC_SCRATCH_BYTES returns EA_ERR_WORKSPACE before any launch
 * (64 MiB holds, e.g., 64 sequences of 64K cached tokens, 512 of 8K, or
 * one of 1M, at 32/8 heads and d = 128).  The first call on a GPU looks up that GPU's
 * array (EA_ERR_HIP if that fails).
 * Concurrency: every call on one GPU uses the same array, so calls whose
 * device work overlaps on one GPU (different streams, or host threads
 * without ordering) race; order them on one stream or use
 * ea_hybrid_attn_decode with separate workspaces.
 */
#define EA_DECODE_NOALLOC_SCRATCH_BYTES (64u << 20)
ea_status ea_hybrid_attn_decode_noalloc(const ea_attn_desc* desc, const void* q_dev,
                                        const void* k_dev, const void* v_dev,
                                        const int32_t* cu_seqlens_dev, const uint8_t* modes_dev,
                                        void* o_out_dev, float* lse_out_dev, void* stream);

/*
 * Attention Router, inference pass (English paper-reading notes, 03 Method,
 * Figure 3 (b)(c) and the configuration taken from Appendix C.1; Chinese
 * notes, 04 Method).  For every (sequence b, KV head g):
 *   x  = mean of k[b, t, g, :] over the boundary tokens t of the sequence:
 *        the first pool_head and the last pool_tail, each token once (a
 *        sequence shorter than pool_head + pool_tail pools all its tokens,
 *        an empty one gives x = 0);
 *   u  = relu(x W1 + b1) W2 + b2                       (Task MLP, d -> H -> d)
 *   z  = relu([x, u] W3 + b3) W4 + b4                  (Router MLP, 2d -> H -> 2)
 *   modes_out[b, g] = z[1] > z[0] ? sparse_mode : retrieval_mode
 * (r = 0 is FA / the retrieval mode, r = 1 the sparse mode; ties go to the
 * retrieval mode).  The pages give pool_head = pool_tail = 100 and
 * H = 4 d; the weights are shared by the KV heads of the layer.  The pages
 * leave the pooling operator and the activation open: mean and ReLU here.
 *
 * router: host struct of device pointers to fp32 arrays, row-major [in][out]:
 *   w1 [d][H], b1 [H], w2 [H][d], b2 [d], w3 [2d][H], b3 [H], w4 [H][2],
 *   b4 [2]; hidden = H, a multiple of 4 in 4..1024; w1, w2 and w3 16-byte
 *   aligned, the biases and w4 4-byte aligned; pool_head, pool_tail >= 0.
 * desc: the layer descriptor (num_seqs, total_tokens, max_seqlen,
 *   num_kv_heads and head_dim are used; the whole descriptor must be valid).
 * k_dev: bf16 [total_tokens, num_kv_heads, head_dim], 16-byte aligned.
 * cu_seqlens_dev: int32 [num_seqs + 1]; values are clamped into
 *   [0, total_tokens] and each length to max_seqlen, so reads stay in bounds
 *   whatever it holds.
 * retrieval_mode, sparse_mode: mode codes 0..2 written for r = 0 and r = 1.
 * modes_out_dev: uint8 [num_seqs, num_kv_heads], written (device memory; can
 *   be passed straight to ea_xa_block_select / ea_hybrid_attn_prefill).
 * logits_out_dev: fp32 [num_seqs, num_kv_heads, 2] or NULL.
 * The caller owns every buffer; the call allocates nothing and needs no
 * workspace.  Returns EA_ERR_INVALID_ARG / EA_ERR_UNSUPPORTED before any
 * launch on bad arguments, EA_ERR_HIP if the launch fails.  Asynchronous on
 * `stream`.
 */
typedef struct {
  const float* w1;
  const float* b1;
  const float* w2;
  const float* b2;
  const float* w3;
  const float* b3;
  const float* w4;
  const float* b4;
  int32_t hidden;
  int32_t pool_head;
  int32_t pool_tail;
} ea_router_desc;

ea_status ea_route_heads(const ea_attn_desc* desc, const ea_router_desc* router,
                         const void* k_dev, const int32_t* cu_seqlens_dev,
                         uint8_t retrieval_mode, uint8_t sparse_mode, uint8_t* modes_out_dev,
                         float* logits_out_dev, void* stream);

/*
 * Diagnostics: byte offset of a named internal buffer inside the workspace of
 * `op` (for example "tiles", "row_off", "row_cost", "sorted_units" of the
 * prefill work list, "xa_lse" of the selector), or -1 if the name is unknown
 * for that operation or the descriptor is invalid.  The layout is an
 * implementation detail; this exists so that tests can check the work list.
 */
int64_t ea_workspace_offset(const ea_attn_desc* desc, int op, const char* name);

/* Static string naming a status code. */
const char* ea_status_string(ea_status status);

#ifdef __cplusplus
}
#endif

#endif /* EA_H */
