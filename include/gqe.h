/*
 * gqe.h - C ABI of the Grouped Query Experts (GQE) attention layer on MI355X.
 *
 * The layer (GQE review, paper.oopus.info, section 二 核心方法与创新):
 *   - N routed query heads split into G groups of M = N/G experts; group g
 *     owns KV head g. For token i and group g a router scores the M experts,
 *     p = softmax(r_g(x_i)), and keeps the top k of them (the TopK equation).
 *   - Only selected heads attend; the KV heads stay dense and are never
 *     repeated (GQA tutorial, zone.ci, sections 4.3/4.4 and 技术深化).
 *   - One always-on shared query head (query column block N) attends KV
 *     head 0.
 *   - y_i = Concat(O_i, obar_i, s(x_i)) W_O, where O_i are the k*G selected
 *     head outputs (group-major, ascending expert index within a group),
 *     obar_i = sum over every group g and selected m of w_{i,g,m} o_{i,g,m}
 *     with w the softmax probabilities renormalised over the selected set,
 *     and s(x_i) the shared head's output (the w and obar equations).
 *
 * Conventions shared by every entry point:
 *   - Every pointer except those named *_or_null is required. Device
 *     pointers must be 16-byte aligned; tensors are dense and row-major in
 *     the layouts given below. The caller owns every buffer (inputs, outputs,
 *     workspaces); the library allocates, frees and synchronises nothing and
 *     keeps no state between calls.
 *   - stream is a hipStream_t passed as void* (NULL = the default stream).
 *     All work is enqueued asynchronously on it; faults inside a kernel
 *     surface at the caller's next synchronisation. Every call enqueues
 *     kernel launches only (no memset, copy or host wait), so it may be
 *     captured into a HIP graph, and calls on different streams may run
 *     concurrently (gqe_attn_decode_noalloc excepted: see there).
 *   - Arguments are validated before anything is enqueued. A call that
 *     returns an error has enqueued nothing and written nothing.
 *   - Supported: head_dim d in {32, 64, 128}; G >= 1 dividing N; 1 <= k <= M;
 *     M <= 32 and G*M <= 256; D a multiple of 8; dtype GQE_BF16 or GQE_F32.
 *     Anything else returns GQE_ERR_UNSUPPORTED: an unsupported head layout
 *     is rejected, never mapped silently (GQA tutorial, 扩展验证组合).
 *   - B == 0 or S == 0 is an empty call: GQE_OK, nothing enqueued.
 *   - Floating-point outputs have the input dtype, except logits and topk_w
 *     which are always fp32. Arithmetic is fp32 (bf16 inputs: bf16 matrix
 *     products with fp32 accumulation, fp32 softmax).
 */
#ifndef GQE_H
#define GQE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GQE_OK = 0,
  GQE_ERR_INVALID_ARG = -1, /* null pointer, negative size, inconsistent sizes */
  GQE_ERR_UNSUPPORTED = -2, /* head layout, head_dim, top-k or dtype not supported */
  GQE_ERR_ALIGNMENT = -3,   /* a device pointer is not 16-byte aligned */
  GQE_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required */
  GQE_ERR_HIP = -5,         /* the HIP runtime refused a launch */
  GQE_ERR_SCRATCH = -6      /* the call needs more than the library's static scratch */
} gqe_status;

typedef enum { GQE_BF16 = 0, GQE_F32 = 1 } gqe_dtype;

/* Slot layouts of the output projection: the method's [O, obar, s] and the
 * two ablation rows of GQE review, section 四, Table 2, each of which keeps
 * the hard slots only (no obar slot, no shared head; the row labels name the
 * one kind of concatenation kept, and the note under the table and the
 * 1kpapers summary, In brief, tie the drops to removing the renormalised
 * slot and the shared head). */
typedef enum {
  GQE_SLOTS_FULL = 0,     /* [O_i, obar_i, s_i], W_O has (G*k+2)*d rows */
  GQE_SLOTS_HARD = 1,     /* hard concatenation only: A_i = O_i, G*k*d rows */
  GQE_SLOTS_WEIGHTED = 2  /* weighted concatenation, renormalised slot removed:
                             A_i = p * O_i, each hard slot scaled by the router
                             probability p of its expert (softmax over all M,
                             not renormalised; gqe_route's topk_p); G*k*d rows */
} gqe_slot_mode;

/* What the slot weights given to gqe_route_bwd are. */
typedef enum {
  GQE_WEIGHTS_RENORM = 0, /* the renormalised weights w (topk_w): GQE_SLOTS_FULL */
  GQE_WEIGHTS_PROB = 1    /* the selected probabilities p (topk_p): GQE_SLOTS_WEIGHTED */
} gqe_weight_kind;

/* Layer shape. B sequences of S tokens, model width D, N routed query heads,
 * G KV heads (= groups), top-k per group, head_dim d; M = N/G. The shared
 * head is always present. For decode, S is the cache capacity S_max. */
typedef struct {
  int32_t B, S, D, N, G, k, d;
  int32_t dtype; /* gqe_dtype */
} gqe_dims;

/* Human-readable name of a gqe_status value (static storage). */
const char* gqe_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int gqe_version(void);

/* Bytes of workspace gqe_route needs to build the token lists (0 when the
 * lists are not requested). */
size_t gqe_route_workspace_bytes(const gqe_dims* dims);

/* Router, top-k and per-(group, expert) token lists for T = B*S tokens.
 * GQE review, section 二 路由器: z_{i,g} = x_i W_r[g]^T (+ b_r[g]) in R^M,
 * p = softmax(z), K_g = TopK(p, k) (taken on z: the same set); ties go to the
 * lower expert index; w_{i,g,m} = p_m / sum_{m' in K_g} p_{m'}.
 *   x              [B*S, D]      dtype
 *   w_router       [G*M, D]      dtype   (row g*M+m scores expert m of group g)
 *   b_router       [G*M] fp32 or NULL
 *   logits_or_null [B*S, G, M]   fp32 out (z, bias included)
 *   topk_idx       [B*S, G, k]   int32 out, expert indices in 0..M-1, ascending
 *   topk_w         [B*S, G, k]   fp32 out, renormalised weights (sum 1; exactly 1 for k=1)
 *   topk_p_or_null [B*S, G, k]   fp32 out, p of the selected experts (the
 *                  weights of the GQE_SLOTS_WEIGHTED layout)
 *   list_off_or_null [B, G, M+1] int32 out: list of expert m of group g in
 *                  sequence b is list_tok[b,g, off[m] : off[m+1]]; off[0]=0, off[M]=k*S
 *   list_tok_or_null [B, G, k*S] int32 out: token positions (0..S-1), each
 *                  list strictly ascending
 *   workspace      >= gqe_route_workspace_bytes(dims) device bytes when the
 *                  lists are requested, else may be NULL.
 * list_off and list_tok must be both NULL or both non-NULL. Selection is a
 * pure function of the emitted fp32 logits: same logits, same indices, bit
 * for bit.
 * Beyond the minimal router call (dims, x, W_r, logits, topk_idx, topk_w,
 * lists, stream) this takes an optional bias (the skewed-router workloads),
 * the optional topk_p, and the lists' count workspace (the library allocates
 * nothing). The lists are the expert-major view of topk_idx for callers that
 * gather rows by expert; no other entry point reads them: the attention and
 * projection kernels read topk_idx, position-major. */
int gqe_route(const gqe_dims* dims, const void* x, const void* w_router,
              const float* b_router, float* logits_or_null, int32_t* topk_idx,
              float* topk_w, float* topk_p_or_null, int32_t* list_off_or_null,
              int32_t* list_tok_or_null, void* workspace, size_t ws_bytes, void* stream);

/* Sparse-query causal prefill attention. The selected rows come from
 * topk_idx (position-major: every tile holds k rows per token whatever the
 * routing skew), not from gqe_route's expert-major lists.
 * For token i (absolute position i in its sequence), group g and slot j the
 * head h = g*M + topk_idx[i,g,j] attends KV head g over keys 0..i:
 * o = sum_{t<=i} softmax_t(q_{i,h}.k_t / sqrt(d)) v_t (GQA tutorial,
 * 技术深化: head h reads KV head floor(h/M); additive causal mask; scale
 * 1/sqrt(d)). The shared head (column block N of q) attends KV head 0.
 * Unselected heads are never computed (GQE review, section 二).
 *   q        [B, S, N+1, d]  dtype
 *   k, v     [B, G, S, d]    dtype  (dense, never repeated per query head)
 *   topk_idx [B*S, G, k]     int32 (as written by gqe_route)
 *   o_routed [B, S, G, k, d] dtype out
 *   o_shared [B, S, d]       dtype out
 * topk_idx entries must lie in 0..M-1. An entry outside breaks the contract:
 * the kernels clamp it into that range wherever it addresses memory (here,
 * in decode and in the backward passes), so that row's outputs are
 * unspecified but nothing outside the buffers is read or written. */
int gqe_attn_prefill(const gqe_dims* dims, const void* q, const void* k,
                     const void* v, const int32_t* topk_idx, void* o_routed,
                     void* o_shared, void* stream);

/* Training forward: gqe_attn_prefill plus each row's log-sum-exp, the
 * softmax normaliser the backward pass rebuilds P from (GQE review, section
 * 二: the routed and shared heads are trained end to end).
 *   lse_routed [B, S, G, k] fp32 out: ln sum_{t<=i} exp(q.k_t / sqrt(d))
 *   lse_shared [B, S]       fp32 out
 * In the bf16 path the scores are those of the bf16 kernel (q scaled and
 * rounded to bf16 before the product). Same errors as gqe_attn_prefill, and
 * GQE_ERR_INVALID_ARG for a NULL lse pointer. */
int gqe_attn_prefill_train(const gqe_dims* dims, const void* q, const void* k,
                           const void* v, const int32_t* topk_idx, void* o_routed,
                           void* o_shared, float* lse_routed, float* lse_shared,
                           void* stream);

/* Bytes of device workspace gqe_attn_prefill_bwd needs (0 for invalid dims):
 * packed q and dO rows, two fp32 scalars per row and, for bf16, fp32 partial
 * sums of KV head 0's dK and dV. */
size_t gqe_attn_prefill_bwd_workspace_bytes(const gqe_dims* dims);

/* Backward of gqe_attn_prefill. With P = softmax(q.k/sqrt(d)) over the
 * visible keys and o = P V (GQA tutorial, 技术深化):
 *   dV_t += P_t dO,  dS_t = P_t (dO.v_t - dO.o),
 *   dq = sum_t dS_t k_t / sqrt(d),  dK_t += dS_t q / sqrt(d).
 * dK and dV of a KV head are summed over every query row that reads it: the
 * selected heads of its group and, for KV head 0, the shared head (GQA-zone
 * page, 训练与部署: shared keys and values sum the gradients of their query
 * heads).
 *   q, k, v, topk_idx          as given to the forward
 *   o_routed, o_shared         the forward's outputs
 *   lse_routed, lse_shared     from gqe_attn_prefill_train on the same inputs
 *   do_routed [B, S, G, k, d], do_shared [B, S, d]   dtype, the output gradients
 *   dq [B, S, N+1, d]  dtype out: written for the selected heads and the
 *                      shared head only; the caller owns (and zeroes, if it
 *                      needs them) the rows of unselected heads
 *   dk, dv [B, G, S, d] dtype out, fully written
 *   workspace >= gqe_attn_prefill_bwd_workspace_bytes(dims) device bytes.
 * Deterministic: no atomics; the same inputs give the same bits. */
int gqe_attn_prefill_bwd(const gqe_dims* dims, const void* q, const void* k,
                         const void* v, const int32_t* topk_idx, const void* o_routed,
                         const void* o_shared, const float* lse_routed,
                         const float* lse_shared, const void* do_routed,
                         const void* do_shared, void* dq, void* dk, void* dv,
                         void* workspace, size_t ws_bytes, void* stream);

/* Bytes of workspace gqe_attn_decode needs (split-sequence partials). */
size_t gqe_decode_workspace_bytes(const gqe_dims* dims, int32_t q_len);

/* Sparse-query attention of q_len new tokens per sequence against a KV
 * cache of capacity S_max = dims->S. Token t of sequence b sits at absolute
 * position kv_len[b] - q_len + t and sees keys 0..that position (GQA
 * tutorial, 技术深化 and 工程实操: decode masks by the query's absolute
 * position, never by a top-left triangle). Heads and groups as for prefill.
 *   q        [B, q_len, N+1, d]   dtype
 *   k_cache, v_cache [B, G, S_max, d] dtype
 *   kv_len   [B] int32 device, valid cache length including the new tokens;
 *            q_len <= kv_len[b] <= S_max is required (not checkable without a
 *            device sync; a violating entry yields unspecified outputs for
 *            that sequence, and the kernels clamp it to 0..S_max, so nothing
 *            outside the sequence's cache is read)
 *   topk_idx [B*q_len, G, k] int32
 *   o_routed [B, q_len, G, k, d] dtype out; o_shared [B, q_len, d] dtype out
 *   workspace >= gqe_decode_workspace_bytes(dims, q_len) device bytes. */
int gqe_attn_decode(const gqe_dims* dims, int32_t q_len, const void* q,
                    const void* k_cache, const void* v_cache,
                    const int32_t* kv_len, const int32_t* topk_idx,
                    void* o_routed, void* o_shared, void* workspace,
                    size_t ws_bytes, void* stream);

/* Bytes of the static device scratch of gqe_attn_decode_noalloc (16 MiB). */
size_t gqe_decode_scratch_bytes(void);

/* gqe_attn_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and kernels, bit for bit, with the split partials in a
 * static device array of gqe_decode_scratch_bytes() bytes instead of a caller
 * workspace. The library holds that array on every GPU it runs on until the
 * process ends; its address is looked up on the first call on each device.
 * No call allocates or frees memory. A call whose partials
 * (gqe_decode_workspace_bytes(dims, q_len)) exceed the scratch returns
 * GQE_ERR_SCRATCH and enqueues nothing. All calls on one GPU share its
 * scratch: calls that overlap in time on one GPU (other streams, other host
 * threads) race and give unspecified outputs; calls ordered on one stream
 * are safe. Arguments and errors otherwise as for gqe_attn_decode. */
int gqe_attn_decode_noalloc(const gqe_dims* dims, int32_t q_len, const void* q,
                            const void* k_cache, const void* v_cache,
                            const int32_t* kv_len, const int32_t* topk_idx,
                            void* o_routed, void* o_shared, void* stream);

/* gqe_attn_decode against a paged KV cache, with optional left padding.
 * The cache of every sequence is a list of pages of page_size consecutive
 * keys for all G heads; key j of sequence b is row j % page_size of head g in
 * page block_table[b, j / page_size]. Keys j < kv_start[b] are padding and
 * visible to no query: visibility = causal and key-valid (GQA tutorial,
 * 工程实操). Everything else is as for gqe_attn_decode, with S_max =
 * dims->S = max_pages * page_size.
 *   k_pages, v_pages [n_pages, G, page_size, d] dtype
 *   block_table [B, max_pages] int32 device; the entries of the pages that
 *            hold keys below kv_len[b] must be valid page indices (others are
 *            not read)
 *   page_size  a power of two, >= 64 (else GQE_ERR_UNSUPPORTED); dims->S must
 *            be a multiple of it (else GQE_ERR_INVALID_ARG)
 *   kv_start_or_null [B] int32 device, 0 <= kv_start[b] <= kv_len[b] - q_len
 *   workspace >= gqe_decode_workspace_bytes(dims, q_len) device bytes. */
int gqe_attn_decode_paged(const gqe_dims* dims, int32_t q_len, const void* q,
                          const void* k_pages, const void* v_pages,
                          const int32_t* block_table, int32_t page_size,
                          const int32_t* kv_start_or_null, const int32_t* kv_len,
                          const int32_t* topk_idx, void* o_routed, void* o_shared,
                          void* workspace, size_t ws_bytes, void* stream);

/* Slot assembly and output projection for T tokens (GQE review, section 二,
 * the y equation): A_t = [o_routed[t] (G*k*d values, group-major, slots as
 * stored), obar_t, o_shared[t]] with obar_t = sum_{g,j} topk_w[t,g,j] *
 * o_routed[t,g,j,:]; y_t = A_t W_O.
 *   o_routed [T, G, k, d] dtype; topk_w [T, G, k] fp32; o_shared [T, d] dtype
 *   w_o      [(G*k+2)*d, D] dtype
 *   y        [T, D] dtype out
 * dims->B and dims->S are ignored; T >= 0. D must be below 2^23 (the tiled
 * kernel addresses a 256-token output tile through a 32-bit byte range),
 * else GQE_ERR_UNSUPPORTED. */
int gqe_out_proj(const gqe_dims* dims, int64_t T, const void* o_routed,
                 const float* topk_w, const void* o_shared, const void* w_o,
                 void* y, void* stream);

/* gqe_out_proj with another slot layout (gqe_slot_mode): y_t = A_t W_O.
 *   slot_w  [T, G, k] fp32: GQE_SLOTS_FULL the renormalised weights topk_w;
 *           GQE_SLOTS_WEIGHTED the selected probabilities topk_p (each hard
 *           slot is scaled by its own); GQE_SLOTS_HARD unused, may be NULL
 *   o_shared [T, d]: read by GQE_SLOTS_FULL only; NULL allowed otherwise
 *   w_o [(G*k+2)*d, D] for GQE_SLOTS_FULL, else [G*k*d, D]; any other mode
 *   returns GQE_ERR_UNSUPPORTED, as does D >= 2^23. */
int gqe_out_proj_variant(const gqe_dims* dims, int32_t mode, int64_t T,
                         const void* o_routed, const float* slot_w,
                         const void* o_shared, const void* w_o, void* y,
                         void* stream);

/* Bytes of device workspace gqe_out_proj_bwd needs (0 for invalid input). */
size_t gqe_out_proj_bwd_workspace_bytes(const gqe_dims* dims, int32_t mode, int64_t T);

/* Backward of gqe_out_proj_variant (GQE review, section 二: y = A W_O with
 * A = Concat(O, obar, s) and obar = sum over groups and selected experts of
 * w * o). With dA = dy W_O^T split into its slots:
 *   dW_O = A^T dy;  dO_s = dA[s];
 *   GQE_SLOTS_FULL:     dO_r = dA[O] + w dA[obar],  dw = o . dA[obar]
 *                       (the renormalised slot is what gives the router a
 *                       gradient, section 二);
 *   GQE_SLOTS_HARD:     dO_r = dA[O], dw = 0, dO_s = 0;
 *   GQE_SLOTS_WEIGHTED: dO_r = p dA[p O], dw = o . dA[p O] (the gradient of
 *                       the slot weights p), dO_s = 0.
 *   o_routed [T, G, k, d], slot_w [T, G, k] fp32 (as for
 *   gqe_out_proj_variant), o_shared [T, d], w_o as for the forward,
 *   dy [T, D]                                                     inputs
 *   do_routed [T, G, k, d] dtype, dw [T, G, k] fp32, do_shared [T, d] dtype,
 *   dw_o [rows of w_o, D] fp32                                    outputs
 *   In the ablation layouts o_shared and do_shared may be NULL; a given
 *   do_shared is filled with zeros. slot_w may be NULL for GQE_SLOTS_HARD.
 *   workspace >= gqe_out_proj_bwd_workspace_bytes(dims, mode, T) device bytes.
 * Deterministic (weight gradient summed over token ranges in a fixed order).
 * In the bf16 path the products take bf16 operands (A rounded as in the
 * forward) with fp32 accumulation. */
int gqe_out_proj_bwd(const gqe_dims* dims, int32_t mode, int64_t T,
                     const void* o_routed, const float* slot_w, const void* o_shared,
                     const void* w_o, const void* dy, void* do_routed, float* dw,
                     void* do_shared, float* dw_o, void* workspace, size_t ws_bytes,
                     void* stream);

/* Bytes of device workspace gqe_route_bwd needs (0 for invalid dims). */
size_t gqe_route_bwd_workspace_bytes(const gqe_dims* dims);

/* Backward of gqe_route's weights for T = B*S tokens (GQE review, section
 * 二: p = softmax(z), w = p_sel / sum p_sel over the TopK set, which is
 * piecewise constant and carries no gradient):
 *   weights GQE_WEIGHTS_RENORM (dw is the gradient of w):
 *     dp_sel = (dw - sum_j dw_j w_j) / sum p_sel on the selected experts;
 *   weights GQE_WEIGHTS_PROB (dw is the gradient of the selected p, as
 *   gqe_out_proj_bwd gives it for GQE_SLOTS_WEIGHTED): dp_sel = dw;
 *   0 on the others; dz = p (dp - p . dp); dW_r = dz^T x; db_r = sum_t dz;
 *   dx = dz W_r. Any other weights value returns GQE_ERR_UNSUPPORTED.
 * aux_coef > 0 adds the load-balancing loss the review says training uses
 * (its formula is not given; reading: per group router, averaged over the
 * groups) L = aux_coef * M * mean_g sum_m f_{g,m} P_{g,m}, f the share of the
 * T*k selections of group g that chose m, P the mean of p over tokens; f is
 * a count and carries no gradient, so dp gains aux_coef*M*f/(T*G).
 *   x [B*S, D] dtype, w_router [G*M, D] dtype, logits [B*S, G, M] fp32 (as
 *   written by gqe_route), topk_idx [B*S, G, k], dw [B*S, G, k] fp32  inputs
 *   dz_or_null [B*S, G, M] fp32, dx [B*S, D] dtype, dw_router [G*M, D] fp32,
 *   db_router [G*M] fp32, aux_loss_or_null [1] fp32 (the loss value) outputs
 *   workspace >= gqe_route_bwd_workspace_bytes(dims) device bytes.
 * aux_coef must be finite and >= 0 (GQE_ERR_INVALID_ARG). */
int gqe_route_bwd(const gqe_dims* dims, const void* x, const void* w_router,
                  const float* logits, const int32_t* topk_idx, const float* dw,
                  int32_t weights, float aux_coef, float* dz_or_null, void* dx, float* dw_router,
                  float* db_router, float* aux_loss_or_null, void* workspace,
                  size_t ws_bytes, void* stream);

/* Query, key and value projections of a prefill with token-compacted
 * queries. GQE review, section 二: only the selected query heads take part in
 * attention, the others are skipped, so only their query rows are projected;
 * GQA tutorial, 4.3: queries carry N heads, keys and values G heads.
 *   q_{i,h} = W_Q[h] x_i for the G*k heads token i selected and for the shared
 *   head h = N; k_{i,g} = W_K[g] x_i and v_{i,g} = W_V[g] x_i for every token
 *   and group, where W[h] is rows h*d .. h*d+d-1 of W (no bias).
 *   x        [B, S, D]       dtype
 *   w_q      [(N+1)*d, D]    dtype (block N projects the shared head)
 *   w_k, w_v [G*d, D]        dtype
 *   topk_idx [B*S, G, k]     int32 (as written by gqe_route); a routed head's
 *            rows are the tokens whose top-k holds it, the rows of its
 *            expert-major token list
 *   q        [B, S, N+1, d]  dtype out: the rows of the selected heads and of
 *            the shared head are written; rows of unselected heads keep their
 *            previous contents
 *   k, v     [B, G, S, d]    dtype out
 * bf16 needs D % 64 == 0 (else GQE_ERR_UNSUPPORTED). */
int gqe_qkv_proj(const gqe_dims* dims, const void* x, const void* w_q,
                 const void* w_k, const void* w_v, const int32_t* topk_idx,
                 void* q, void* k, void* v, void* stream);

/* The same projections for q_len new tokens per sequence in decode, with the
 * new keys and values written into the cache: token t of sequence b goes to
 * cache row kv_len[b] - q_len + t, its absolute position (GQA tutorial,
 * 技术深化). No other cache row is touched.
 *   x        [B, q_len, D]   dtype; topk_idx [B*q_len, G, k] int32
 *   kv_len   [B] int32 device, q_len <= kv_len[b] <= S_max = dims->S (not
 *            checkable without a device sync; with a violating entry the
 *            rows kv_len[b] - q_len + t outside 0..S_max-1 are not written,
 *            so no write leaves the sequence's cache)
 *   q        [B, q_len, N+1, d] dtype out (selected heads and shared head)
 *   k_cache, v_cache [B, G, S_max, d] dtype, updated in place
 * bf16 needs D % 64 == 0. */
int gqe_qkv_proj_decode(const gqe_dims* dims, int32_t q_len, const void* x,
                        const void* w_q, const void* w_k, const void* w_v,
                        const int32_t* topk_idx, const int32_t* kv_len,
                        void* q, void* k_cache, void* v_cache, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQE_H */
