/*
 * still.h -- C ABI of libstill.so: the forward pass of one STILL attention
 * layer (intra-layer hybrid of softmax and linear attention) on gfx950.
 *
 * Pages cited (short tag -> page title):
 *   [P2] "NeurIPS 2026|层内混合注意力：告别位置「伪混合」，STILL首个内容感知的层内混合注意力架构",
 *        sections 亮点一 (固定预算路由, 延迟选择与分块并行), 亮点二
 *   [P3] "STILL: Content-Aware Intra-Layer Hybrid Attention for Efficient
 *        LLM Linearization", sections "Content-Aware Routing with Fixed
 *        Budget", "Delayed Chunk-Level Selection for Unified
 *        Training-Inference Parallelism", "Self-Saliency Score",
 *        "NP-Map: Norm-Preserving Feature Map"
 *
 * What one layer computes, per batch row b and kv head k (query heads
 * h = k*G .. k*G+G-1 share k's keys, values, routing and state):
 *   score(t)  Self-Saliency Score [P3 "Self-Saliency Score"], reading:
 *             sum over the group's heads of KL(a_diag || (1-eps) a_nodiag +
 *             eps delta_t) over the window [t-W+1, t], logits scaled by
 *             sm_scale.
 *   routing   [P3 "Content-Aware Routing ..."], [P2 固定预算路由]: budget m =
 *             W window slots + m-W kept slots; when chunk c+1 begins, chunk c
 *             keeps its lambda = min(C, floor((m-W)/T_max)) best tokens by
 *             (score desc, position asc) [P3 "Delayed Chunk-Level
 *             Selection ..."], while the kept pool has room; kept tokens stay.
 *   output    softmax over A(t) = window, own chunk's prefix and kept tokens;
 *             NP-Map linear attention over B(t) = every other past token
 *             (decided, not kept, left the window) [P3 "NP-Map ..."]; one
 *             normaliser over exp(logit) and gate[h] * <phi(q), phi(k)>.
 *   state     S = sum phi(k_j) v_j^T, z = sum phi(k_j) over the unkept tokens
 *             of the chunks lying wholly before the window of every query of
 *             the current chunk; the kept pool; the recent tokens (ring); the
 *             fp64 scores of the undecided chunk; the position.
 *
 * Conventions (all entry points):
 *   - Tensor pointers are DEVICE pointers to contiguous arrays, 16-byte
 *     aligned; params are host memory. The caller owns every buffer; the
 *     library never allocates, frees or synchronises in these calls.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream)
 *     and is asynchronous. Arguments are validated on the host before any
 *     launch: on failure a negative status is returned and nothing is
 *     written or launched. A launch failure returns STILL_EHIP.
 *   - Layouts are row-major: q/out [B, Hq, L, d], k/v [B, Hkv, L, d].
 *     Element type of q, k, v, fmap_w, out is params.dtype (out is float32
 *     when STILL_FLAG_FP32_OUT is set). gate is float32 [Hq], each in [0,1].
 *   - Supported: head_dim 64 or 128; chunk 16, 32, 64 or 128; window >= 1;
 *     budget >= window; t_max >= 1; n_q_heads a multiple of n_kv_heads
 *     with G = n_q_heads / n_kv_heads <= 8. All sequences of a batch share
 *     one length / position.
 *   - Thread safety: every entry point may be called from several host
 *     threads at once (on different buffers). The only shared host state is
 *     a mutex-protected table of per-device kernel attributes.
 *   - Value range (bf16): values and NP-Map features enter their products
 *     as fp16, so every |v_i| and every key / query norm |x| (the NP-Map
 *     feature of x has norm |x|) must stay below 65504; larger inputs give
 *     undefined outputs (inf / NaN). This is not checked.
 *   - Accuracy: bf16 outputs and the float32 state follow the float64
 *     definition to about 2e-3 max-abs on the 16K and 64K workloads (state
 *     entries up to 4e4); float32 scores to 1e-6 of max(1, |score|) (tokens
 *     whose estimated float32 error is larger are recomputed in float64).
 *     float32 data: logits, features and weights are float32 products, so
 *     the error grows with |q| |k| scale max|v|; it stays below 1e-4 for
 *     inputs of the small float32 workload's range (norms ~ sqrt(d) times a
 *     LogNormal(0, 0.5) factor, no outliers).
 */
#ifndef STILL_H
#define STILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define STILL_ABI_VERSION 1

enum { STILL_DTYPE_F32 = 0, STILL_DTYPE_BF16 = 1 };

/* flags */
#define STILL_FLAG_FP32_OUT 1u /* write `out` as float32 whatever the dtype */
/* Branch variants (the pages' ablation axes; the default is one normaliser
 * over exp(logit) and gate * <phi(q), phi(k)>):
 *   SOFTMAX_ONLY: the linear branch is dropped, unkept tokens are discarded
 *     (the "sparse attention only" alternative [P3 "Problems with Existing
 *     Intra-Layer Hybrid Attention"]); y = softmax over A(t). The state is
 *     still maintained. Prefill and decode.
 *   MERGE_SUM: y = y_SA + gate * y_LA, each branch normalised on its own (a
 *     merge of separately normalised branches, [P4 §4 Gating]). Prefill
 *     only (decode returns STILL_EUNSUPPORTED). */
#define STILL_FLAG_SOFTMAX_ONLY 2u
#define STILL_FLAG_MERGE_SUM 4u
/* Paged kept pool (serving layout for ragged batches, [P3 "Delayed
 * Chunk-Level Selection ..."]: each sequence keeps its own pool): the decode
 * state holds no pool rows (its pool_k and pool_v regions are empty) and the
 * rows live in pages of an arena the caller allocates and maps per unit
 * through a page table (see still_prefill_paged); only the _paged entries
 * accept such params (the others return STILL_EINVAL). The pool's capacity
 * (budget - window rows) may span at most 256 pages. */
#define STILL_FLAG_PAGED_POOL 16u
#define STILL_POOL_PAGE_ROWS 16 /* kept tokens per page */
/* 8-bit kept pool (the fp8 pool K/V of the pages' precision work; the
 * format is a reading, the pages name none): the decode state stores each
 * kept key and value row as OCP E4M3 codes of x_i / 2^e with one scale
 * exponent per row (as the E8M0 scales of the OCP microscaling formats):
 * e the smallest integer with amax_i |x_i| <= 448 * 2^e, at least -126, 0
 * for a zero row; x_i / 2^e (exact) rounded to the nearest E4M3 value, ties
 * to the even code, beyond 448 to 448. Region pool_k holds the
 * (budget - window) rows of head_dim key codes, then one byte e + 127 per
 * row; pool_v likewise. Decode steps read the kept tokens below the window
 * band from this store (exactly: 2^e multiplies the logit, and the weight
 * of the value); the band, the linear state and the prefill's own outputs
 * keep the data's precision. bf16 data only, not with
 * STILL_FLAG_PAGED_POOL (STILL_EUNSUPPORTED). */
#define STILL_FLAG_POOL_FP8 32u
/* Routing metric, flags bits 8..11 (STILL_FLAG_ROUTE(r)): the score that
 * ranks a chunk's tokens for the delayed Top-lambda. The default is the
 * Self-Saliency Score; the others are the alternatives of the STILL
 * article's routing-metric ablation [P3 "Ablation Studies"], each computed
 * in float64 and summed over the group's query heads where it is per head:
 *   DIAG      the window softmax's weight on the token itself;
 *   QK        the scaled self logit scale * q_t . k_t;
 *   KEYNORM   ||k_t|| (per kv head);
 *   UNIFORM   1 at the chunk offsets floor(i C / lambda), i < lambda, else
 *             0 (evenly spaced picks);
 *   EXTERNAL  the caller's scores: still_prefill's `score` argument becomes
 *             a required input [B, Hkv, L] float32 (e.g. random draws for
 *             random routing) and is not written. Prefill only (decode
 *             returns STILL_EUNSUPPORTED).
 * Ties rank the lower position first, as for the default score. */
#define STILL_ROUTE_SALIENCY 0u
#define STILL_ROUTE_DIAG 1u
#define STILL_ROUTE_QK 2u
#define STILL_ROUTE_KEYNORM 3u
#define STILL_ROUTE_UNIFORM 4u
#define STILL_ROUTE_EXTERNAL 5u
#define STILL_FLAG_ROUTE(r) ((uint32_t)(r) << 8)
#define STILL_ROUTE_OF(flags) (((uint32_t)(flags) >> 8) & 15u)
/* Any other bit, a routing metric above STILL_ROUTE_EXTERNAL, or
 * SOFTMAX_ONLY and MERGE_SUM together make every entry that takes the
 * params return STILL_EINVAL. */

/* status codes */
#define STILL_OK 0
#define STILL_EINVAL (-1)       /* null pointer, bad size or value */
#define STILL_EUNSUPPORTED (-2) /* valid but not built (head_dim, chunk, G) */
#define STILL_EWORKSPACE (-3)   /* workspace smaller than still_workspace_bytes */
#define STILL_EHIP (-4)         /* a HIP launch failed */
#define STILL_ESTATE (-5)       /* decode position does not follow the state */
#define STILL_ESCRATCH (-6)     /* needs more than still_prefill_noalloc's scratch */

typedef struct still_params {
  int32_t abi_version; /* STILL_ABI_VERSION */
  int32_t dtype;       /* STILL_DTYPE_F32 or STILL_DTYPE_BF16 */
  int32_t batch, n_q_heads, n_kv_heads, head_dim;
  int32_t window; /* W: recent tokens always kept for softmax */
  int32_t chunk;  /* C: routing decision granularity */
  int32_t budget; /* m: softmax KV slots per kv head (window + kept) */
  int32_t t_max;  /* T_max: chunks the m - W kept slots are spread over */
  float eps;      /* score smoothing, > 0 (1e-6 if <= 0) */
  float sm_scale; /* logit scale; <= 0 means 1/sqrt(head_dim) */
  uint32_t flags; /* STILL_FLAG_* */
} still_params;

/* Byte offsets of one unit's (batch row, kv head) state inside the state
 * blob; unit u = b * n_kv_heads + k starts at u * unit_bytes. */
typedef struct still_state_layout {
  int64_t unit_bytes;
  int64_t S;        /* float32 [d][d], S[i][j] = sum phi(k)_i v_j     */
  int64_t z;        /* float32 [d]                                     */
  int64_t pool_k;   /* dtype [m-W][d], kept keys, ascending position   */
  int64_t pool_v;   /* dtype [m-W][d]                                  */
  int64_t pool_pos; /* int32 [m-W]                                     */
  int64_t ring_k;   /* dtype [R][d], token at position p in slot p % R */
  int64_t ring_v;   /* dtype [R][d]                                    */
  int64_t ring_phi; /* dtype [R][d], NP-Map feature of ring_k          */
  int64_t ring_flag;/* int32 [R], 1 = kept                             */
  int64_t pending;  /* float64 [C], scores of the undecided chunk      */
  int64_t meta;     /* int64 [4]: position, pool count, error, spare   */
  int32_t ring_slots; /* R = W + 2C */
  int32_t pool_slots; /* m - W */
} still_state_layout;

/* Kept tokens per decided chunk: min(C, floor((m - W) / T_max)).
 * Returns >= 0, or STILL_EINVAL. No device work. */
int still_lambda(const still_params* p);

/* Fills *out with the state layout. No device work. */
int still_state_layout_get(const still_params* p, still_state_layout* out);

/* Bytes of the state blob (batch * n_kv_heads units), or < 0 on error. */
int64_t still_state_bytes(const still_params* p);

/* Bytes of scratch needed by still_prefill for seq_len tokens (or by
 * still_decode_step when seq_len <= 0), or < 0 on error. */
int64_t still_workspace_bytes(const still_params* p, int64_t seq_len);

/* Prefill: runs the layer over seq_len >= 1 tokens (chunk-parallel form,
 * [P3 "Delayed Chunk-Level Selection ..."]) and writes
 *   out     [B, Hq, L, d]   outputs,
 *   sel_idx int32 [B, Hkv, n_dec, lambda], n_dec = (L-1)/C: positions kept
 *           from each decided chunk, ascending, -1 where the budget was full,
 *   score   float32 [B, Hkv, L] or NULL: scores (float32 evaluation; the
 *           routing metric's scores rounded once from float64 for the
 *           alternative metrics; an input for STILL_ROUTE_EXTERNAL),
 *   state   still_state_bytes(p) bytes: the decode state after token L-1.
 * q, k, v, fmap_w ([Hkv, d, d], phi uses x @ fmap_w[k]) and gate are read
 * only. workspace: ws_bytes >= still_workspace_bytes(p, seq_len), device
 * memory, contents need not be initialised. */
int still_prefill(const still_params* p, int64_t seq_len, const void* q, const void* k,
                  const void* v, const void* fmap_w, const float* gate, void* out,
                  int32_t* sel_idx, float* score, void* state, void* workspace,
                  size_t ws_bytes, void* stream);

/* still_prefill with a channel-wise sigmoid output gate [P4 "Synergizing
 * Linear and Sparse Attention: A Deep Dive into Hybrid LLM Architectures",
 * §4 Gating Mechanism]: out = y * sigmoid(out_gate), y the output
 * still_prefill writes. out_gate [B, Hq, L, d] holds the gate before the
 * sigmoid, in the params' dtype (read only, required, 16-byte aligned;
 * the caller computes it, e.g. as a projection of the layer input). The
 * gate is applied to the float32 merged output before the one rounding to
 * the output dtype. sel_idx, score and state are as for still_prefill;
 * same errors (a NULL out_gate returns STILL_EINVAL). */
int still_prefill_gated(const still_params* p, int64_t seq_len, const void* q, const void* k,
                        const void* v, const void* fmap_w, const float* gate,
                        const void* out_gate, void* out, int32_t* sel_idx, float* score,
                        void* state, void* workspace, size_t ws_bytes, void* stream);

/* still_prefill with a forget gate on the linear state (reading of the
 * gated linear attention of [P4 "Synergizing Linear and Sparse Attention:
 * A Deep Dive into Hybrid LLM Architectures", §2] with write strength 1,
 * applied to the NP-Map state of [P3 "NP-Map ..."]): the state decays by
 * decay[kv] every token, so a linear key j enters query t with weight
 * gate * decay^(t - j) * <phi(q), phi(k_j)>. decay: device float32 [Hkv],
 * values in (0, 1] (1 = the plain layer; other values are not checked and
 * give undefined results), 16-byte aligned, required. The exported state
 * holds decay^(R - j) phi(k_j) v_j^T, R the first position past the
 * chunks it covers; still_decode_step_decay continues it with the same
 * decay. Same outputs, workspace and errors as still_prefill otherwise;
 * STILL_FLAG_MERGE_SUM returns STILL_EUNSUPPORTED. */
int still_prefill_decay(const still_params* p, int64_t seq_len, const void* q, const void* k,
                        const void* v, const void* fmap_w, const float* gate, const float* decay,
                        void* out, int32_t* sel_idx, float* score, void* state, void* workspace,
                        size_t ws_bytes, void* stream);

/* still_prefill with the kept pool in pages (STILL_FLAG_PAGED_POOL set in
 * p->flags). pool_pages: the arena, n_pages pages of the params' dtype,
 * page = STILL_POOL_PAGE_ROWS key rows of d elements then as many value
 * rows (2 * 16 * d elements), 16-byte aligned, at most 2^31 bytes.
 * page_table: device int32 [B * Hkv][ceil((budget - window) / 16)], entry i
 * of unit u = b * Hkv + kv the arena page holding pool rows 16 i .. 16 i + 15
 * of that unit. The caller allocates and maps the pages (the library
 * allocates nothing): after a prefill of L tokens the pool holds
 * still_pool_rows(p, L) rows, whose pages must be mapped; an entry outside
 * [0, n_pages) for a needed row sets the state's error word (meta[2] =
 * STILL_ESTATE) and that row is not written. Outputs, selection, scores and
 * state as still_prefill otherwise. */
int still_prefill_paged(const still_params* p, int64_t seq_len, const void* q, const void* k,
                        const void* v, const void* fmap_w, const float* gate, void* out,
                        int32_t* sel_idx, float* score, void* state, void* pool_pages,
                        const int32_t* page_table, int64_t n_pages, void* workspace, size_t ws_bytes,
                        void* stream);

/* Rows of the kept pool once n_tokens tokens have been processed (prefill
 * or decode): lambda rows per decided chunk until the budget is full. For a
 * paged pool, the pages of rows [0, still_pool_rows(p, pos + 1)) must be
 * mapped before the decode step at position pos. < 0 on error. */
int64_t still_pool_rows(const still_params* p, int64_t n_tokens);

/* still_prefill with per-kernel timing, for benchmarks: for i < n_pairs it
 * records events[2i] before and events[2i+1] after the i-th kernel of the
 * prefill on `stream` (events are caller-created hipEvent_t handles; a NULL
 * handle is not recorded, so a caller can time some kernels only: every
 * recorded event costs the stream a drain). Kernel order: 0 F^T copy (made
 * by extra workgroups of the score launch, so its two events are recorded
 * back to back), 1 score, 2 select, 3 state deltas, 4 state scan,
 * 5 attention walk, 6 state export; a kernel not launched for a given
 * length gets its two events recorded back to back (so does 2, select, where
 * the score kernel decides the chunks: Self-Saliency routing with C <= 64).
 * n_pairs <= 7. Same
 * results and errors as still_prefill. */
int still_prefill_timed(const still_params* p, int64_t seq_len, const void* q, const void* k,
                        const void* v, const void* fmap_w, const float* gate, void* out,
                        int32_t* sel_idx, float* score, void* state, void* workspace,
                        size_t ws_bytes, void* stream, void* const* events, int n_pairs);

/* still_prefill that also returns the two branches apart, per (batch row,
 * query head, position), float32, [B, Hq, L, d] and [B, Hq, L]:
 *   y_sa   softmax-branch output sum_A e^s v / Z,  lse_sa = ln Z, Z = sum_A e^s
 *   y_la   linear-branch output  sum_B w v / D,    lse_la = ln D, D = sum_B w,
 *          w = <phi(q), phi(k)> without the gate (y_la = 0, lse_la = -inf
 *          where B(t) is empty)
 * so that the default output is (Z y_sa + g D y_la) / (Z + g D). out, sel_idx,
 * score and state are written as by still_prefill (with the params' merge);
 * the walk keeps the branches apart (slower). All four pointers are
 * required (16-byte aligned); STILL_FLAG_SOFTMAX_ONLY is rejected. */
int still_prefill_partials(const still_params* p, int64_t seq_len, const void* q, const void* k,
                           const void* v, const void* fmap_w, const float* gate, void* out,
                           int32_t* sel_idx, float* score, void* state, void* workspace,
                           size_t ws_bytes, void* stream, float* y_sa, float* lse_sa, float* y_la,
                           float* lse_la);

/* still_prefill without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the workspace is a static device array
 * of still_noalloc_scratch_bytes() bytes (64 MiB) inside the library, one per
 * GPU, held until the process ends. The call allocates nothing. Problems
 * whose still_workspace_bytes exceeds that size return STILL_ESCRATCH (e.g.
 * batch 1 at 32/8 heads, d = 128 fits up to L = 64K). Every call on a GPU
 * uses that GPU's one array: calls that overlap on one GPU (other streams,
 * other threads) race and give undefined results; serialise them. Same
 * outputs, errors and stream semantics as still_prefill otherwise (the
 * array needs no initialisation; nothing in it must start at zero). */
int still_prefill_noalloc(const still_params* p, int64_t seq_len, const void* q, const void* k,
                          const void* v, const void* fmap_w, const float* gate, void* out,
                          int32_t* sel_idx, float* score, void* state, void* stream);

/* Size in bytes of still_prefill_noalloc's static scratch. */
int64_t still_noalloc_scratch_bytes(void);

/* Decode one token per sequence at position pos (the state must hold
 * position pos, i.e. pos tokens already processed), [P3 "Delayed
 * Chunk-Level Selection ..."]: the same routing and memory update as the
 * prefill. q [B, Hq, d], k/v [B, Hkv, d]; out [B, Hq, d]; sel_new int32
 * [B, Hkv, lambda] receives the positions kept from chunk pos/C - 1 when
 * pos % C == 0 (and -1 otherwise or where the budget was full; may be NULL).
 * The state is updated in place. A position mismatch found on the device
 * sets the state's error word (meta[2] = STILL_ESTATE) and skips the step;
 * a mismatch between pos and C-boundaries is not possible to detect earlier
 * because the state lives on the device. workspace may be NULL when
 * still_workspace_bytes(p, 0) is 0. */
int still_decode_step(const still_params* p, int64_t pos, const void* q, const void* k,
                      const void* v, const void* fmap_w, const float* gate, void* state,
                      void* out, int32_t* sel_new, void* workspace, size_t ws_bytes,
                      void* stream);

/* still_decode_step with the channel-wise sigmoid output gate of
 * still_prefill_gated: out = y * sigmoid(out_gate), out_gate [B, Hq, d] in
 * the params' dtype (required, 16-byte aligned, read only). Needs no
 * workspace. Same state update, selection and errors as still_decode_step
 * (a NULL out_gate returns STILL_EINVAL). */
int still_decode_step_gated(const still_params* p, int64_t pos, const void* q, const void* k,
                            const void* v, const void* fmap_w, const float* gate,
                            const void* out_gate, void* state, void* out, int32_t* sel_new,
                            void* stream);

/* still_decode_step with the forget gate of still_prefill_decay: decay
 * device float32 [Hkv] in (0, 1] (required, 16-byte aligned, read only), the
 * same factors the state was built with; linear keys and the state are
 * weighted decay^(t - j), the chunk-boundary fold moves the state on by
 * decay^C. Needs no workspace. Same errors as still_decode_step (a NULL
 * decay returns STILL_EINVAL). */
int still_decode_step_decay(const still_params* p, int64_t pos, const void* q, const void* k,
                            const void* v, const void* fmap_w, const float* gate,
                            const float* decay, void* state, void* out, int32_t* sel_new,
                            void* stream);

/* still_decode_step with the kept pool in pages (STILL_FLAG_PAGED_POOL), the
 * arena and table as for still_prefill_paged: the step reads pool rows
 * [0, n_pool) and at a chunk boundary appends the kept tokens' rows, whose
 * pages must be mapped beforehand (still_pool_rows(p, pos + 1) rows in
 * all); an unmapped page sets the state's error word (meta[2] =
 * STILL_ESTATE) and skips the step. Same results and errors as
 * still_decode_step otherwise. */
int still_decode_step_paged(const still_params* p, int64_t pos, const void* q, const void* k,
                            const void* v, const void* fmap_w, const float* gate, void* state,
                            void* pool_pages, const int32_t* page_table, int64_t n_pages, void* out,
                            int32_t* sel_new, void* stream);

/* Ragged batches [P3 "Delayed Chunk-Level Selection ..."]: prefill and
 * decode keep one routing and memory-update rule per sequence, so each row
 * of a batch may be at its own length.
 *
 * still_prefill_varlen: rows of their own lengths seq_lens[b] >= 1 (host
 * array of p->batch entries). Every array is packed row after row: row b
 * starts after the tokens of rows 0 .. b-1 and is laid out as for a batch
 * of one ([H][L_b][d] for q, k, v and out; [Hkv][n_dec_b][lambda] for
 * sel_idx, n_dec_b = (L_b - 1) / C; [Hkv][L_b] for score). state is the
 * batch's state (still_state_bytes(p)); row b's units are b * Hkv .. b * Hkv
 * + Hkv - 1. workspace: ws_bytes >= still_workspace_bytes_varlen(p,
 * seq_lens). The rows run one after another on the stream (each one a
 * whole prefill). Same flags, results and errors as still_prefill; all
 * arguments are checked before the first row runs. */
int64_t still_workspace_bytes_varlen(const still_params* p, const int64_t* seq_lens);
int still_prefill_varlen(const still_params* p, const int64_t* seq_lens, const void* q,
                         const void* k, const void* v, const void* fmap_w, const float* gate,
                         void* out, int32_t* sel_idx, float* score, void* state, void* workspace,
                         size_t ws_bytes, void* stream);

/* n_tokens decode steps in one call (multi-token decode), each row at its
 * own position if asked. Token s of every row is q[s], k[s], v[s] ([n_tokens]
 * [B][H][d]) and writes out[s] ([n_tokens][B][Hq][d]) and, if sel_new is
 * not NULL, sel_new[s] ([n_tokens][B][Hkv][lambda], as for
 * still_decode_step). Positions: row_pos NULL: every row's token s is at pos
 * + s (pos >= 1, checked on the host); else row_pos is a device array of B
 * int32 and row b's token s is at row_pos[b] + s (pos is ignored). Positions
 * are checked against each unit's state on the device: a unit whose
 * position does not follow its state gets the error word (meta[2] =
 * STILL_ESTATE) and is skipped from then on; other rows go on. Steps run in
 * order on the stream. */
int still_decode_tokens(const still_params* p, int64_t pos, const int32_t* row_pos, int n_tokens,
                        const void* q, const void* k, const void* v, const void* fmap_w,
                        const float* gate, void* state, void* out, int32_t* sel_new,
                        void* stream);

/* Backward of one layer [P3 "Delayed Chunk-Level Selection for Unified
 * Training-Inference Parallelism": training runs the same chunk-parallel
 * form]: gradients of sum(y * dy) with respect to q, k, v, fmap_w and gate,
 * the routing held fixed (reading: which tokens are kept carries no
 * gradient; sel_idx is the forward's selection). Inputs: the forward's
 * inputs, its sel_idx, its float32 output y [B, Hq, L, d] (STILL_FLAG_
 * FP32_OUT), its branch log-normalisers lse_sa, lse_la [B, Hq, L] (from
 * still_prefill_partials) and dy [B, Hq, L, d] float32. Outputs (float32,
 * overwritten): dq [B, Hq, L, d], dk, dv [B, Hkv, L, d], dfmap [Hkv, d, d],
 * dgate [Hq]. Default merge only (the branch-variant flags return
 * STILL_EUNSUPPORTED). workspace: ws_bytes >= still_backward_workspace_bytes
 * (p, seq_len), 16-byte aligned. Chunked form, linear in L: the linear
 * branch through per-chunk prefix states (query side) and suffix states
 * (key side), the band and kept-pool pairs one by one. Accuracy: float32
 * arithmetic (float64 chunk scans) on top of the forward's y and
 * normalisers. */
int64_t still_backward_workspace_bytes(const still_params* p, int64_t seq_len);
int still_backward(const still_params* p, int64_t seq_len, const void* q, const void* k, const void* v,
                   const void* fmap_w, const float* gate, const int32_t* sel_idx, const float* y,
                   const float* lse_sa, const float* lse_la, const float* dy, float* dq, float* dk,
                   float* dv, float* dfmap, float* dgate, void* workspace, size_t ws_bytes,
                   void* stream);

/* Human-readable text of a status code (static storage). */
const char* still_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* STILL_H */
