/*
 * lra.h -- C ABI of liblra.so: Flash-LoRA-Attention and the PreLRShared LR precompute on
 * AMD Instinct MI355X (gfx950).
 *
 * The method (LRAgent, "Resumen Técnico" on gist.science; PReCache abstract on arxivdaily):
 * a multi-LoRA agent system keeps ONE base KV cache, produced by the frozen pretrained
 * weights and shared by every agent, plus per agent a low-rank (LR) value cache
 * L_a = X·A_a of width r_a (the activations after the LoRA down-projection).  Agent a's
 * value cache is V_base + L_a·B_a, where B_a is its LoRA up-projection.  Attention for a
 * query of agent a is
 *
 *     O = P·V_base + (P·L_a)·B_a,     P = causal softmax(Q·K_baseᵀ / sqrt(head_dim)),
 *
 * the regrouping of P·(V_base + L_a·B_a) given in the LRAgent summary, section
 * "3. Flash-LoRA-Attention": L_a is never expanded to the full value width and B_a is
 * applied once per block of query rows.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - dtype: LRA_DTYPE_BF16 (all tensors bf16, fp32 accumulation, bf16 outputs rounded to
 *    nearest even) or LRA_DTYPE_F32 (all tensors and all arithmetic fp32).  One dtype per
 *    call.
 *  - "device" pointers point to GPU memory of the current HIP device; "host" arrays are
 *    read during the call only and may be reused or freed when it returns.  The caller
 *    owns every buffer; the library allocates no memory.
 *  - Layouts are row-major and token-major:
 *        Q, O            [q_rows,  n_q_heads,  head_dim]
 *        K_base, V_base  [kv_rows, n_kv_heads, head_dim]
 *        L_a             [kv_rows, r_a]   with row stride ldl[a] elements (>= r_a)
 *        B_a             [r_a, n_kv_heads*head_dim]   (column g*head_dim + j feeds kv head g,
 *                                                     lane j)
 *    q head h reads kv head h / (n_q_heads / n_kv_heads) (grouped-query attention).
 *  - Causal alignment is bottom-right: a request with q_len queries over k_len keys places
 *    query t at position k_len - q_len + t; it sees keys 0 .. k_len - q_len + t.
 *  - Work is queued on `stream` (a hipStream_t; NULL = the null stream) and the call
 *    returns without synchronising.  Device-side faults surface at the caller's next
 *    synchronisation.
 *  - Return value: LRA_OK, or an error code with a message from lra_last_error().
 *    Arguments are validated on the host before anything is queued; an invalid call
 *    queues nothing and leaves every output untouched.
 *  - Calls are reentrant.  Calls on different streams may run concurrently when their
 *    outputs and workspaces do not overlap.
 */
#ifndef LRA_H
#define LRA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum lra_status {
  LRA_OK = 0,
  LRA_ERR_INVALID = 1,      /* malformed arguments (null pointer, bad shape or range)       */
  LRA_ERR_UNSUPPORTED = 2,  /* well-formed but not implemented (see limits below)           */
  LRA_ERR_WORKSPACE = 3,    /* workspace pointer null or smaller than the call needs        */
  LRA_ERR_HIP = 4           /* the HIP runtime reported an error while queueing work        */
};

enum lra_dtype { LRA_DTYPE_F32 = 0, LRA_DTYPE_BF16 = 1 };

/* Implementation limits (LRA_ERR_UNSUPPORTED beyond them). */
#define LRA_MAX_AGENTS 16      /* adapters per call                                          */
#define LRA_MAX_RANK 64        /* r_a <= 64 and r_a % 8 == 0 (r_a == 0 means no adapter)      */
#define LRA_MAX_GROUP 8        /* n_q_heads / n_kv_heads                                    */
#define LRA_MAX_BATCH 1024     /* requests per call                                          */
/* bf16 attention also needs 64 K/V rows (n_kv_heads * head_dim * 2 bytes each) and 64 rows
 * of each LR cache (ldl[a] * 2 bytes each) to stay below 2 GiB: tiles are addressed with
 * 32-bit byte offsets. */

/*
 * lra_precompute_lr -- PreLRShared LR precompute (PReCache abstract, English text on the
 * arxivdaily page: the LR caches of all agents are computed on the first pass over the
 * shared context; LRAgent summary, section 2, BaseShared: the LR cache of agent a holds
 * X·A_a, r_a values per token).
 *
 *     L_a[t, :] = X[t, :] · A_cat[:, off_a : off_a + r_a],   off_a = r_0 + ... + r_{a-1}
 *
 * for every token t < T and agent a < n_agents, computed in one pass over X.
 *   X        device [T, d_model], row stride ldx elements (>= d_model)
 *   A_cat    device [d_model, sum(r_a)], row stride lda elements (>= sum(r_a)):
 *            the agents' down-projections side by side
 *   ranks    host   [n_agents]
 *   L_out    host   [n_agents] array of device pointers; L_out[a] is [T, r_a] with row
 *            stride ldl[a] elements (>= r_a).  Outputs may be column blocks of one buffer.
 *   ldl      host   [n_agents]
 * Requires d_model % 8 == 0, ldx % 8 == 0, sum(r_a) <= 256, a 16-byte aligned X, and for
 * bf16 also d_model % 64 == 0, lda % 8 == 0 and a 16-byte aligned A_cat.  Outputs are rounded to the dtype
 * (bf16: nearest even) from fp32 accumulation.  T == 0 is a no-op.
 */
int lra_precompute_lr(int dtype, int64_t T, int64_t d_model,
                      const void* X, int64_t ldx,
                      const void* A_cat, int64_t lda,
                      int32_t n_agents, const int32_t* ranks,
                      void* const* L_out, const int64_t* ldl,
                      void* stream);

/*
 * lra_append_lr -- decode-step append to the LR caches.  PreLRShared keeps every agent's
 * LR cache over the shared context (PReCache abstract; LRAgent summary, section 2), so when
 * new tokens are generated every agent's cache gains their rows, and no agent needs an LR
 * prefill when it takes over:
 *
 *     L_a[rows[b], :] = X[b, :] · A_cat[:, off_a : off_a + r_a]
 *
 * for every new token b < batch and agent a < n_agents.
 *   X        device [batch, d_model], row stride ldx: the new tokens' hidden states
 *   A_cat, ranks, ldl: as for lra_precompute_lr
 *   L_out    host [n_agents] array of device pointers; L_out[a] is [l_rows, r_a] with row
 *            stride ldl[a]
 *   rows     host [batch]: the cache row of token b, distinct, in [0, l_rows)
 *   workspace  device scratch of at least lra_append_workspace_bytes(...) bytes, 16-byte
 *            aligned (may be NULL when that size is 0; it is 0 for fp32): the bf16 path
 *            splits d_model across workgroups and adds their fp32 partial sums there in a
 *            fixed order, so results are deterministic.  Its contents on entry do not
 *            matter; calls that may overlap in time need separate workspaces.
 * Only the rows listed are written.  Same requirements as lra_precompute_lr, and batch <=
 * LRA_MAX_BATCH; duplicate or out-of-range rows are LRA_ERR_INVALID, a missing or short
 * workspace LRA_ERR_WORKSPACE.  The base K/V rows of the new tokens come from the model's
 * own projections and are appended by the caller.  batch == 0 is a no-op.
 */
int lra_append_lr(int dtype, int32_t batch, int64_t d_model,
                  const void* X, int64_t ldx,
                  const void* A_cat, int64_t lda,
                  int32_t n_agents, const int32_t* ranks,
                  void* const* L_out, const int64_t* ldl,
                  const int32_t* rows, int64_t l_rows,
                  void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * lra_append_workspace_bytes -- scratch bytes lra_append_lr needs with these arguments
 * (ranks: host [n_agents]).  Returns 0 when no scratch is needed (fp32, batch 0, all ranks
 * 0), and (size_t)-1 when lra_append_lr would refuse them: a dtype, batch, agent count,
 * rank, sum of ranks or d_model outside its rules.
 */
size_t lra_append_workspace_bytes(int dtype, int32_t batch, int64_t d_model,
                                  int32_t n_agents, const int32_t* ranks);

/*
 * lra_attn_prefill -- Flash-LoRA-Attention over a batch of requests (LRAgent summary,
 * section 3).  Request b:
 *   query rows  [q_start[b], q_start[b] + q_len[b])  of Q and O,
 *   key rows    [k_start[b], k_start[b] + k_len[b])  of K_base, V_base and L_{agent_idx[b]},
 *   with 0 <= q_len[b] <= k_len[b] (q_len[b] == 0: nothing to do for b).
 * Requests may read the same key rows (a shared context: the BaseShared scheme); their
 * query/output rows must not overlap.  Every L_a may alias one buffer (one LR cache for
 * all agents: the BaseLRShared scheme).
 *
 *   n_q_heads % n_kv_heads == 0, n_q_heads / n_kv_heads <= LRA_MAX_GROUP,
 *   head_dim in {64, 128}.
 *   q_start, q_len, k_start, k_len, agent_idx   host [batch]
 *   Q, O            device [q_rows, n_q_heads, head_dim]   (16-byte aligned)
 *   K_base, V_base  device [kv_rows, n_kv_heads, head_dim] (16-byte aligned)
 *   ranks           host [n_agents], each 0 or a multiple of 8 up to LRA_MAX_RANK
 *   L               host [n_agents] array of device pointers, L[a] is [kv_rows, ldl[a]]
 *                   (16-byte aligned; ldl[a] % 8 == 0 for bf16, % 4 == 0 for fp32)
 *   B               host [n_agents] array of device pointers, B[a] is [r_a, n_kv_heads*head_dim]
 *   workspace       device scratch of at least lra_attn_workspace_bytes(...) bytes (may be
 *                   NULL when that size is 0); its contents on entry do not matter.
 */
int lra_attn_prefill(int dtype, int32_t batch,
                     int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                     const int32_t* q_start, const int32_t* q_len,
                     const int32_t* k_start, const int32_t* k_len,
                     const int32_t* agent_idx,
                     const void* Q, int64_t q_rows,
                     const void* K_base, const void* V_base, int64_t kv_rows,
                     int32_t n_agents, const int32_t* ranks,
                     const void* const* L, const int64_t* ldl,
                     const void* const* B,
                     void* O,
                     void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * lra_attn_decode -- one new query token per request: the lra_attn_prefill contract with
 * q_start[b] = b and q_len[b] = 1, i.e. Q and O are [batch, n_q_heads, head_dim] and the
 * token sits at the last key position k_len[b] - 1.  Runs as a split-K pass over the key
 * rows followed by a combine pass that merges the partial softmax states and applies B
 * once per query.
 */
int lra_attn_decode(int dtype, int32_t batch,
                    int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                    const int32_t* k_start, const int32_t* k_len,
                    const int32_t* agent_idx,
                    const void* Q,
                    const void* K_base, const void* V_base, int64_t kv_rows,
                    int32_t n_agents, const int32_t* ranks,
                    const void* const* L, const int64_t* ldl,
                    const void* const* B,
                    void* O,
                    void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * Comparators of the regrouping (LRAgent summary, section "3. Flash-LoRA-Attention": the
 * naive reconstruction expands the LR term V_lr·B to the full value width, work that
 * scales with r·d_out per key, and keeps a full-width value cache per agent).  They give
 * the same attention output by the ungrouped route, for measuring the regrouped kernels
 * against; bf16 only (LRA_DTYPE_F32 is LRA_ERR_UNSUPPORTED).
 *
 * lra_expand_values -- the agent's full-width values, materialised:
 *     V_full[s, g, :] = V_base[s, g, :] + L_a[s, :] · B_a[:, g*head_dim : (g+1)*head_dim]
 * for every row s of span i, s in [start[i], start[i] + len[i]), with a = agent_idx[i],
 * from fp32 accumulation rounded to bf16 (nearest even).  Rows outside the spans are left
 * untouched.
 *   start, len, agent_idx   host [n_spans]; spans must not overlap and lie in [0, kv_rows)
 *   V_base, V_full          device [kv_rows, n_kv_heads, head_dim] (16-byte aligned);
 *                           V_full may be V_base itself (in place), else must not overlap it
 *   ranks, L, ldl, B        the adapters, as for lra_attn_prefill
 * Plain attention over V_full (lra_attn_prefill / lra_attn_decode with rank-0 adapters)
 * then completes the naive route.
 */
int lra_expand_values(int dtype, int32_t n_spans,
                      const int32_t* start, const int32_t* len, const int32_t* agent_idx,
                      const void* V_base, int64_t kv_rows,
                      int32_t n_kv_heads, int32_t head_dim,
                      int32_t n_agents, const int32_t* ranks,
                      const void* const* L, const int64_t* ldl,
                      const void* const* B,
                      void* V_full,
                      void* stream);

/*
 * lra_attn_prefill_expand, lra_attn_decode_expand -- the in-tile expansion route: the
 * arguments, results and workspace of lra_attn_prefill / lra_attn_decode, but each tile of
 * V_base rows is expanded to full width in on-chip memory, V_tile + L_tile·B_g (rounded to
 * bf16), before P·V, instead of carrying P·L and applying B once per block of query rows.
 * Requests are not grouped by shared context (one expanded tile serves one agent).
 */
int lra_attn_prefill_expand(int dtype, int32_t batch,
                            int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                            const int32_t* q_start, const int32_t* q_len,
                            const int32_t* k_start, const int32_t* k_len,
                            const int32_t* agent_idx,
                            const void* Q, int64_t q_rows,
                            const void* K_base, const void* V_base, int64_t kv_rows,
                            int32_t n_agents, const int32_t* ranks,
                            const void* const* L, const int64_t* ldl,
                            const void* const* B,
                            void* O,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

int lra_attn_decode_expand(int dtype, int32_t batch,
                           int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                           const int32_t* k_start, const int32_t* k_len,
                           const int32_t* agent_idx,
                           const void* Q,
                           const void* K_base, const void* V_base, int64_t kv_rows,
                           int32_t n_agents, const int32_t* ranks,
                           const void* const* L, const int64_t* ldl,
                           const void* const* B,
                           void* O,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * lra_attn_decode_noalloc -- lra_attn_decode for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments and results without `workspace`.  The split-key scratch is a fixed
 * array of LRA_NOALLOC_SCRATCH_BYTES bytes inside this library, one copy per GPU, held
 * until the process ends; the call allocates nothing.  A call whose plan needs more scratch
 * (lra_attn_workspace_bytes(dtype, 1, ...) above the limit) returns LRA_ERR_WORKSPACE and
 * queues nothing.  The scratch needs no initial contents.  Every call on one GPU uses that
 * GPU's single array, so two calls whose work may overlap in time on one GPU (other
 * streams, or other host threads) race on it and must be ordered by the caller; calls
 * queued on one stream are ordered already.
 */
#define LRA_NOALLOC_SCRATCH_BYTES (32u << 20)
int lra_attn_decode_noalloc(int dtype, int32_t batch,
                            int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                            const int32_t* k_start, const int32_t* k_len,
                            const int32_t* agent_idx,
                            const void* Q,
                            const void* K_base, const void* V_base, int64_t kv_rows,
                            int32_t n_agents, const int32_t* ranks,
                            const void* const* L, const int64_t* ldl,
                            const void* const* B,
                            void* O,
                            void* stream);

/*
 * lra_attn_workspace_bytes -- scratch bytes the call with these arguments needs
 * (is_decode = 0: lra_attn_prefill, 1: lra_attn_decode; q_len is ignored for decode and
 * may be NULL).  max_rank is the largest r_a of the call.  Returns 0 when no scratch is
 * needed, and (size_t)-1 when the arguments are invalid.
 */
size_t lra_attn_workspace_bytes(int dtype, int is_decode, int32_t batch,
                                const int32_t* q_len, const int32_t* k_len,
                                int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                int32_t max_rank);

/* Message describing the calling thread's last non-OK status ("" if none). */
const char* lra_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LRA_H */
