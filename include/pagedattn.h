/*
 * libpagedattn — paged-attention decode for AMD MI355X (gfx950), C ABI.
 *
 * Pages cited (title, then slide / section / equation on that page):
 *   [Slides]  "PagedAttention：让 KV cache 按需生长"
 *   [Budgets] "内存预算约束下的语言模型服务：注意力、分页与调度"
 *   [Serving] "PagedAttention 与在线推理：KV 分页、共享及调度的联合分析"
 *
 * Data layout (all row-major, all device memory owned by the caller):
 *   q             [S, Hq, d]            element type `dtype`
 *   k_pool/v_pool [NB, B, Hkv, d]       physical block, slot, KV head, dim — K and V
 *                                       in separate pools ([Slides] "把 token 6 变成
 *                                       真正的内存地址")
 *   block_tables  int32 [S, MB]         logical block -> physical block ([Slides]
 *                                       "顺序留在表里，数据放进空闲块")
 *   seq_lens      int32 [S]             tokens each request attends to
 *   out           float32 [S, Hq, d]
 * The several-token entry points (paged_attn_extend, kv_append_tokens) put a
 * token axis after the request axis: q and out [S, T, Hq, d], new K/V
 * [S, T, Hkv, d].
 *
 * Conventions shared by every entry point:
 *   - Pointers are device pointers unless stated; the library never allocates,
 *     frees or synchronises inside these calls.  Work is enqueued on `stream`
 *     (NULL = the default stream) and the call returns.
 *   - Arguments that live on the host (sizes, the dims struct) are validated
 *     before anything is enqueued; a failed check returns an error status and
 *     enqueues nothing.  pa_last_error() then describes the failure
 *     (thread-local, valid until the next call on that thread).
 *   - Values that live on the device (lengths, table entries, positions) are
 *     the caller's contract: tables must be published only after capacity was
 *     checked ([Slides] "三个空闲块，四个请求同时跨边界").  The kernels still
 *     never access memory outside the buffers described by `dims`: a request
 *     whose length exceeds MB*B, or whose table names a block outside [0, NB),
 *     gets NaN outputs; an append or copy that would leave the pool is skipped.
 *   - Query head h reads KV head h / (Hq / Hkv) (contiguous GQA groups).
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 4

/*
 * pa_dims.flags bits.
 *
 * PA_FLAG_BF16_WEIGHTS: in paged_attn_extend steps that take the bf16
 * shared-tile path (more query tokens than two sets of 16 matrix-core
 * columns hold), round each softmax weight p = 2^(s - m) once to bf16
 * (round to nearest even) for the p.v product, and sum the softmax
 * denominator from the same rounded weights on the matrix core.  The output
 * is then an exact weighted mean of V with weights within 2^-9 of the exact
 * ones, relative.  Without the flag each weight is carried as a bf16 head
 * plus a bf16 remainder (two p.v products, weights within 2^-18), which
 * costs a third more matrix-core work; measured on a 512-token prompt chunk
 * over 4096 positions: about 20 % less time, and a largest error of about
 * 2e-3 of max|out| against the exact attention instead of about 4e-6.
 * Every other path (decode, the fused append, fewer query tokens, float32)
 * ignores the flag and keeps the remainder.
 */
#define PA_FLAG_BF16_WEIGHTS 1

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1, /* null pointer, bad size, Hq % Hkv != 0, ... */
  PA_ERR_UNSUPPORTED = -2, /* a shape or dtype no kernel here is built for */
  PA_ERR_WORKSPACE = -3,   /* split-K workspace missing, misaligned or too small */
  PA_ERR_LAUNCH = -4       /* the HIP runtime refused the launch */
} pa_status;

typedef enum {
  PA_F32 = 0, /* IEEE binary32 */
  PA_BF16 = 1 /* bfloat16 (upper half of a binary32) */
} pa_dtype;

/* Shape descriptor.  Sizes are element counts. */
typedef struct {
  int32_t num_seqs;           /* S  >= 0 (0 makes every call a no-op)          */
  int32_t num_q_heads;        /* Hq >= 1                                       */
  int32_t num_kv_heads;       /* Hkv >= 1, Hq % Hkv == 0                       */
  int32_t head_dim;           /* d; the kernels support 128                    */
  int32_t max_blocks_per_seq; /* MB >= 1: row stride of block_tables          */
  int32_t num_blocks;         /* NB >= 1: blocks in each pool                  */
  pa_dtype dtype;             /* element type of q, pools, new K/V             */
  int32_t num_splits;         /* split-K parts: 0 = chosen by the library from
                                 host-known values (S, Hq, Hkv, MB, B, dtype,
                                 the query-token count and flags), >= 1 asks
                                 for that count (rounded as paged_attn_plan
                                 states)                                       */
  void* workspace;            /* device scratch for split-K partial states,
                                 256-byte aligned, caller-owned; may be NULL when
                                 paged_attn_plan reports 0 bytes                */
  size_t workspace_bytes;
  int32_t flags;              /* PA_FLAG_* bits; 0 for the defaults; any other
                                 bit is PA_ERR_INVALID_ARG                     */
  const int32_t* order;       /* optional, device [num_seqs]: the order in which
                                 the bf16 matrix-core decode kernel (which also
                                 runs paged_attn_extend steps of a few tokens)
                                 issues the requests' work, in launches of more
                                 than one round of resident work items
                                 (paged_attn_order writes longest first);
                                 NULL = request order.  A scheduling hint only:
                                 every output bit is the same with or without
                                 it.  Must be a permutation of 0..num_seqs-1;
                                 an entry outside [0, num_seqs) stands for its
                                 own position (never read out of bounds), a
                                 repeated entry leaves another request's rows
                                 unwritten.  Other kernels ignore it.          */
} pa_dims;

/* Library version of this header's ABI (PA_ABI_VERSION). */
int32_t pa_abi_version(void);

/* Human-readable name of a status code (static storage). */
const char* pa_status_string(pa_status status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* pa_last_error(void);

/*
 * Split-K plan for paged_attn_decode at block size B: the number of splits
 * the decode will use and the workspace it needs.  A history cut into
 * contiguous block ranges is attended range by range, and each range leaves
 * an online-softmax state (m, l, o) that a merge combines exactly ([Budgets]
 * eq. (4): the running max, the rescaled normaliser and the value
 * accumulator rescaled by the same factor).  The workspace holds the
 * partial states that reach the merge, float32 o [rows, P', d], then m and
 * l [rows, P'] (rows = S * T * Hq): P' = P with bf16; with float32 the
 * splits run in groups of up to 4 that merge inside one workgroup, so P' is
 * the number of groups, and no workspace is needed for up to 4 splits.  0
 * bytes when nothing reaches the merge.  Every call writes every partial
 * state it later reads, so the workspace never needs clearing.
 *
 * The plan depends only on host-known values: S, Hq, Hkv, MB, B, dtype,
 * the query-token count T (1 here) and dims->flags, never on lengths or
 * table contents, so repeated calls agree.  The table's MB * B slots are cut into units of
 * max(16, B) slots (16-slot tiles, whole blocks).
 *   - dims->num_splits = 0: enough splits to occupy the GPU's compute units
 *     given the work items (S * Hkv, times the token groups of T), but no
 *     split shorter than 256 slots with bf16 (16 with float32), and at least
 *     one.
 *   - dims->num_splits = P0 >= 1: P0 capped at the unit count.
 * The requested count P0 then becomes P = ceil(units / ceil(units / P0)):
 * each split takes ceil(units / P0) whole units, the last one the rest, and
 * splits that would hold no unit are dropped.  So a forced count may come
 * back smaller (MB * B = 160 slots at B = 16 is 10 units: 6 or 7 give 5).
 * Callers size the workspace, and read partial states, by the num_splits
 * returned here.
 */
pa_status paged_attn_plan(const pa_dims* dims, int32_t B, int32_t* num_splits,
                          size_t* workspace_bytes);

/*
 * Workspace bytes paged_attn_decode needs for dims (dims->num_splits as
 * given, 0 = the automatic plan) at block size B: the workspace_bytes
 * paged_attn_plan reports for the same arguments, returned directly.  The
 * workspace holds the mergeable (m, l, o) partial states of [Budgets]
 * eq. (4), one per split and output row.  Returns 0 when the decode needs
 * none, and SIZE_MAX when dims or B are rejected (pa_last_error() says why).
 */
size_t paged_attn_workspace_bytes(const pa_dims* dims, int32_t B);

/*
 * Longest-first order of a batch's requests, for dims->order: order[r] is
 * the request with the r-th longest history (seq_lens descending, equal
 * lengths by request index), a permutation of 0..S-1 written on stream.
 * Requests of different lengths share one batch ([Slides] "调度决定谁上场，
 * 分页决定住哪里"; the mixed-length batch of [Budgets] §5 draws lengths
 * uniformly from 1 to 512).  A decode launch with more work items than fit
 * on the GPU at once runs them in rounds as workgroups finish; issuing the
 * longest first (the longest-processing-time rule) leaves short items to
 * fill the end, so the last round is shorter.  Measured on 256 requests of
 * 1-513 tokens, 32 layers: 49.6 -> 47.6 us per layer.  The lengths do not
 * change between the layers of a step, so one call serves them all.
 *
 * seq_lens: device int32 [S], any values (compared as given); order: device
 * int32 [S], caller-owned, overwritten.  One launch of ceil(S / 256)
 * workgroups and S^2 comparisons.  S = 0 is a no-op; S < 0 or a NULL
 * pointer with S > 0 is PA_ERR_INVALID_ARG; S > 65536 is PA_ERR_UNSUPPORTED
 * (the comparisons grow as S^2: about 0.5 ms at that size).
 */
pa_status paged_attn_order(const int32_t* seq_lens, int32_t S, int32_t* order, hipStream_t stream);

/*
 * One decode step of one layer: for every request s and query head h,
 *   out[s,h,:] = sum_t softmax_t(scale * <q[s,h,:], K_s[t,g,:]>) * V_s[t,g,:],
 * t over the seq_lens[s] tokens of request s, g = h / (Hq/Hkv), where token t
 * lives in slot t % B of physical block block_tables[s][t / B] ([Slides]
 * "读 token 6，先查表，再找偏移").  Table entries at or past ceil(n/B) never
 * address the pools (their values may be anything; the row's MB entries must
 * be readable); slots of the last block at or past n are masked and their contents
 * never enter the result ([Slides] "分页以后，attention 仍然按完整历史归一化",
 * quiz "逻辑顺序没错，为什么 attention 输出还是错？").  Blocks are combined with
 * the online-softmax state of [Budgets] eq. (4); long histories are divided
 * into contiguous block ranges whose (m, l, o) states are merged afterwards,
 * so the result depends only on logical positions, never on physical ids.
 * A request with seq_lens[s] == 0 gets out = 0.
 *
 * B: block size in tokens: 4, 8, 16, 32 or 64 (the pages' block-size
 * trade-off, [Slides] "块越小，省下的是空位，多出来的是管理").  scale:
 * multiplies q.k (e.g. 1/sqrt(d)).  Accumulation is float32; out is float32.
 */
pa_status paged_attn_decode(const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_tables, const int32_t* seq_lens,
                            int32_t B, float scale, float* out, hipStream_t stream,
                            const pa_dims* dims);

/* Bytes of the static device scratch paged_attn_decode_noalloc uses (16 MiB). */
#define PA_NOALLOC_SCRATCH_BYTES (16 << 20)

/*
 * paged_attn_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and errors as paged_attn_decode, bit
 * for bit, except that dims->workspace and dims->workspace_bytes are ignored:
 * the split-K partial states go to a static device array inside the library,
 * PA_NOALLOC_SCRATCH_BYTES long, of which each GPU the library runs on holds
 * one copy until the process ends.  The caller still passes q, the pools, the
 * tables, the lengths and out.  Nothing is allocated or freed, here or in the
 * kernels; the first call on a device looks up that device's copy of the
 * array (hipGetSymbolAddress) and keeps its address.
 *   - A plan whose workspace (paged_attn_plan) exceeds the scratch returns
 *     PA_ERR_WORKSPACE and enqueues nothing: ask for fewer splits, or use
 *     paged_attn_decode with a workspace.
 *   - `stream` must belong to the current device (PA_ERR_INVALID_ARG
 *     otherwise).
 *   - Every call on one GPU shares that GPU's copy, and the kernels write
 *     every partial state before reading it, so nothing needs clearing
 *     between calls; but calls that overlap on one GPU (two streams, or two
 *     threads) race on it and may return wrong results.  Serialise them, for
 *     example on one stream.
 */
pa_status paged_attn_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                    const int32_t* block_tables, const int32_t* seq_lens, int32_t B, float scale,
                                    float* out, hipStream_t stream, const pa_dims* dims);

/*
 * One decode step with the step's token appended in the same call:
 * kv_append(k_pool, v_pool, k_new, v_new, block_tables, positions, B) then
 * paged_attn_decode(q, k_pool, v_pool, block_tables, seq_lens, B, scale,
 * out), with the same results bit for bit (the append order of [Slides]
 * "写满一块，再拿下一块" and the attention of paged_attn_decode).  k_new / v_new
 * are [S, Hkv, d] of `dtype`, positions int32 [S] (negative: no append for
 * that request), all device memory; seq_lens counts the appended token.
 * With bf16 one kernel does both: the work item that attends position
 * positions[s] of KV head g writes that head's row into the pool and uses
 * the new K/V for the position directly, so one launch replaces two.  With
 * float32 the two kernels run one after the other on `stream`.  The target
 * block must be in the table and privately owned (copy-on-write first, as
 * for kv_append).  Workspace and splits as for paged_attn_decode.
 */
pa_status paged_attn_decode_append(const void* q, const void* k_pool, const void* v_pool, const void* k_new,
                                   const void* v_new, const int32_t* block_tables, const int32_t* positions,
                                   const int32_t* seq_lens, int32_t B, float scale, float* out, hipStream_t stream,
                                   const pa_dims* dims);

/*
 * Split-K plan for paged_attn_extend with num_q_tokens (T >= 1) query tokens
 * per request; T = 1 gives paged_attn_plan's answer.  The workspace holds
 * partial states for S*T*Hq rows.  With bf16, when every query token of a
 * (request, KV head) fits one workgroup of the several-token kernels, a
 * plan of 2 splits (and of 4 where the tokens fill at most 96 (token, head)
 * columns per KV head, as 9-24 tokens of a 4-head group) runs them as the
 * parts of one workgroup that merge inside it: no workspace (0 bytes).  The
 * automatic plan takes 4 splits where it would take 2 when the tokens fill
 * 49-64 columns (13-16 tokens of a 4-head group; not with
 * PA_FLAG_BF16_WEIGHTS) or 65-96 columns (17-24 tokens).
 */
pa_status paged_attn_extend_plan(const pa_dims* dims, int32_t B, int32_t num_q_tokens, int32_t* num_splits,
                                 size_t* workspace_bytes);

/*
 * Attention of T = num_q_tokens new tokens per request over the paged
 * history: a speculative-verification step or one chunk of a prompt
 * ([Serving] §5 sets speculative decoding and tiled exact attention beside
 * paging).  The T tokens are already appended (kv_append_tokens) as the last
 * T of the seq_lens[s] = n positions; query token i sits at position n-T+i
 * and attends positions 0 .. n-T+i (itself and everything before it):
 *   out[s,i,h,:] = sum_{t <= n-T+i} softmax_t(scale * <q[s,i,h,:], K_s[t,g,:]>) * V_s[t,g,:]
 * with the addressing, masking and online-softmax merging of
 * paged_attn_decode.  A query whose position n-T+i is negative (n < T)
 * attends nothing and gets 0.  q and out are [S, T, Hq, d] (q of `dtype`,
 * out float32).  T = 1 is exactly paged_attn_decode.  Several (token, head)
 * pairs share each K/V byte read: with bf16, up to 32/G tokens of a G-head
 * group in one pass over the history (two sets of 16 matrix-core columns);
 * more tokens go to workgroups whose waves take different tokens and share
 * each K/V tile through LDS (16 or 32 tokens of a 4-head group per
 * workgroup), each workgroup streaming the history once.  With float32, 8/G
 * tokens per pass.  The workspace is sized by paged_attn_extend_plan.
 * dims->flags may carry PA_FLAG_BF16_WEIGHTS (the shared-tile path's faster,
 * less exact weights; see its definition above).
 */
pa_status paged_attn_extend(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_tables,
                            const int32_t* seq_lens, int32_t num_q_tokens, int32_t B, float scale, float* out,
                            hipStream_t stream, const pa_dims* dims);

/*
 * Append one token per request ([Slides] "写满一块，再拿下一块"):
 *   k_pool[block_tables[s][p / B], p % B, :, :] = k_new[s, :, :]   (p = positions[s])
 * and the same for V.  k_new/v_new are [S, Hkv, d] of `dtype`; positions is
 * int32 [S] on the device, the logical index the token takes (the request's
 * length before the write); a negative position skips the request.  The
 * target block must already be in the table and privately owned — a shared
 * tail is first copied with kv_cow_copy on the same stream ([Slides]
 * "先确保分配成功，再改变可见状态").  Bytes are copied exactly.
 */
pa_status kv_append(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                    const int32_t* block_tables, const int32_t* positions, int32_t B,
                    hipStream_t stream, const pa_dims* dims);

/*
 * kv_append in every layer at once ([Slides] "写满一块，再拿下一块"; all layers
 * share one block numbering, so the token's block and slot are the same in
 * each): for every layer l < num_layers,
 *   pool_l[block_tables[s][p / B], p % B, :, :] = new[l, s, :, :]   (p = positions[s])
 * for K and V, one launch.  k_new/v_new are [num_layers, S, Hkv, d] of
 * `dtype`; layer l's pool starts layer_stride_elems elements after layer
 * l-1's (num_layers = 1 ignores the stride and is kv_append).  For when the
 * new K/V of every layer are known together (restoring recomputed tokens, a
 * step whose projections ran ahead); a model computing one layer after the
 * other appends per layer, or with paged_attn_decode_append.  Positions,
 * ownership and skipping as for kv_append.  Bytes are copied exactly.
 */
pa_status kv_append_layers(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                           const int32_t* block_tables, const int32_t* positions, int32_t B, int32_t num_layers,
                           int64_t layer_stride_elems, hipStream_t stream, const pa_dims* dims);

/*
 * kv_append for T = num_tokens consecutive tokens per request (draft tokens
 * or a prompt chunk, [Serving] §5): k_new/v_new are [S, T, Hkv, d] and
 * token i of request s goes to logical position positions[s] + i.  A
 * negative positions[s] skips the request; the blocks of every position
 * written must already be in the table and private (pa_bm_prepare_extend
 * reserves them and reports the copies to make first).  T = 1 is kv_append.
 */
pa_status kv_append_tokens(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                           const int32_t* block_tables, const int32_t* positions, int32_t num_tokens, int32_t B,
                           hipStream_t stream, const pa_dims* dims);

/*
 * Copy-on-write of shared tail blocks ([Slides] "只读时共用，要写入时再分开",
 * "先确保分配成功，再改变可见状态"): for each pair i and each layer l,
 *   pool_l[dst_blocks[i], 0:n_valid[i], :, :] = pool_l[src_blocks[i], 0:n_valid[i], :, :]
 * for both K and V.  src_blocks, dst_blocks, n_valid are int32 [num_pairs] on
 * the device.  Layer l's pool starts layer_stride_elems elements after layer
 * l-1's (all layers share one block numbering, so a copied block is copied in
 * every layer); num_layers = 1 ignores the stride.  Slots at or past n_valid
 * and all other blocks are left untouched.  Destinations must be distinct
 * and differ from every source.  Enqueue it before the branch's kv_append on
 * the same stream: stream order makes the copy visible to the write.
 */
pa_status kv_cow_copy(void* k_pool, void* v_pool, const int32_t* src_blocks,
                      const int32_t* dst_blocks, const int32_t* n_valid, int32_t num_pairs,
                      int32_t B, int32_t num_layers, int64_t layer_stride_elems,
                      hipStream_t stream, const pa_dims* dims);

/*
 * Block swap ([Slides] "腾出显存以后，还要付一次恢复成本": a preempted
 * request's KV can be moved out and back in instead of recomputed).  Whole
 * blocks — all B slots, all KV heads, K and V, in every layer — move between
 * the pools and a contiguous buffer laid out
 *   buf[layer][pool: 0 = K, 1 = V][i][B][Hkv][d]   (dtype of the pools)
 * for the num_list block ids in `blocks` (int32, device).
 *   kv_swap_out: buf <- pools;   kv_swap_in: pools <- buf.
 * buf may be device memory or host memory the device can address (pinned,
 * e.g. hipHostMalloc); then the kernel reads or writes it across the host
 * link directly.  buf must be 16-byte aligned and hold
 * num_layers * 2 * num_list * B * Hkv * d elements.  Layers and strides as in
 * kv_cow_copy.  Ids outside [0, NB) are skipped.  Bytes are copied exactly;
 * nothing else in the pools changes.  A swap-in may target other block ids
 * than the swap-out (the caller's new table then points at them).
 */
pa_status kv_swap_out(const void* k_pool, const void* v_pool, const int32_t* blocks, int32_t num_list, void* buf,
                      int32_t B, int32_t num_layers, int64_t layer_stride_elems, hipStream_t stream,
                      const pa_dims* dims);
pa_status kv_swap_in(void* k_pool, void* v_pool, const int32_t* blocks, int32_t num_list, const void* buf, int32_t B,
                     int32_t num_layers, int64_t layer_stride_elems, hipStream_t stream, const pa_dims* dims);

/*
 * Debug helper, not on the decode path: materialise each request's history
 * contiguously through the same address computation the decode uses, the
 * address function of [Slides] "把 token 6 变成真正的内存地址" (logical token t
 * lives in slot t % B of the physical block the table names for logical
 * block t / B):
 *   k_out[s, t, :, :] = k_pool[block_tables[s][t / B], t % B, :, :]  for t < seq_lens[s]
 * k_out/v_out are [S, MB*B, Hkv, d] of `dtype`, device memory; positions
 * t >= seq_lens[s] are not written.  Lengths are clamped to [0, MB*B]; a table
 * entry outside [0, NB) leaves that block's positions unwritten.  Bytes are
 * copied exactly.  Errors: PA_ERR_INVALID_ARG for a NULL or misaligned
 * pointer, PA_ERR_UNSUPPORTED for MB > 65535.
 */
pa_status paged_kv_gather(const void* k_pool, const void* v_pool, const int32_t* block_tables,
                          const int32_t* seq_lens, int32_t B, void* k_out, void* v_out,
                          hipStream_t stream, const pa_dims* dims);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
