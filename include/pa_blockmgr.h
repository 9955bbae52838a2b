/*
 * libpagedattn block manager: the host-side bookkeeping around the K/V pool.
 *
 * Pages cited (title, then slide / section on that page):
 *   [Slides]  "PagedAttention：让 KV cache 按需生长"
 *   [Serving] "PagedAttention 与在线推理：KV 分页、共享及调度的联合分析"
 *
 * It keeps the state the pages list ([Slides] "引用计数管理“谁还在读”，长度管理
 * “哪里能写”"):
 *   per request  block table (logical block -> physical block) and length
 *                (tokens whose K/V are written or reserved);
 *   per block    refcount (requests whose table holds it, not tokens) and a
 *                free queue of blocks with refcount 0.
 * Growth follows [Slides] "先确保分配成功，再改变可见状态": a full tail takes
 * a fresh block; a partly filled tail that another request also reads is
 * copied first (copy-on-write), the writer's table is switched to the copy,
 * and only then is the token written.  The manager decides and records;
 * the data movement is the caller's, with kv_cow_copy and kv_append of
 * pagedattn.h on one stream, copy before write.
 *
 * All operations are host-only (no device memory, no HIP calls) and
 * all-or-nothing: capacity is checked before any table changes ([Slides]
 * "三个空闲块，四个请求同时跨边界"), so a failed call leaves every table,
 * refcount and the free queue exactly as they were.  Not thread-safe: one
 * manager is driven by one thread.  Prefix caching of released blocks is not
 * modelled: a block whose refcount drops to 0 goes straight back to the free
 * queue ([Slides] "请求结束，块就能交给下一位").
 *
 * Errors use pa_status from pagedattn.h plus PA_ERR_NO_SPACE below;
 * pa_last_error() describes the failure.
 */
#ifndef PA_BLOCKMGR_H
#define PA_BLOCKMGR_H

#include <stdint.h>

#include "pagedattn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* The pool has fewer free blocks than the call needs; nothing was changed. */
#define PA_ERR_NO_SPACE ((pa_status)-5)

typedef struct pa_block_manager pa_block_manager;

/*
 * A pool of num_blocks physical blocks of block_size tokens; a request may
 * hold at most max_blocks_per_seq blocks (the row width of exported tables).
 * free_order (may be NULL) gives the order in which free blocks are handed
 * out: a permutation of 0 .. num_blocks-1 (NULL = ascending).  *out receives
 * the manager, owned by the caller until pa_bm_destroy.
 */
pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                       const int32_t* free_order, pa_block_manager** out);
void pa_bm_destroy(pa_block_manager* bm);

/* A new request with length 0 and an empty table; its id goes to *req. */
pa_status pa_bm_add_request(pa_block_manager* bm, int32_t* req);

/*
 * A new request that shares every block of `parent` (same table, same
 * length); each shared block's refcount grows by one ([Slides]
 * "只读时共用，要写入时再分开").  Takes no free block.
 */
pa_status pa_bm_fork(pa_block_manager* bm, int32_t parent, int32_t* child);

/*
 * End (finish or cancel) a request: its table is dropped and every block
 * whose refcount falls to 0 returns to the back of the free queue ([Slides]
 * "请求结束，块就能交给下一位"; a cancel must take this path too, or the
 * pool leaks).  Blocks other requests still read stay.
 */
pa_status pa_bm_release(pa_block_manager* bm, int32_t req);

/*
 * Grow request `req` by n_tokens (n_tokens >= 0), e.g. for a prefill.
 * If its tail block is partly filled and shared, the tail is first replaced
 * by a fresh private copy: *cow_src / *cow_dst / *cow_n receive the copy
 * (source block, destination block, valid slots), else *cow_n = 0.  Pointers
 * may be NULL only when the caller knows no copy can arise.
 */
pa_status pa_bm_reserve(pa_block_manager* bm, int32_t req, int32_t n_tokens, int32_t* cow_src,
                        int32_t* cow_dst, int32_t* cow_n);

/*
 * One decode step: reserve one token for each of the n requests in reqs
 * (distinct ids), in the given order.  positions[i] receives the logical
 * index of request i's new token (its length before the step), ready for
 * kv_append.  Copy-on-write pairs are appended to cow_src / cow_dst / cow_n
 * (arrays of at least n entries) and their count goes to *num_cow; enqueue
 * them with kv_cow_copy before the appends.  When two requests share a
 * partly filled tail, the first in reqs copies and the last one left
 * writes in place.
 */
pa_status pa_bm_prepare_append(pa_block_manager* bm, const int32_t* reqs, int32_t n, int32_t* positions,
                               int32_t* cow_src, int32_t* cow_dst, int32_t* cow_n, int32_t* num_cow);

/*
 * pa_bm_prepare_append with n_tokens >= 1 new tokens per request: a
 * speculative verification step or one chunk of a prompt ([Serving] §5).
 * positions[i] receives the logical index of request i's first new token,
 * ready for kv_append_tokens.  All or nothing over the whole step, with the
 * same copy-on-write order; n_tokens = 1 is pa_bm_prepare_append.
 */
pa_status pa_bm_prepare_extend(pa_block_manager* bm, const int32_t* reqs, int32_t n, int32_t n_tokens,
                               int32_t* positions, int32_t* cow_src, int32_t* cow_dst, int32_t* cow_n,
                               int32_t* num_cow);

/*
 * Roll request `req` back to its first new_length tokens (0 <= new_length
 * <= its length), e.g. to drop the draft tokens a verification step
 * rejected ([Serving] §5: speculative decoding writes KV positions that may
 * be taken back).  Table entries past ceil(new_length / B) drop one
 * reference each and join the free queue at refcount 0, in table order, as
 * in pa_bm_release.  The tail block stays: its slots at or past the new
 * length are dead, and the next growth overwrites them (or copies only the
 * valid slots first if the tail is shared).  Never fails for lack of space.
 */
pa_status pa_bm_truncate(pa_block_manager* bm, int32_t req, int32_t new_length);

/*
 * Export, for the n requests in reqs, host arrays ready to copy to the
 * device for the kernels: tables [n, max_blocks_per_seq] (entries past a
 * request's last block hold pad_block) and lens [n].
 */
pa_status pa_bm_export(const pa_block_manager* bm, const int32_t* reqs, int32_t n, int32_t* tables, int32_t* lens,
                       int32_t pad_block);

/* Queries: free blocks; refcount of a block; length and block count of a
 * request (-1 for an unknown id or block). */
int32_t pa_bm_num_free(const pa_block_manager* bm);
int32_t pa_bm_refcount(const pa_block_manager* bm, int32_t block);
int32_t pa_bm_length(const pa_block_manager* bm, int32_t req);
int32_t pa_bm_num_blocks(const pa_block_manager* bm, int32_t req);

/*
 * Consistency check ([Slides] "占用率只有 70%，为什么请求还是进不来？", the
 * conservation line): every block's refcount equals the number of tables
 * holding it, the free queue holds exactly the blocks with refcount 0, each
 * once, and referenced blocks + free blocks = pool capacity.  PA_OK or
 * PA_ERR_INVALID_ARG with the first violation in pa_last_error().
 */
pa_status pa_bm_check(const pa_block_manager* bm);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCKMGR_H */
