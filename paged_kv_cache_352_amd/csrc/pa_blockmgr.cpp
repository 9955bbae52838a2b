// Host-side block manager of libpagedattn (declared in include/pa_blockmgr.h).
//
// [Slides] = "PagedAttention：让 KV cache 按需生长"
//
// State ([Slides] "引用计数管理“谁还在读”，长度管理“哪里能写”"): each request
// has a block table and a length; each physical block has a refcount (how
// many tables hold it); blocks with refcount 0 sit in a FIFO free queue.
// Invariant kept by every operation: a request of length L holds exactly
// ceil(L / B) blocks.
//
// Every mutating call first computes how many free blocks it needs, and only
// when the pool has them does it change anything ([Slides] "先确保分配成功，
// 再改变可见状态" and "三个空闲块，四个请求同时跨边界"); otherwise it returns
// PA_ERR_NO_SPACE with all state untouched.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_blockmgr.h"
#include "pa_internal.h"

namespace {

struct Request {
  std::vector<int32_t> table;
  int32_t length = 0;
};

pa_status err(pa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pa_status err(pa_status st, const char* fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  pa::set_last_error(buf);
  return st;
}

int64_t blocks_for(int64_t tokens, int32_t B) { return (tokens + B - 1) / B; }

}  // namespace

struct pa_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  int32_t max_blocks = 0;
  std::vector<int32_t> refcount;
  std::deque<int32_t> free_q;
  std::unordered_map<int32_t, Request> reqs;
  int32_t next_id = 0;

  Request* find(int32_t id) {
    auto it = reqs.find(id);
    return it == reqs.end() ? nullptr : &it->second;
  }
  const Request* find(int32_t id) const {
    auto it = reqs.find(id);
    return it == reqs.end() ? nullptr : &it->second;
  }

  int32_t take() {  // caller has checked that the queue is long enough
    const int32_t b = free_q.front();
    free_q.pop_front();
    refcount[b] = 1;
    return b;
  }

  // Free blocks needed to grow r by n > 0 tokens, given the refcount the tail
  // has at that moment; *cow says whether the tail must be copied first.
  int64_t need(const Request& r, int64_t n, int32_t tail_refcount, bool* cow) const {
    *cow = (r.length % block_size != 0) && tail_refcount > 1;
    return (*cow ? 1 : 0) + blocks_for(r.length + n, block_size) - (int64_t)r.table.size();
  }

  // Grow r by n tokens; the pool is known to have the blocks.  A shared,
  // partly filled tail is replaced by a private copy first.
  void grow(Request& r, int32_t n, int32_t* cs, int32_t* cd, int32_t* cn) {
    if (cn) *cn = 0;
    if (n == 0) return;
    if (r.length % block_size != 0 && refcount[r.table.back()] > 1) {
      const int32_t tail = r.table.back();
      const int32_t fresh = take();
      refcount[tail] -= 1;
      r.table.back() = fresh;
      if (cs) *cs = tail;
      if (cd) *cd = fresh;
      if (cn) *cn = r.length % block_size;
    }
    const int64_t want = blocks_for((int64_t)r.length + n, block_size);
    while ((int64_t)r.table.size() < want) r.table.push_back(take());
    r.length += n;
  }
};

extern "C" {

pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                       const int32_t* free_order, pa_block_manager** out) {
  pa::set_last_error("");
  if (!out) return err(PA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (num_blocks < 1 || block_size < 1 || max_blocks_per_seq < 1)
    return err(PA_ERR_INVALID_ARG, "num_blocks, block_size and max_blocks_per_seq must be >= 1");
  try {
    auto* bm = new pa_block_manager();
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->max_blocks = max_blocks_per_seq;
    bm->refcount.assign(num_blocks, 0);
    if (free_order) {
      std::vector<uint8_t> seen(num_blocks, 0);
      for (int32_t i = 0; i < num_blocks; ++i) {
        const int32_t b = free_order[i];
        if (b < 0 || b >= num_blocks || seen[b]) {
          delete bm;
          return err(PA_ERR_INVALID_ARG, "free_order is not a permutation of 0..%d (entry %d = %d)", num_blocks - 1,
                     i, b);
        }
        seen[b] = 1;
        bm->free_q.push_back(b);
      }
    } else {
      for (int32_t b = 0; b < num_blocks; ++b) bm->free_q.push_back(b);
    }
    *out = bm;
    return PA_OK;
  } catch (const std::bad_alloc&) {
    return err(PA_ERR_INVALID_ARG, "out of host memory");
  }
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

pa_status pa_bm_add_request(pa_block_manager* bm, int32_t* req) {
  pa::set_last_error("");
  if (!bm || !req) return err(PA_ERR_INVALID_ARG, "NULL argument");
  try {
    const int32_t id = bm->next_id++;
    bm->reqs.emplace(id, Request{});
    *req = id;
    return PA_OK;
  } catch (const std::bad_alloc&) {
    return err(PA_ERR_INVALID_ARG, "out of host memory");
  }
}

pa_status pa_bm_fork(pa_block_manager* bm, int32_t parent, int32_t* child) {
  pa::set_last_error("");
  if (!bm || !child) return err(PA_ERR_INVALID_ARG, "NULL argument");
  const Request* p = bm->find(parent);
  if (!p) return err(PA_ERR_INVALID_ARG, "unknown request %d", parent);
  try {
    Request copy = *p;
    const int32_t id = bm->next_id++;
    for (int32_t b : copy.table) bm->refcount[b] += 1;
    bm->reqs.emplace(id, std::move(copy));
    *child = id;
    return PA_OK;
  } catch (const std::bad_alloc&) {
    return err(PA_ERR_INVALID_ARG, "out of host memory");
  }
}

pa_status pa_bm_release(pa_block_manager* bm, int32_t req) {
  pa::set_last_error("");
  if (!bm) return err(PA_ERR_INVALID_ARG, "NULL manager");
  Request* r = bm->find(req);
  if (!r) return err(PA_ERR_INVALID_ARG, "unknown request %d", req);
  for (int32_t b : r->table) {
    if (--bm->refcount[b] == 0) bm->free_q.push_back(b);
  }
  bm->reqs.erase(req);
  return PA_OK;
}

pa_status pa_bm_reserve(pa_block_manager* bm, int32_t req, int32_t n_tokens, int32_t* cow_src, int32_t* cow_dst,
                        int32_t* cow_n) {
  pa::set_last_error("");
  if (!bm) return err(PA_ERR_INVALID_ARG, "NULL manager");
  Request* r = bm->find(req);
  if (!r) return err(PA_ERR_INVALID_ARG, "unknown request %d", req);
  if (n_tokens < 0) return err(PA_ERR_INVALID_ARG, "n_tokens = %d < 0", n_tokens);
  if (cow_n) *cow_n = 0;
  if (n_tokens == 0) return PA_OK;
  if ((int64_t)r->length + n_tokens > (int64_t)bm->max_blocks * bm->block_size)
    return err(PA_ERR_INVALID_ARG, "request %d would exceed %d blocks", req, bm->max_blocks);
  bool cow = false;
  const int32_t tail_rc = r->table.empty() ? 0 : bm->refcount[r->table.back()];
  const int64_t need = bm->need(*r, n_tokens, tail_rc, &cow);
  if (cow && (!cow_src || !cow_dst || !cow_n))
    return err(PA_ERR_INVALID_ARG, "request %d needs a copy-on-write but the copy outputs are NULL", req);
  if (need > (int64_t)bm->free_q.size())
    return err(PA_ERR_NO_SPACE, "request %d needs %lld free blocks, the pool has %zu", req, (long long)need,
               bm->free_q.size());
  bm->grow(*r, n_tokens, cow_src, cow_dst, cow_n);
  return PA_OK;
}

pa_status pa_bm_prepare_extend(pa_block_manager* bm, const int32_t* reqs, int32_t n, int32_t n_tokens,
                               int32_t* positions, int32_t* cow_src, int32_t* cow_dst, int32_t* cow_n,
                               int32_t* num_cow) {
  pa::set_last_error("");
  if (!bm || !num_cow) return err(PA_ERR_INVALID_ARG, "NULL argument");
  *num_cow = 0;
  if (n < 0) return err(PA_ERR_INVALID_ARG, "n = %d < 0", n);
  if (n_tokens < 1) return err(PA_ERR_INVALID_ARG, "n_tokens = %d < 1", n_tokens);
  if (n == 0) return PA_OK;
  if (!reqs || !positions || !cow_src || !cow_dst || !cow_n) return err(PA_ERR_INVALID_ARG, "NULL array");
  try {
    // Dry run in request order: tails of shared blocks lose one reader at
    // each copy, so a later sharer of the same tail may write in place.
    std::unordered_map<int32_t, int32_t> tail_rc;  // refcount a tail has at this point of the step
    std::unordered_map<int32_t, int32_t> seen;
    int64_t need = 0;
    for (int32_t i = 0; i < n; ++i) {
      const Request* r = bm->find(reqs[i]);
      if (!r) return err(PA_ERR_INVALID_ARG, "unknown request %d", reqs[i]);
      if (!seen.emplace(reqs[i], i).second) return err(PA_ERR_INVALID_ARG, "request %d listed twice", reqs[i]);
      if ((int64_t)r->length + n_tokens > (int64_t)bm->max_blocks * bm->block_size)
        return err(PA_ERR_INVALID_ARG, "request %d would exceed %d blocks", reqs[i], bm->max_blocks);
      int32_t rc = 0;
      if (!r->table.empty()) {
        const int32_t tail = r->table.back();
        auto it = tail_rc.find(tail);
        rc = it != tail_rc.end() ? it->second : bm->refcount[tail];
      }
      bool cow = false;
      need += bm->need(*r, n_tokens, rc, &cow);
      if (cow) tail_rc[r->table.back()] = rc - 1;
    }
    if (need > (int64_t)bm->free_q.size())
      return err(PA_ERR_NO_SPACE, "the step needs %lld free blocks, the pool has %zu", (long long)need,
                 bm->free_q.size());
    for (int32_t i = 0; i < n; ++i) {
      Request& r = *bm->find(reqs[i]);
      positions[i] = r.length;
      int32_t cs = -1, cd = -1, cn = 0;
      bm->grow(r, n_tokens, &cs, &cd, &cn);
      if (cn > 0) {
        cow_src[*num_cow] = cs;
        cow_dst[*num_cow] = cd;
        cow_n[*num_cow] = cn;
        *num_cow += 1;
      }
    }
    return PA_OK;
  } catch (const std::bad_alloc&) {
    return err(PA_ERR_INVALID_ARG, "out of host memory");
  }
}

pa_status pa_bm_prepare_append(pa_block_manager* bm, const int32_t* reqs, int32_t n, int32_t* positions,
                               int32_t* cow_src, int32_t* cow_dst, int32_t* cow_n, int32_t* num_cow) {
  return pa_bm_prepare_extend(bm, reqs, n, 1, positions, cow_src, cow_dst, cow_n, num_cow);
}

pa_status pa_bm_truncate(pa_block_manager* bm, int32_t req, int32_t new_length) {
  pa::set_last_error("");
  if (!bm) return err(PA_ERR_INVALID_ARG, "NULL manager");
  Request* r = bm->find(req);
  if (!r) return err(PA_ERR_INVALID_ARG, "unknown request %d", req);
  if (new_length < 0 || new_length > r->length)
    return err(PA_ERR_INVALID_ARG, "new length %d outside [0, %d]", new_length, r->length);
  const size_t keep = (size_t)blocks_for(new_length, bm->block_size);
  for (size_t j = keep; j < r->table.size(); ++j) {
    const int32_t b = r->table[j];
    if (--bm->refcount[b] == 0) bm->free_q.push_back(b);
  }
  r->table.resize(keep);
  r->length = new_length;
  return PA_OK;
}

pa_status pa_bm_export(const pa_block_manager* bm, const int32_t* reqs, int32_t n, int32_t* tables, int32_t* lens,
                       int32_t pad_block) {
  pa::set_last_error("");
  if (!bm) return err(PA_ERR_INVALID_ARG, "NULL manager");
  if (n < 0) return err(PA_ERR_INVALID_ARG, "n = %d < 0", n);
  if (n > 0 && (!reqs || !tables || !lens)) return err(PA_ERR_INVALID_ARG, "NULL array");
  for (int32_t i = 0; i < n; ++i)
    if (!bm->find(reqs[i])) return err(PA_ERR_INVALID_ARG, "unknown request %d", reqs[i]);
  for (int32_t i = 0; i < n; ++i) {
    const Request& r = *bm->find(reqs[i]);
    int32_t* row = tables + (int64_t)i * bm->max_blocks;
    std::fill(row, row + bm->max_blocks, pad_block);
    std::copy(r.table.begin(), r.table.end(), row);
    lens[i] = r.length;
  }
  return PA_OK;
}

int32_t pa_bm_num_free(const pa_block_manager* bm) { return bm ? (int32_t)bm->free_q.size() : -1; }

int32_t pa_bm_refcount(const pa_block_manager* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->refcount[block];
}

int32_t pa_bm_length(const pa_block_manager* bm, int32_t req) {
  const Request* r = bm ? bm->find(req) : nullptr;
  return r ? r->length : -1;
}

int32_t pa_bm_num_blocks(const pa_block_manager* bm, int32_t req) {
  const Request* r = bm ? bm->find(req) : nullptr;
  return r ? (int32_t)r->table.size() : -1;
}

pa_status pa_bm_check(const pa_block_manager* bm) {
  pa::set_last_error("");
  if (!bm) return err(PA_ERR_INVALID_ARG, "NULL manager");
  std::vector<int32_t> holders(bm->num_blocks, 0);
  for (const auto& kv : bm->reqs) {
    const Request& r = kv.second;
    if ((int64_t)r.table.size() != blocks_for(r.length, bm->block_size))
      return err(PA_ERR_INVALID_ARG, "request %d: %zu blocks for length %d", kv.first, r.table.size(), r.length);
    for (int32_t b : r.table) {
      if (b < 0 || b >= bm->num_blocks) return err(PA_ERR_INVALID_ARG, "request %d holds block %d", kv.first, b);
      holders[b] += 1;
    }
  }
  std::vector<int32_t> in_free(bm->num_blocks, 0);
  for (int32_t b : bm->free_q) {
    if (b < 0 || b >= bm->num_blocks) return err(PA_ERR_INVALID_ARG, "free queue holds block %d", b);
    in_free[b] += 1;
  }
  int64_t referenced = 0;
  for (int32_t b = 0; b < bm->num_blocks; ++b) {
    if (holders[b] != bm->refcount[b])
      return err(PA_ERR_INVALID_ARG, "block %d: refcount %d but %d tables hold it", b, bm->refcount[b], holders[b]);
    if (in_free[b] != (bm->refcount[b] == 0 ? 1 : 0))
      return err(PA_ERR_INVALID_ARG, "block %d: refcount %d, %d times in the free queue", b, bm->refcount[b],
                 in_free[b]);
    referenced += bm->refcount[b] > 0;
  }
  if (referenced + (int64_t)bm->free_q.size() != bm->num_blocks)
    return err(PA_ERR_INVALID_ARG, "referenced %lld + free %zu != capacity %d", (long long)referenced,
               bm->free_q.size(), bm->num_blocks);
  return PA_OK;
}

}  // extern "C"
