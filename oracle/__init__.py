"""Float64 CPU oracle for the paged-attention decode path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code,
headers, tables or helpers with the HIP library in ``paged_kv_cache_352_amd``,
and it imports nothing from there.

It is deliberately plain and slow: explicit per-token index lists, one
library matrix-vector product per head, float64 throughout.

Pages cited (by title, then section / slide / equation on that page):

  [Serving]  "PagedAttention 与在线推理：KV 分页、共享及调度的联合分析"
             (auturnal.com guide, paged-attention-serving v6)
  [Slides]   "PagedAttention：让 KV cache 按需生长"
             (hs-black.github.io/posts/paged-attention/)
  [Budgets]  "内存预算约束下的语言模型服务：注意力、分页与调度"
             (auturnal.com guide, llm-serving-budgets v5)

Modules
-------
accounting  byte / block / slot accounting ([Serving] M_KV, A_B, W_B, U;
            [Budgets] eq. (1)-(3)).  Pinned to every figure the pages print.
attention   gather through the block table + dense softmax attention: the
            definition the paged kernel must reproduce, for one new token
            per request and for T new tokens attending causally (the
            verification / prompt-chunk form).  Pinned by brute force, by a
            library routine (with an explicit mask or its causal flag), by
            closed forms and invariants.
kvcache     token append (one or T tokens per request) and copy-on-write of
            a block's valid slots.  Pinned by invariants and by hand-checked
            tiny cases.
online      the (m, l, o) recurrence of [Budgets] eq. (4) and the merge of
            partial states.  Not the oracle: it checks the merge algebra the
            kernel relies on, and is pinned against ``attention``.
blockmgr    the per-request / per-block bookkeeping and the copy-on-write
            growth protocol of [Slides], as a plain Python model of the
            library's block manager, with multi-token growth and rollback.
            Pinned by the pages' worked examples
            (free counts of the shared-tail quiz, the lab's block counts, the
            24 GiB and 8 GiB pool figures, the 3-blocks / 4-requests case).

Every function here is pinned by something other than itself (see the
tests named in each module).  The sampled-row checkers
``attention.paged_decode_rows`` and ``attention.paged_extend_rows`` are pinned
by the plain-Python brute force on tiny poisoned cases, row by row, and by
bitwise equality with the full ``paged_decode`` / ``paged_extend``;
``accounting.tail_waste_bound`` by exhaustive enumeration (the bound holds for
every length list and equals the largest total tail waste among lists with
the same number of non-empty requests).  Planted indexing mistakes in each
are caught.  No function here is "parity unpinned".
"""

from . import accounting, attention, blockmgr, kvcache, online  # noqa: F401
