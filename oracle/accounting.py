"""KV byte, block and slot accounting (exact integers / fractions).

Test infrastructure only (see the package docstring).

Sources:
  [Serving] "PagedAttention 与在线推理：KV 分页、共享及调度的联合分析":
      formula M_KV = 2 L n h_KV d_h b; formula A_B(n) = B*ceil(n/B),
      W_B(n) = A_B(n) - n; utilisation formula U; the five-sequence result.
  [Budgets] "内存预算约束下的语言模型服务：注意力、分页与调度":
      eq. (1) KV bytes summed over requests, eq. (2) tail waste and its bound
      N(B-1), eq. (3) mean tail waste (B-1)/2 for lengths uniform on [1, kB].
  [Slides] "PagedAttention：让 KV cache 按需生长": slides "128 KiB：…",
      "24 GiB 的 KV 池…", "把浪费限制在尾块里", the tail-waste and block-size
      tables, quiz "8 GiB 池能容纳多少条 1,025-token 请求？".
"""

from fractions import Fraction

KiB = 1 << 10
MiB = 1 << 20
GiB = 1 << 30


def kv_bytes(layers, tokens, kv_heads, head_dim, elem_bytes):
    """Uncompressed K+V bytes for ``tokens`` retained tokens.

    The leading 2 counts K and V ([Serving] formula M_KV; [Budgets] eq. (1)).
    Excludes tables, workspace, padding and weights, as both pages state.
    """
    return 2 * layers * tokens * kv_heads * head_dim * elem_bytes


def kv_bytes_per_token(layers, kv_heads, head_dim, elem_bytes):
    """Bytes one extra retained token costs ([Slides] "128 KiB：每新增一个位置的账单")."""
    return kv_bytes(layers, 1, kv_heads, head_dim, elem_bytes)


def blocks_for(n, B):
    """ceil(n / B): physical blocks a request of n tokens occupies ([Serving] §2)."""
    if n < 0 or B <= 0:
        raise ValueError("need n >= 0 and B > 0")
    return -(-n // B)


def allocated_slots(n, B):
    """A_B(n) = B * ceil(n / B) ([Serving] formula A_B; [Budgets] §5)."""
    return B * blocks_for(n, B)


def tail_waste(n, B):
    """W_B(n) = A_B(n) - n: empty slots of the last block ([Serving] formula W_B)."""
    return allocated_slots(n, B) - n


def total_tail_waste(lengths, B):
    """W_tail = sum_i (B*ceil(T_i/B) - T_i) ([Budgets] eq. (2))."""
    return sum(tail_waste(n, B) for n in lengths)


def tail_waste_bound(lengths, B):
    """N (B - 1) for the N non-empty requests ([Budgets] eq. (2))."""
    return sum(1 for n in lengths if n > 0) * (B - 1)


def utilisation(lengths, B):
    """U = sum n_i / sum B*ceil(n_i/B), exactly ([Serving] formula U).

    A slot utilisation, not a device utilisation (the page says so).
    """
    useful = sum(lengths)
    alloc = sum(allocated_slots(n, B) for n in lengths)
    return Fraction(useful, alloc)


def fixed_reservation_slots(lengths, M):
    """Slots a per-request fixed reservation of M slots takes ([Serving] §2)."""
    return M * len(lengths)


def mean_tail_waste_uniform(B, k):
    """Mean of W_B(n) over integer n uniform on [1, k*B], by enumeration.

    [Budgets] eq. (3) states the closed form (B-1)/2; this routine sums every
    case instead, so the closed form is checked rather than assumed.
    """
    top = k * B
    return Fraction(sum(tail_waste(n, B) for n in range(1, top + 1)), top)


def mean_fixed_reservation_waste(M):
    """Mean of M - n for n uniform on [1, M] ([Budgets] §5: 255.5 at M = 512)."""
    return Fraction(sum(M - n for n in range(1, M + 1)), M)


def pool_blocks(pool_bytes, B, bytes_per_token):
    """Whole blocks of B tokens that fit in ``pool_bytes`` ([Slides] quiz 1 step 2)."""
    return pool_bytes // (B * bytes_per_token)


def pool_leftover_bytes(pool_bytes, B, bytes_per_token):
    """Bytes of the pool too small to hold one more block ([Slides] quiz 1 step 4)."""
    return pool_bytes - pool_blocks(pool_bytes, B, bytes_per_token) * B * bytes_per_token


def requests_that_fit(free_blocks, blocks_per_request):
    """(requests admitted, blocks left) for equal, unshared requests ([Slides] quiz 1; 24 GiB slide)."""
    return free_blocks // blocks_per_request, free_blocks % blocks_per_request
