// Data-movement kernels beside the decode: token append, copy-on-write of a
// tail block's valid slots, and the debug gather; and the longest-first
// order of a batch's requests (paged_attn_order).  All three move whole
// slots, and a slot of one block (all KV heads, all dims) is one contiguous
// run of Hkv*d elements in the [NB, B, Hkv, d] pool, so each kernel is a
// 16-byte-vector copy of contiguous runs.  Bytes are copied exactly.
//
// [Slides] = "PagedAttention：让 KV cache 按需生长".
#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

__device__ inline void copy16(uint8_t* __restrict__ dst, const uint8_t* __restrict__ src, int64_t bytes) {
  for (int64_t i = (int64_t)threadIdx.x * 16; i < bytes; i += (int64_t)blockDim.x * 16)
    *reinterpret_cast<uint4*>(dst + i) = *reinterpret_cast<const uint4*>(src + i);
}

// Threads of one append workgroup: one 16-byte vector per thread per slot
// row (Hkv * d elements), in whole waves, at most kThreads: 128 for the
// 2 KiB bf16 rows of 8 KV heads, which one pass then covers.
int append_threads(int row_bytes) {
  const int vecs = (row_bytes + 15) / 16;
  const int waves = (vecs + 63) / 64;
  return waves >= kThreads / 64 ? kThreads : 64 * waves;
}

// One workgroup per (request, new token, layer), K and V both.  Token i of
// request s takes logical index p = positions[s] + i and goes to slot p % B
// of block table[p / B] of the layer's pools; nothing else moves ([Slides]
// "写满一块，再拿下一块").  A negative start skips the request; positions or
// blocks outside the pool are skipped.  New rows are [L, S, T, Hkv, d]
// (layer stride S*T rows), pools [L, NB, B, Hkv, d] (layer stride given).
__global__ __launch_bounds__(kThreads) void append_kernel(KvArgs a, const uint8_t* __restrict__ k_new,
                                                          const uint8_t* __restrict__ v_new,
                                                          const int32_t* __restrict__ tables,
                                                          const int32_t* __restrict__ positions, int T,
                                                          int64_t layer_stride_bytes) {
  const int s = blockIdx.x / T;
  const int i = blockIdx.x % T;
  const int start = positions[s];
  if (start < 0) return;
  const int64_t p = (int64_t)start + i;
  if (p >= (int64_t)a.MB * a.B) return;
  const int blk = tables[(int64_t)s * a.MB + p / a.B];
  if (blk < 0 || blk >= a.NB) return;
  const int layer = blockIdx.y;
  const int64_t src = ((int64_t)layer * gridDim.x + blockIdx.x) * a.row_bytes;
  const int64_t dst = layer * layer_stride_bytes + ((int64_t)blk * a.B + p % a.B) * a.row_bytes;
  copy16(a.k_pool + dst, k_new + src, a.row_bytes);
  copy16(a.v_pool + dst, v_new + src, a.row_bytes);
}

// One workgroup per (pair, layer, pool): slots [0, n) of block src -> block dst
// ([Slides] "先确保分配成功，再改变可见状态", copy_valid_kv).  The valid prefix
// of a block is one contiguous run of n*row_bytes.
__global__ __launch_bounds__(kThreads) void cow_kernel(KvArgs a, const int32_t* __restrict__ srcs,
                                                       const int32_t* __restrict__ dsts,
                                                       const int32_t* __restrict__ n_valid,
                                                       int64_t layer_stride_bytes) {
  const int i = blockIdx.x;
  const int src = srcs[i], dst = dsts[i], n = n_valid[i];
  if (src < 0 || src >= a.NB || dst < 0 || dst >= a.NB || n <= 0 || n > a.B || src == dst) return;
  uint8_t* pool = (blockIdx.z ? a.v_pool : a.k_pool) + (int64_t)blockIdx.y * layer_stride_bytes;
  const int64_t blk_bytes = (int64_t)a.B * a.row_bytes;
  copy16(pool + dst * blk_bytes, pool + src * blk_bytes, (int64_t)n * a.row_bytes);
}

// One workgroup per (request, logical block, pool): the valid slots of that
// block land at their logical positions in a [S, MB*B, Hkv, d] buffer.
__global__ __launch_bounds__(kThreads) void gather_kernel(KvArgs a, const int32_t* __restrict__ tables,
                                                          const int32_t* __restrict__ lens,
                                                          uint8_t* __restrict__ k_out,
                                                          uint8_t* __restrict__ v_out) {
  const int s = blockIdx.x, j = blockIdx.y;
  int n = lens[s];
  n = n < 0 ? 0 : (n > a.MB * a.B ? a.MB * a.B : n);
  if (j * a.B >= n) return;
  const int blk = tables[(int64_t)s * a.MB + j];
  if (blk < 0 || blk >= a.NB) return;
  const int cnt = min(a.B, n - j * a.B);
  const uint8_t* pool = blockIdx.z ? a.v_pool : a.k_pool;
  uint8_t* out = blockIdx.z ? v_out : k_out;
  const int64_t blk_bytes = (int64_t)a.B * a.row_bytes;
  copy16(out + ((int64_t)s * a.MB * a.B + (int64_t)j * a.B) * a.row_bytes, pool + blk * blk_bytes,
         (int64_t)cnt * a.row_bytes);
}

// One workgroup per (listed block i, layer, pool): the whole block (all
// slots, all KV heads) moves between the pool and slot i of a contiguous
// buffer laid out [layer][pool (K, V)][listed block][slot, head, dim] ([Slides]
// "腾出显存以后，还要付一次恢复成本": swapping a request's KV out and back in).
// The buffer may be host memory the device can address; then the copy crosses
// the host link directly.  Block ids outside the pool are skipped.
__global__ __launch_bounds__(kThreads) void swap_kernel(KvArgs a, const int32_t* __restrict__ blocks, int nlist,
                                                        uint8_t* buf, int64_t layer_stride_bytes, int to_buffer) {
  const int i = blockIdx.x;
  const int blk = blocks[i];
  if (blk < 0 || blk >= a.NB) return;
  const int64_t blk_bytes = (int64_t)a.B * a.row_bytes;
  uint8_t* pool = (blockIdx.z ? a.v_pool : a.k_pool) + (int64_t)blockIdx.y * layer_stride_bytes + blk * blk_bytes;
  uint8_t* slot = buf + (((int64_t)blockIdx.y * 2 + blockIdx.z) * nlist + i) * blk_bytes;
  if (to_buffer)
    copy16(slot, pool, blk_bytes);
  else
    copy16(pool, slot, blk_bytes);
}

// One thread per request: its rank among all requests by (length
// descending, index ascending), a strict total order, so the ranks are a
// permutation; the lengths pass through LDS 256 at a time, read four at a
// time (every lane the same address: a broadcast).
__global__ __launch_bounds__(kThreads) void order_kernel(const int32_t* __restrict__ lens, int S,
                                                         int32_t* __restrict__ order) {
  __shared__ __attribute__((aligned(16))) int32_t tile[kThreads];
  const int s = blockIdx.x * kThreads + threadIdx.x;
  const int32_t mine = s < S ? lens[s] : 0;
  int rank = 0;
  auto before = [&](int32_t o, int idx) { return (int)((o > mine) | ((o == mine) & (idx < s))); };
  for (int base = 0; base < S; base += kThreads) {
    __syncthreads();
    if (base + (int)threadIdx.x < S) tile[threadIdx.x] = lens[base + threadIdx.x];
    __syncthreads();
    const int cnt = min(kThreads, S - base);
    if (cnt == kThreads) {
#pragma unroll 8
      for (int i = 0; i < kThreads; i += 4) {
        const int4 o = *reinterpret_cast<const int4*>(&tile[i]);
        rank += before(o.x, base + i) + before(o.y, base + i + 1) + before(o.z, base + i + 2) +
                before(o.w, base + i + 3);
      }
    } else {
      for (int i = 0; i < cnt; ++i) rank += before(tile[i], base + i);
    }
  }
  if (s < S) order[rank] = s;
}

}  // namespace

hipError_t launch_order(const int32_t* lens, int S, int32_t* order, hipStream_t stream) {
  hipLaunchKernelGGL(order_kernel, dim3((S + kThreads - 1) / kThreads), dim3(kThreads), 0, stream, lens, S, order);
  return hipGetLastError();
}

hipError_t launch_swap(const KvArgs& a, const int32_t* blocks, int nlist, uint8_t* buf, int num_layers,
                       int64_t layer_stride_bytes, bool to_buffer, hipStream_t stream) {
  hipLaunchKernelGGL(swap_kernel, dim3(nlist, num_layers, 2), dim3(kThreads), 0, stream, a, blocks, nlist, buf,
                     layer_stride_bytes, to_buffer ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_append(const KvArgs& a, const uint8_t* k_new, const uint8_t* v_new, const int32_t* tables,
                         const int32_t* positions, int T, int num_layers, int64_t layer_stride_bytes,
                         hipStream_t stream) {
  hipLaunchKernelGGL(append_kernel, dim3(a.S * T, num_layers), dim3(append_threads(a.row_bytes)), 0, stream, a,
                     k_new, v_new, tables, positions, T, layer_stride_bytes);
  return hipGetLastError();
}

hipError_t launch_cow(const KvArgs& a, const int32_t* src, const int32_t* dst, const int32_t* n_valid,
                      int num_pairs, int num_layers, int64_t layer_stride_bytes, hipStream_t stream) {
  hipLaunchKernelGGL(cow_kernel, dim3(num_pairs, num_layers, 2), dim3(kThreads), 0, stream, a, src, dst,
                     n_valid, layer_stride_bytes);
  return hipGetLastError();
}

hipError_t launch_gather(const KvArgs& a, const int32_t* tables, const int32_t* lens, uint8_t* k_out,
                         uint8_t* v_out, hipStream_t stream) {
  hipLaunchKernelGGL(gather_kernel, dim3(a.S, a.MB, 2), dim3(kThreads), 0, stream, a, tables, lens, k_out,
                     v_out);
  return hipGetLastError();
}

}  // namespace pa
