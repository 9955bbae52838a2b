// C-ABI entry points of libpagedattn: host-side validation, split planning
// and launches.  Every check on host-resident arguments happens before any
// work is enqueued; nothing here allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "pa_internal.h"

namespace {

thread_local std::string g_last_error;

pa_status fail(pa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

}  // namespace

namespace pa {

void set_last_error(const char* msg) { g_last_error = msg ? msg : ""; }

}  // namespace pa

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_size(pa_dtype t) { return t == PA_BF16 ? 2 : 4; }

// Shape checks shared by every entry point.
pa_status check_dims(const pa_dims* d, int32_t B, bool need_attention_shape) {
  if (!d) return fail(PA_ERR_INVALID_ARG, "dims is NULL");
  if (d->num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs = %d < 0", d->num_seqs);
  if (d->num_kv_heads < 1) return fail(PA_ERR_INVALID_ARG, "num_kv_heads = %d < 1", d->num_kv_heads);
  if (d->head_dim < 1) return fail(PA_ERR_INVALID_ARG, "head_dim = %d < 1", d->head_dim);
  if (d->max_blocks_per_seq < 1) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq = %d < 1", d->max_blocks_per_seq);
  if (d->num_blocks < 1) return fail(PA_ERR_INVALID_ARG, "num_blocks = %d < 1", d->num_blocks);
  if (B < 1) return fail(PA_ERR_INVALID_ARG, "block size B = %d < 1", B);
  if (d->dtype != PA_F32 && d->dtype != PA_BF16) return fail(PA_ERR_UNSUPPORTED, "dtype %d", (int)d->dtype);
  if (d->flags & ~PA_FLAG_BF16_WEIGHTS) return fail(PA_ERR_INVALID_ARG, "unknown flags 0x%x", (unsigned)d->flags);
  if ((int64_t)d->max_blocks_per_seq * B > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq * B overflows int32");
  if (need_attention_shape) {
    if (d->num_q_heads < 1) return fail(PA_ERR_INVALID_ARG, "num_q_heads = %d < 1", d->num_q_heads);
    if (d->num_q_heads % d->num_kv_heads)
      return fail(PA_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d", d->num_q_heads,
                  d->num_kv_heads);
    const int G = d->num_q_heads / d->num_kv_heads;
    const bool g_ok = G == 1 || G == 2 || G == 4 || G == 8 || (G == 16 && d->dtype == PA_BF16);
    if (!g_ok)
      return fail(PA_ERR_UNSUPPORTED, "query heads per KV head = %d (supported: 1, 2, 4, 8; 16 for bf16)", G);
    if (d->head_dim != pa::kHeadDim) return fail(PA_ERR_UNSUPPORTED, "head_dim %d (supported: 128)", d->head_dim);
    if (B != 4 && B != 8 && B != 16 && B != 32 && B != 64)
      return fail(PA_ERR_UNSUPPORTED, "block size %d (supported: 4, 8, 16, 32, 64)", B);
    if (d->num_splits < 0) return fail(PA_ERR_INVALID_ARG, "num_splits = %d < 0", d->num_splits);
  }
  // slot rows are copied as 16-byte vectors
  if (((int64_t)d->num_kv_heads * d->head_dim * elem_size(d->dtype)) % 16)
    return fail(PA_ERR_UNSUPPORTED, "Hkv * d * element size must be a multiple of 16 bytes");
  return PA_OK;
}

// Splits depend only on host-known sizes (S, Hq, Hkv, MB, B, dtype and the
// query-token count T), so repeated calls agree.  A split boundary is both a 16-slot tile boundary and a block
// boundary: split p covers tokens [p*tps, (p+1)*tps) with tps a multiple of
// max(16, B).  Returns (P, tps).
//   bf16 (matrix-core kernel, kMfmaWaves waves per work item): about one
//     wave per SIMD (1024 on MI355X), each wave keeping at least 4 tiles.
//     Measured on 32 x 4096 tokens: every extra split costs more in partial
//     states and their merge than the added parallelism returns;
//   fp32 (vector-ALU kernel, one wave per work item): about 2048 waves, each
//     split keeping at least 2 tiles.  A wave walks its blocks one dependent
//     read after another, so few requests want many short splits: 5 requests
//     of at most 511 tokens took 24.8 us with 4 splits, 16.8 us with 8 and
//     14.1 us with 16 (merge included).
// Several query tokens multiply the work items by the token groups (TG), so
// fewer splits reach the same wave count.  The shared-tile kernel (bf16, more
// tokens than two 16-column sets hold) streams each tile once per workgroup of
// 4 waves (8 in the ping-pong form), all of which walk every tile of the
// split: about 2048 waves, each split keeping at least 16 tiles (more splits
// measured slower for 32 x 4096 tokens).
int64_t token_groups(const pa_dims* d, int32_t T) {
  const int per = pa::tokens_per_item(d->dtype, d->num_q_heads / d->num_kv_heads, T);
  return ((int64_t)T + per - 1) / per;
}

void plan_splits(const pa_dims* d, int32_t B, int32_t T, int* P_out, int* tps_out) {
  const int64_t max_tokens = (int64_t)d->max_blocks_per_seq * B;
  const int64_t unit = B > 16 ? B : 16;
  const int64_t units = (max_tokens + unit - 1) / unit;
  int64_t P = d->num_splits;
  if (P == 0) {
    const int64_t items = (int64_t)d->num_seqs * d->num_kv_heads * token_groups(d, T);
    const bool mfma = d->dtype == PA_BF16;
    const bool shared = pa::use_shared_tile(d->dtype, d->num_q_heads / d->num_kv_heads, T);
    const int64_t waves_per_item =
        shared ? pa::shared_tile_waves(d->dtype, d->num_q_heads / d->num_kv_heads, T) : (mfma ? pa::kMfmaWaves : 1);
    const int64_t target = (mfma && !shared) ? 1024 : 2048;
    const int64_t per = items * waves_per_item;
    P = (target + per - 1) / (per > 0 ? per : 1);
    // Shortest split worth a work item: 256 tokens for the shared-tile kernel,
    // 64 per wave for the matrix-core decode, one 16-slot tile for the float32
    // kernel (5 requests of 37-511 tokens: 32 splits 10.3 us, 16 splits 12.1 us).
    // No automatic split is shorter: 3 x 300 bf16 tokens run as one split in
    // 6.8 us, as two of 160 tokens plus the merge in 7.7 us.
    const int64_t min_tokens = shared ? 256 : (mfma ? 64 * pa::kMfmaWaves : 16);
    const int64_t maxP = max_tokens / min_tokens > 1 ? max_tokens / min_tokens : 1;
    P = P < 1 ? 1 : (P > maxP ? maxP : P);
    // Two splits become four, which run as the four parts of one workgroup
    // on the 32-column kernel, for 49-64 columns per KV head with the default
    // weights (two waves per part, the second more than half full) and for
    // 65-96 columns (three waves per part).  32 x 4096 tokens: at 64 columns
    // 94-97 against 101-106 us for two halves of 16-column waves (G = 1, 2,
    // 4, 8, 16), but at 40-48 columns the halves were 1-3 % faster, and with
    // PA_FLAG_BF16_WEIGHTS 2-4 % faster; at 72-96 columns (T = 18-24, G = 4)
    // 111.7-115.2 against 117.6-123.9 us for two halves of four 32-column
    // waves, with bf16 weights 98.6-101.4 against 100.7-106.9 us.
    const int G = d->num_q_heads / d->num_kv_heads;
    const int sets = pa::shared_tile_sets(d->dtype, G, T);
    if (P == 2 && maxP >= 4 && shared &&
        ((sets == 1 && (int64_t)T * G > 48 && !(d->flags & PA_FLAG_BF16_WEIGHTS)) ||
         (sets == 2 && (int64_t)T * G <= 96)))
      P = 4;
  }
  if (P > units) P = units;
  const int64_t upp = (units + P - 1) / P;  // units per split
  *P_out = (int)((units + upp - 1) / upp);  // drop splits that could never hold a token
  *tps_out = (int)(upp * unit);
}

pa_status launched(hipError_t e) {
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "HIP launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

}  // namespace

extern "C" {

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

const char* pa_status_string(pa_status st) {
  switch (st) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
    case PA_ERR_LAUNCH: return "PA_ERR_LAUNCH";
  }
  if ((int)st == -5) return "PA_ERR_NO_SPACE";  // block manager (pa_blockmgr.h)
  return "PA_UNKNOWN_STATUS";
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

static pa_status plan_common(const pa_dims* dims, int32_t B, int32_t T, int32_t* num_splits,
                             size_t* workspace_bytes) {
  pa_status st = check_dims(dims, B, true);
  if (st != PA_OK) return st;
  if (T < 1) return fail(PA_ERR_INVALID_ARG, "num_q_tokens = %d < 1", T);
  if (!num_splits || !workspace_bytes) return fail(PA_ERR_INVALID_ARG, "output pointer is NULL");
  int P, tps;
  plan_splits(dims, B, T, &P, &tps);
  *num_splits = P;
  const int Pm = pa::shared_tile_parts(dims->dtype, dims->num_q_heads / dims->num_kv_heads, T, P) > 1
                     ? 1
                     : pa::merged_splits(dims->dtype, P);
  *workspace_bytes =
      (Pm > 1 && dims->num_seqs > 0)
          ? pa::decode_workspace_floats((int64_t)dims->num_seqs * T * dims->num_q_heads, Pm) * sizeof(float)
          : 0;
  return PA_OK;
}

// Validation, split plan and launch shared by the one-token decode (T = 1)
// and the several-token causal form.
static pa_status kv_common(const pa_dims* dims, int32_t B, void* k_pool, void* v_pool, pa::KvArgs* a);

// k_new / v_new / positions non-NULL: append the step's token first (fused
// into the bf16 decode kernel; fp32 runs the append kernel, then the decode).
static pa_status attend(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_tables,
                        const int32_t* seq_lens, int32_t T, int32_t B, float scale, float* out, hipStream_t stream,
                        const pa_dims* dims, const void* k_new = nullptr, const void* v_new = nullptr,
                        const int32_t* positions = nullptr) {
  pa_status st = check_dims(dims, B, true);
  if (st != PA_OK) return st;
  if (T < 1) return fail(PA_ERR_INVALID_ARG, "num_q_tokens = %d < 1", T);
  if (dims->num_seqs == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !seq_lens || !out)
    return fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 16))
    return fail(PA_ERR_INVALID_ARG, "q, pools and out must be 16-byte aligned");
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale is not finite");
  int P, tps;
  plan_splits(dims, B, T, &P, &tps);
  const int64_t TG = token_groups(dims, T);
  const int64_t items = (int64_t)dims->num_kv_heads * dims->num_seqs * P * TG;
  const int64_t rows = (int64_t)dims->num_seqs * T * dims->num_q_heads;
  if (items > INT32_MAX || rows > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "grid too large");
  if (dims->num_seqs > (1 << 28)) return fail(PA_ERR_UNSUPPORTED, "more than 2^28 requests");  // 32-bit byte offsets

  pa::DecodeArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.tables = block_tables;
  a.lens = seq_lens;
  a.out = out;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.S = dims->num_seqs;
  a.Hq = dims->num_q_heads;
  a.Hkv = dims->num_kv_heads;
  a.MB = dims->max_blocks_per_seq;
  a.NB = dims->num_blocks;
  // float32 runs its splits as the waves of workgroups (valu_waves) and
  // keeps P for the groups that reach the merge.
  a.W = dims->dtype == PA_F32 ? pa::valu_waves(P) : 1;
  a.P = pa::merged_splits(dims->dtype, P);
  a.tps = tps;
  a.T = T;
  a.TG = (int)TG;
  a.bf16_weights = (dims->flags & PA_FLAG_BF16_WEIGHTS) != 0;
  a.order = dims->order;
  if (k_new) {
    if (!aligned(k_new, 16) || !aligned(v_new, 16)) return fail(PA_ERR_INVALID_ARG, "k_new/v_new must be 16-byte aligned");
    if (dims->dtype == PA_BF16) {
      a.k_new = k_new;
      a.v_new = v_new;
      a.positions = positions;
    }
  }
  if (a.P > 1 && pa::shared_tile_parts(dims->dtype, a.Hq / a.Hkv, T, a.P) == 1) {
    const size_t need = pa::decode_workspace_floats(rows, a.P) * sizeof(float);
    if (!dims->workspace || dims->workspace_bytes < need)
      return fail(PA_ERR_WORKSPACE, "split-K needs %zu workspace bytes, got %zu", need,
                  dims->workspace ? dims->workspace_bytes : (size_t)0);
    if (!aligned(dims->workspace, 256)) return fail(PA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    float* ws = static_cast<float*>(dims->workspace);
    const size_t no = (size_t)rows * a.P * pa::kHeadDim;
    a.ws_o = ws;
    a.ws_m = ws + no;
    a.ws_l = ws + no + (size_t)rows * a.P;
  }
  if (k_new && dims->dtype != PA_BF16) {
    pa::KvArgs ka{};
    st = kv_common(dims, B, const_cast<void*>(k_pool), const_cast<void*>(v_pool), &ka);
    if (st != PA_OK) return st;
    st = launched(pa::launch_append(ka, static_cast<const uint8_t*>(k_new), static_cast<const uint8_t*>(v_new),
                                    block_tables, positions, 1, 1, 0, stream));
    if (st != PA_OK) return st;
  }
  return launched(pa::launch_decode(a, dims->dtype, B, a.Hq / a.Hkv, stream));
}

pa_status paged_attn_plan(const pa_dims* dims, int32_t B, int32_t* num_splits, size_t* workspace_bytes) {
  g_last_error.clear();
  return plan_common(dims, B, 1, num_splits, workspace_bytes);
}

size_t paged_attn_workspace_bytes(const pa_dims* dims, int32_t B) {
  g_last_error.clear();
  int32_t P = 0;
  size_t bytes = 0;
  if (plan_common(dims, B, 1, &P, &bytes) != PA_OK) return SIZE_MAX;
  return bytes;
}

pa_status paged_attn_order(const int32_t* seq_lens, int32_t S, int32_t* order, hipStream_t stream) {
  g_last_error.clear();
  if (S < 0) return fail(PA_ERR_INVALID_ARG, "S = %d < 0", S);
  if (S == 0) return PA_OK;
  if (!seq_lens || !order) return fail(PA_ERR_INVALID_ARG, "seq_lens and order are required");
  if (S > (1 << 16)) return fail(PA_ERR_UNSUPPORTED, "more than 65536 requests to order");
  return launched(pa::launch_order(seq_lens, S, order, stream));
}

pa_status paged_attn_extend_plan(const pa_dims* dims, int32_t B, int32_t num_q_tokens, int32_t* num_splits,
                                 size_t* workspace_bytes) {
  g_last_error.clear();
  return plan_common(dims, B, num_q_tokens, num_splits, workspace_bytes);
}

pa_status paged_attn_decode(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_tables,
                            const int32_t* seq_lens, int32_t B, float scale, float* out, hipStream_t stream,
                            const pa_dims* dims) {
  g_last_error.clear();
  return attend(q, k_pool, v_pool, block_tables, seq_lens, 1, B, scale, out, stream, dims);
}

pa_status paged_attn_decode_append(const void* q, const void* k_pool, const void* v_pool, const void* k_new,
                                   const void* v_new, const int32_t* block_tables, const int32_t* positions,
                                   const int32_t* seq_lens, int32_t B, float scale, float* out, hipStream_t stream,
                                   const pa_dims* dims) {
  g_last_error.clear();
  if (dims && dims->num_seqs > 0 && (!k_new || !v_new || !positions))
    return fail(PA_ERR_INVALID_ARG, "k_new, v_new and positions are required");
  return attend(q, k_pool, v_pool, block_tables, seq_lens, 1, B, scale, out, stream, dims, k_new, v_new, positions);
}

pa_status paged_attn_extend(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_tables,
                            const int32_t* seq_lens, int32_t num_q_tokens, int32_t B, float scale, float* out,
                            hipStream_t stream, const pa_dims* dims) {
  g_last_error.clear();
  return attend(q, k_pool, v_pool, block_tables, seq_lens, num_q_tokens, B, scale, out, stream, dims);
}

static pa_status kv_common(const pa_dims* dims, int32_t B, void* k_pool, void* v_pool, pa::KvArgs* a) {
  pa_status st = check_dims(dims, B, false);
  if (st != PA_OK) return st;
  if (!k_pool || !v_pool) return fail(PA_ERR_INVALID_ARG, "pool pointer is NULL");
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16)) return fail(PA_ERR_INVALID_ARG, "pools must be 16-byte aligned");
  const int64_t row = (int64_t)dims->num_kv_heads * dims->head_dim * elem_size(dims->dtype);
  if (row > INT32_MAX / 2) return fail(PA_ERR_UNSUPPORTED, "slot row too large");
  a->k_pool = static_cast<uint8_t*>(k_pool);
  a->v_pool = static_cast<uint8_t*>(v_pool);
  a->S = dims->num_seqs;
  a->MB = dims->max_blocks_per_seq;
  a->NB = dims->num_blocks;
  a->B = B;
  a->row_bytes = (int)row;
  return PA_OK;
}

static pa_status append_common(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                               const int32_t* block_tables, const int32_t* positions, int32_t T, int32_t B,
                               hipStream_t stream, const pa_dims* dims, int32_t num_layers = 1,
                               int64_t layer_stride_elems = 0) {
  if (T < 1) return fail(PA_ERR_INVALID_ARG, "num_tokens = %d < 1", T);
  if (num_layers < 1 || num_layers > 65535)
    return fail(PA_ERR_INVALID_ARG, "num_layers = %d outside [1, 65535]", num_layers);
  pa::KvArgs a{};
  if (dims && dims->num_seqs == 0) return check_dims(dims, B, false);
  pa_status st = kv_common(dims, B, k_pool, v_pool, &a);
  if (st != PA_OK) return st;
  if (!k_new || !v_new || !block_tables || !positions) return fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(k_new, 16) || !aligned(v_new, 16)) return fail(PA_ERR_INVALID_ARG, "k_new/v_new must be 16-byte aligned");
  if ((int64_t)a.S * T > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "too many tokens");
  const int64_t pool_elems = (int64_t)dims->num_blocks * B * dims->num_kv_heads * dims->head_dim;
  if (num_layers > 1 && layer_stride_elems < pool_elems)
    return fail(PA_ERR_INVALID_ARG, "layer_stride_elems %lld smaller than one layer's pool (%lld)",
                (long long)layer_stride_elems, (long long)pool_elems);
  const int64_t stride_bytes = num_layers > 1 ? layer_stride_elems * (int64_t)elem_size(dims->dtype) : 0;
  if (stride_bytes % 16) return fail(PA_ERR_INVALID_ARG, "layer stride must be a multiple of 16 bytes");
  return launched(pa::launch_append(a, static_cast<const uint8_t*>(k_new), static_cast<const uint8_t*>(v_new),
                                    block_tables, positions, T, num_layers, stride_bytes, stream));
}

pa_status kv_append(void* k_pool, void* v_pool, const void* k_new, const void* v_new, const int32_t* block_tables,
                    const int32_t* positions, int32_t B, hipStream_t stream, const pa_dims* dims) {
  g_last_error.clear();
  return append_common(k_pool, v_pool, k_new, v_new, block_tables, positions, 1, B, stream, dims);
}

pa_status kv_append_layers(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                           const int32_t* block_tables, const int32_t* positions, int32_t B, int32_t num_layers,
                           int64_t layer_stride_elems, hipStream_t stream, const pa_dims* dims) {
  g_last_error.clear();
  return append_common(k_pool, v_pool, k_new, v_new, block_tables, positions, 1, B, stream, dims, num_layers,
                       layer_stride_elems);
}

pa_status kv_append_tokens(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                           const int32_t* block_tables, const int32_t* positions, int32_t num_tokens, int32_t B,
                           hipStream_t stream, const pa_dims* dims) {
  g_last_error.clear();
  return append_common(k_pool, v_pool, k_new, v_new, block_tables, positions, num_tokens, B, stream, dims);
}

pa_status kv_cow_copy(void* k_pool, void* v_pool, const int32_t* src_blocks, const int32_t* dst_blocks,
                      const int32_t* n_valid, int32_t num_pairs, int32_t B, int32_t num_layers,
                      int64_t layer_stride_elems, hipStream_t stream, const pa_dims* dims) {
  g_last_error.clear();
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARG, "num_pairs = %d < 0", num_pairs);
  if (num_layers < 1 || num_layers > 65535) return fail(PA_ERR_INVALID_ARG, "num_layers = %d outside [1, 65535]", num_layers);
  pa::KvArgs a{};
  pa_status st = kv_common(dims, B, k_pool, v_pool, &a);
  if (st != PA_OK) return st;
  if (num_pairs == 0) return PA_OK;
  if (!src_blocks || !dst_blocks || !n_valid) return fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
  const int64_t pool_elems = (int64_t)dims->num_blocks * B * dims->num_kv_heads * dims->head_dim;
  if (num_layers > 1 && layer_stride_elems < pool_elems)
    return fail(PA_ERR_INVALID_ARG, "layer_stride_elems %lld smaller than one layer's pool (%lld)",
                (long long)layer_stride_elems, (long long)pool_elems);
  const int64_t stride_bytes = num_layers > 1 ? layer_stride_elems * (int64_t)elem_size(dims->dtype) : 0;
  if (stride_bytes % 16) return fail(PA_ERR_INVALID_ARG, "layer stride must be a multiple of 16 bytes");
  return launched(pa::launch_cow(a, src_blocks, dst_blocks, n_valid, num_pairs, num_layers, stride_bytes, stream));
}

static pa_status kv_swap(void* k_pool, void* v_pool, const int32_t* blocks, int32_t num_list, void* buf,
                         int32_t B, int32_t num_layers, int64_t layer_stride_elems, bool to_buffer, hipStream_t stream,
                         const pa_dims* dims) {
  if (num_list < 0) return fail(PA_ERR_INVALID_ARG, "num_blocks listed = %d < 0", num_list);
  if (num_list > 2147483647 / 2) return fail(PA_ERR_UNSUPPORTED, "too many blocks listed");
  if (num_layers < 1 || num_layers > 65535) return fail(PA_ERR_INVALID_ARG, "num_layers = %d outside [1, 65535]", num_layers);
  pa::KvArgs a{};
  pa_status st = kv_common(dims, B, k_pool, v_pool, &a);
  if (st != PA_OK) return st;
  if (num_list == 0) return PA_OK;
  if (!blocks || !buf) return fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(buf, 16)) return fail(PA_ERR_INVALID_ARG, "the swap buffer must be 16-byte aligned");
  const int64_t pool_elems = (int64_t)dims->num_blocks * B * dims->num_kv_heads * dims->head_dim;
  if (num_layers > 1 && layer_stride_elems < pool_elems)
    return fail(PA_ERR_INVALID_ARG, "layer_stride_elems %lld smaller than one layer's pool (%lld)",
                (long long)layer_stride_elems, (long long)pool_elems);
  const int64_t stride_bytes = num_layers > 1 ? layer_stride_elems * (int64_t)elem_size(dims->dtype) : 0;
  if (stride_bytes % 16) return fail(PA_ERR_INVALID_ARG, "layer stride must be a multiple of 16 bytes");
  return launched(pa::launch_swap(a, blocks, num_list, static_cast<uint8_t*>(buf), num_layers, stride_bytes,
                                  to_buffer, stream));
}

pa_status kv_swap_out(const void* k_pool, const void* v_pool, const int32_t* blocks, int32_t num_list, void* buf,
                      int32_t B, int32_t num_layers, int64_t layer_stride_elems, hipStream_t stream,
                      const pa_dims* dims) {
  g_last_error.clear();
  return kv_swap(const_cast<void*>(k_pool), const_cast<void*>(v_pool), blocks, num_list, buf, B, num_layers,
                 layer_stride_elems, true, stream, dims);
}

pa_status kv_swap_in(void* k_pool, void* v_pool, const int32_t* blocks, int32_t num_list, const void* buf, int32_t B,
                     int32_t num_layers, int64_t layer_stride_elems, hipStream_t stream, const pa_dims* dims) {
  g_last_error.clear();
  return kv_swap(k_pool, v_pool, blocks, num_list, const_cast<void*>(buf), B, num_layers, layer_stride_elems, false,
                 stream, dims);
}

pa_status paged_kv_gather(const void* k_pool, const void* v_pool, const int32_t* block_tables, const int32_t* seq_lens,
                          int32_t B, void* k_out, void* v_out, hipStream_t stream, const pa_dims* dims) {
  g_last_error.clear();
  pa::KvArgs a{};
  pa_status st = kv_common(dims, B, const_cast<void*>(k_pool), const_cast<void*>(v_pool), &a);
  if (st != PA_OK) return st;
  if (dims->num_seqs == 0) return PA_OK;
  if (!block_tables || !seq_lens || !k_out || !v_out) return fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(k_out, 16) || !aligned(v_out, 16)) return fail(PA_ERR_INVALID_ARG, "outputs must be 16-byte aligned");
  if (dims->max_blocks_per_seq > 65535) return fail(PA_ERR_UNSUPPORTED, "max_blocks_per_seq > 65535");
  return launched(pa::launch_gather(a, block_tables, seq_lens, static_cast<uint8_t*>(k_out),
                                    static_cast<uint8_t*>(v_out), stream));
}

}  // extern "C"
