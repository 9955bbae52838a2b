// Internal launch interface shared by the host entry points (pa_api.hip) and
// the kernel translation units.  Not installed; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pagedattn.h"

namespace pa {

constexpr int kHeadDim = 128;  // d supported by the decode kernels
constexpr int kNumXcd = 8;     // MI355X: 8 accelerator dies, each with its own L2
constexpr int kMfmaWaves = 4;  // waves per workgroup of the bf16 matrix-core decode

struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* tables;
  const int32_t* lens;
  float* out;       // final output [S, T, Hq, d]
  float* ws_o;      // split partial o [S, T, Hq, P, d]   (P > 1 only)
  float* ws_m;      // split partial m [S, T, Hq, P]      (log2 domain)
  float* ws_l;      // split partial l [S, T, Hq, P]
  float scale_log2; // scale * log2(e): scores are kept in base 2
  int S, Hq, Hkv, MB, NB;
  int P;            // number of splits
  int tps;          // tokens per split: split p covers tokens [p*tps, (p+1)*tps), a multiple of max(16, B)
  const void* k_new;          // fused append (bf16 decode only): new K/V [S, Hkv, d] written at
  const void* v_new;          //   positions[s] and used for that position in this step; NULL
  const int32_t* positions;   //   otherwise
  int T;            // query tokens per request (q is [S, T, Hq, d]); the last T of the history, causal
  int TG;           // work items per (request, KV head, split) along the query tokens: ceil(T / tokens per item)
  bool bf16_weights;  // PA_FLAG_BF16_WEIGHTS: the shared-tile kernel rounds p once to bf16
  bool plain_order;   // bf16 decode: work items in launch order, not grouped by XCD (set at launch)
  int W;              // float32: splits per workgroup, one wave each, merged in LDS (P counts the groups)
  const int32_t* order;  // bf16 decode with plain_order: request issued r-th is order[r] (NULL: r)
};

// float32 decode: the P splits of one (request, KV head, token group) run in
// groups of up to kMaxValuWaves (the smallest power of two >= P), one wave
// each, as the waves of one workgroup, and each group merges its states in
// LDS; with more than one group the groups' partial states go to the merge
// kernel.  Measured on 5 requests of 37-511 tokens (16 splits): 13.6 us with
// one wave per workgroup, 12.1 us with groups of 4, 22 us with one group of
// 16 (a CU's four SIMDs then run a whole request's vector-ALU work).
constexpr int kMaxValuWaves = 4;

constexpr int valu_waves(int P) {
  int w = 1;
  while (w < P && w < kMaxValuWaves) w *= 2;
  return w;
}

// Partial states per output row that reach the split workspace and the
// merge kernel: P for bf16, the groups of valu_waves(P) splits for float32.
constexpr int merged_splits(pa_dtype dtype, int P) {
  return dtype == PA_F32 ? (P + valu_waves(P) - 1) / valu_waves(P) : P;
}

constexpr int kSharedTileWaves = 4;  // waves of the shared-tile several-token kernel

// Query tokens whose (token, head) pairs fill one wave's columns for group
// size G: the 16 MFMA columns (bf16) or 8 accumulator sets of the
// vector-ALU kernel (fp32).
constexpr int tokens_per_wave(pa_dtype dtype, int G) {
  return dtype == PA_BF16 ? (G >= 16 ? 1 : 16 / G) : (G >= 8 ? 1 : 8 / G);
}

// bf16 with more query tokens than two waves' columns hold: the shared-tile
// kernel (pa_extend_mfma.hip), whose waves take different tokens and share
// each K/V tile through LDS.  Up to two column sets, separate work items of
// the decode kernel (each streaming the history, the second mostly from L2)
// measured faster: 124.6 vs 132 us for 8 tokens of 4-head groups over
// 32 x 4096 tokens.
constexpr bool use_shared_tile(pa_dtype dtype, int G, int T) {
  return dtype == PA_BF16 && T > 2 * tokens_per_wave(dtype, G);
}

// 16-column sets per wave of the shared-tile kernel: two (each K and V
// operand read from LDS feeds both) once one set per wave would take more
// than one workgroup per (request, KV head) and so more than one pass over
// the history, else one.  Measured on 32 x 4096 tokens of 4-head groups:
// 639 vs 675 us for a 512-token chunk; 148-155 vs 169-171 us for 17-28
// tokens (some waves idle, one pass instead of two); but 184 vs 143 us for
// 16 tokens, which one set per wave covers in one pass.  Two sets per wave
// run as one 32-column set of the 32x32 kernel (launch_extend_wide).
constexpr int shared_tile_sets(pa_dtype dtype, int G, int T) {
  return T > kSharedTileWaves * tokens_per_wave(dtype, G) ? 2 : 1;
}

// 16-column sets per wave of the bf16 decode kernel: two when the query
// tokens need both (one work item then reads the history once for all of
// them), else one.
constexpr int decode_column_sets(pa_dtype dtype, int G, int T) {
  return dtype == PA_BF16 && T > tokens_per_wave(dtype, G) && !use_shared_tile(dtype, G, T) ? 2 : 1;
}

constexpr int kPingPongWaves = 8;  // waves of the ping-pong shared-tile kernel

// bf16 query groups wider than one workgroup of four 32-column waves (more
// than 128 (token, head) columns per KV head): the ping-pong kernel
// (launch_extend_wide), whose 8 waves run two per SIMD in opposite phases,
// one issuing its matrix products while the other runs its softmax.
// Measured on the 512-token chunk of 4-head groups over 8 x 4096 tokens:
// 375-382 vs 406-443 us (default weights), 298-300 vs 329-337 us (bf16
// weights), outputs bitwise equal.  At 24 or 32 tokens of 4-head groups half
// or more of its columns would be empty: 207-223 vs 136-147 us, so those stay
// on the 4-wave kernel.
constexpr bool use_pingpong(pa_dtype dtype, int G, int T) {
  return use_shared_tile(dtype, G, T) && shared_tile_sets(dtype, G, T) == 2 && (int64_t)T * G > kSharedTileWaves * 32;
}

// A two-split plan of the 4-wave shared-tile kernels (one set per wave or
// the 32-column form; one workgroup then holds all T tokens of its (request,
// KV head)) runs as one workgroup of two 4-wave halves, one per split, that
// merge their states in LDS at the end: no partial state reaches the split
// workspace and no merge kernel runs.
constexpr bool shared_tile_halves(pa_dtype dtype, int G, int T, int P) {
  return use_shared_tile(dtype, G, T) && !use_pingpong(dtype, G, T) && P == 2;
}

// A four-split plan of up to 96 (token, head) columns per KV head runs on
// the 32-column kernel as one workgroup of four parts, one part per split,
// that merge their states in LDS at the end (no split workspace, no merge
// kernel): two 32-column waves per part for the one-set-per-wave case
// (33-64 columns, e.g. 9-16 tokens of a 4-head group), three for 65-96
// columns (17-24 tokens of a 4-head group).
constexpr bool shared_tile_quarters(pa_dtype dtype, int G, int T, int P) {
  return use_shared_tile(dtype, G, T) && (shared_tile_sets(dtype, G, T) == 1 || (int64_t)T * G <= 96) &&
         !use_pingpong(dtype, G, T) && P == 4;
}

// Splits of one (request, KV head) that run as the parts of one workgroup
// and merge inside it: 4 or 2, else 1 (each split a workgroup of its own,
// merged afterwards by the merge kernel through the split workspace).  The
// workspace size, its check and the merge launch all follow this.
constexpr int shared_tile_parts(pa_dtype dtype, int G, int T, int P) {
  return shared_tile_quarters(dtype, G, T, P) ? 4 : (shared_tile_halves(dtype, G, T, P) ? 2 : 1);
}

// Waves of one shared-tile work item.
constexpr int shared_tile_waves(pa_dtype dtype, int G, int T) {
  return use_pingpong(dtype, G, T) ? kPingPongWaves : kSharedTileWaves;
}

// Query tokens one work item covers (DecodeArgs::TG = ceil(T / this)).
constexpr int tokens_per_item(pa_dtype dtype, int G, int T) {
  if (T <= 1) return 1;
  if (use_pingpong(dtype, G, T)) return kPingPongWaves * (32 / G);
  if (use_shared_tile(dtype, G, T)) return kSharedTileWaves * shared_tile_sets(dtype, G, T) * tokens_per_wave(dtype, G);
  return decode_column_sets(dtype, G, T) * tokens_per_wave(dtype, G);
}

// Sets the thread's pa_last_error() text (used by the host-only parts).
void set_last_error(const char* msg);

// Workspace floats for P splits: S*T*Hq*P*(d + 2).
size_t decode_workspace_floats(int64_t rows, int P);

// T == 1 runs the decode kernels; T > 1 their causal variants.
hipError_t launch_decode(const DecodeArgs& a, pa_dtype dtype, int B, int G, hipStream_t stream);

// bf16 on the matrix cores (pa_decode_mfma.hip); G in {1, 2, 4, 8, 16},
// B in {4, 8, 16, 32, 64}.
hipError_t launch_decode_mfma(const DecodeArgs& a, int B, int G, bool causal, hipStream_t stream);

// bf16, several query tokens per wave group (pa_extend_mfma.hip); G and B as above.
hipError_t launch_extend_shared(const DecodeArgs& a, int B, int G, hipStream_t stream);

// bf16, 32 query columns per wave on the 32x32 matrix-core tiles
// (pa_extend_wide.hip): the shared-tile step when each wave would take two
// 16-column sets, on 4 waves, or on the 8-wave ping-pong kernel when
// use_pingpong.  G and B as above.
hipError_t launch_extend_wide(const DecodeArgs& a, int B, int G, hipStream_t stream);

struct KvArgs {
  uint8_t* k_pool;
  uint8_t* v_pool;
  int S, MB, NB, B;
  int row_bytes;  // Hkv * d * element size: one slot of one block
};

// T tokens per request in each of num_layers layers: k_new/v_new
// [L, S, T, Hkv, d], token i at positions[s] + i; layer l's pools start
// l * layer_stride_bytes after layer 0's.
hipError_t launch_append(const KvArgs& a, const uint8_t* k_new, const uint8_t* v_new,
                         const int32_t* tables, const int32_t* positions, int T, int num_layers,
                         int64_t layer_stride_bytes, hipStream_t stream);

// order[r] = the request with the r-th longest length (ties by index).
hipError_t launch_order(const int32_t* lens, int S, int32_t* order, hipStream_t stream);

hipError_t launch_cow(const KvArgs& a, const int32_t* src, const int32_t* dst, const int32_t* n_valid,
                      int num_pairs, int num_layers, int64_t layer_stride_bytes, hipStream_t stream);

hipError_t launch_swap(const KvArgs& a, const int32_t* blocks, int nlist, uint8_t* buf, int num_layers,
                       int64_t layer_stride_bytes, bool to_buffer, hipStream_t stream);

hipError_t launch_gather(const KvArgs& a, const int32_t* tables, const int32_t* lens, uint8_t* k_out,
                         uint8_t* v_out, hipStream_t stream);

}  // namespace pa
