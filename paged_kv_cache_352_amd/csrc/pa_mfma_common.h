// Device helpers shared by the bf16 matrix-core kernels (the decode kernel
// in pa_decode_mfma.hip and the shared-tile several-token kernel in
// pa_extend_mfma.hip): vector types, the LDS tile layout, buffer-load
// descriptors, the XCD-aware work numbering, and the per-tile q.k / softmax /
// p.v step on the matrix cores.
//
// [Slides]  = "PagedAttention：让 KV cache 按需生长"
// [Budgets] = "内存预算约束下的语言模型服务：注意力、分页与调度"
#pragma once

#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pa {
namespace mfma {

constexpr int kWave = 64;
constexpr int kTile = 16;  // slots per MFMA tile (the M dimension of q.k)
constexpr float kNegInf = -__builtin_huge_valf();

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
#define PA_LDS __attribute__((address_space(3)))

// K tile in LDS: slot t, dims 8k .. 8k+7 (16-byte chunk k) at byte
//   256 * t + 16 * k_pos(k, t),  k_pos = k ^ t;
// V tile: the 32-byte pair of chunks k/2 is swizzled instead,
//   256 * t + 16 * v_pos(k, t),  v_pos = ((k/2 ^ (t % 8)) * 2) | (k % 2).
// A 16-byte row-wise write covers a whole row per 16 lanes, so any order of
// the chunks in a row suits it.  The K operand reads (16 lanes: 16 slots, one
// chunk each) need the chunk to move with the slot; the transposing V reads
// (32 lanes: 8 slots, 32 bytes each) need the pair to move with the slot, so
// that the 8 slots of one half-wave fall on 8 different 32-byte bank groups.
constexpr int kVtBytes = kTile * kHeadDim * 2;  // 4096

__device__ inline int k_pos(int k, int t) { return k ^ t; }
__device__ inline int v_pos(int k, int t) { return (((k >> 1) ^ (t & 7)) << 1) | (k & 1); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline int xcd_remap(int bid, int nwg) {
  const int x = bid % kNumXcd, k = bid / kNumXcd;
  const int q = nwg / kNumXcd, rem = nwg % kNumXcd;
  return x * q + min(x, rem) + k;
}

// bf16 head of an fp32 value by truncation, and the remainder's head:
// x - hi is exact in fp32 and lo = trunc(x - hi) leaves |x - hi - lo| < 2^-16 |x|.
__device__ inline void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const uint32_t b0 = __float_as_uint(x0) & 0xffff0000u;
  const uint32_t b1 = __float_as_uint(x1) & 0xffff0000u;
  const float r0 = x0 - __uint_as_float(b0);
  const float r1 = x1 - __uint_as_float(b1);
  hi = (b0 >> 16) | b1;
  lo = (__float_as_uint(r0) >> 16) | (__float_as_uint(r1) & 0xffff0000u);
}

// Orders this wave's LDS accesses around it without waiting for anything:
// one wave's LDS operations execute in issue order, so only the compiler has
// to be kept from moving them.
__device__ inline void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// K/V tiles are read with buffer loads: a descriptor for one physical block
// (uniform, in SGPRs) plus a 32-bit per-lane byte offset, so the per-lane
// addresses are four constant registers instead of a 64-bit address per load.
// The descriptor's size is the block's byte count: the hardware returns zero
// for any offset past it.
constexpr int kBufferFlags = 0x00020000;  // word 3 of a raw buffer descriptor on CDNA (32-bit data format)

__device__ inline __amdgpu_buffer_rsrc_t block_rsrc(const char* block, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(block), (short)0, (int)bytes, kBufferFlags);
}

// kStream: the load carries the non-temporal hint (cache-policy bit nt on
// gfx950), for data that one work item reads once and no other reads again
// soon: the decode kernel's K/V rows, and the shared-tile kernel's when one
// workgroup covers all query tokens of a history.  Same box, against plain
// loads, decode:
// 32 x 4096 tokens 96.0 -> 86.7 us, 256 mixed-length requests 59.3-60.0 ->
// 54.6 us per layer, 168 x 1025 tokens 70.8 -> 64.7 us per layer.
constexpr int kCachePolicyNT = 2;

template <bool kStream = false>
__device__ inline uint4 load_kv16(__amdgpu_buffer_rsrc_t r, uint32_t off, int soff) {
  return __builtin_bit_cast(uint4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, soff, kStream ? kCachePolicyNT : 0));
}

// LDS read addresses of one lane for a swizzled 16-slot K/V tile at kt / vt.
// K operand reads: slot n16, chunk 4*i + c4.  Transposing V reads for output
// dims 16*jj + n16: this lane fetches slot r = 4*c4 + n16/4, dims
// 16*jj + 4*(n16%4) .. +3, i.e. half (n16 & 1) of chunk 2*jj + (n16%4)/2,
// which sits at v_pos = ((jj ^ (r % 8)) * 2) | (n16%4)/2.
struct TileReads {
  const PA_LDS uint8_t* k;  // + 16 * chunk
  const PA_LDS uint8_t* v;  // + 16 * vchunk(jj)
  int rx, bsel;             // r % 8 and (n16 % 4) / 2

  __device__ inline TileReads(const uint8_t* kt, const uint8_t* vt, int n16, int c4) {
    const int rr = 4 * c4 + (n16 >> 2);
    k = (const PA_LDS uint8_t*)kt + 256 * n16;
    v = (const PA_LDS uint8_t*)vt + 256 * rr + 8 * (n16 & 1);
    bsel = (n16 & 3) >> 1;
    rx = rr & 7;
  }
  __device__ inline int vchunk(int jj) const { return ((jj ^ rx) << 1) | bsel; }
};

// Fold one 16-slot tile, already in LDS, into one wave's state for its 16
// columns ([Budgets] eq. (4)):
//   q.k  four v_mfma_f32_16x16x32_bf16, A = the K tile (M = 16 slots), B = q
//        (N = 16 columns); lane (n16, c4) gets column n16's scores for slots
//        4*c4 .. 4*c4+3;
//   mask slots at or past vq (the column's limit minus the tile's first
//        slot), the column's reference m (below), weights p = 2^(s - m),
//        partial l over the lane's four slots;
//   p.v  p split into a bf16 head and remainder (both through the matrix
//        core), B = V read transposed with ds_read_b64_tr_b16; acc[jj][r]
//        holds o of column 4*c4 + r, dims 16*jj + n16.
// The running max m is a reference, not always the exact max: it moves only
// when a tile's max exceeds it by more than kLazyMax (base 2), and then to
// that tile's max.  Weights are taken against it, so they stay below
// 2^kLazyMax, and l and o carry the same reference, so o / l and the merge
// of states (which rescales by 2^(m_w - M) whatever m_w is) are unchanged;
// the accumulators are rescaled only in the rare tiles where a reference
// moves.  With kMayBeEmpty a column may have no valid slot yet (m stays -inf
// and its state empty); without it the caller guarantees slot 0 of the tile
// is valid for every column.
// The core of the online-softmax step for one lane: sv holds the lane's R
// scores of column n16 (base 2, already masked to -inf past the column's
// limit); update the reference m (over the four lanes of the column, which
// sit 16 lanes apart), the partial sum l, rescale acc when some column's
// reference moved, and leave the weights p = 2^(s - m) in pw.
constexpr float kLazyMax = 8.f;

// With kRaw, sv holds unscaled scores and c >= 0 the base-2 scale (c > 0
// where a masked score is -inf): the tile max is taken on them and scaled
// once (c * max s = max c*s for c >= 0, rounding included), and each weight
// is 2^(fma(s, c, -m)), so no score is multiplied on its own.
//
// softmax_weights updates the column's state and weights, sets move where
// its reference moved and returns its alpha (1 where it stayed), leaving o
// to the caller; softmax_core also rescales o in the layout of the 16x16
// accumulators, where lane (n16, c4) holds columns 4*c4 .. +3.
template <int R, bool kMayBeEmpty, bool kSumL = true, bool kRaw = false>
__device__ __attribute__((always_inline)) inline float softmax_weights(const float (&sv)[R], float& m, float& l,
                                                                       float (&pw)[R], bool& move, float c = 1.f) {
  // Tile max over the column's slots.  v_permlane16_swap / 32_swap exchange
  // rows of 16 / 32 lanes in the vector ALU, so the max of each returned
  // pair is the max over the lane and its partner (lane ^ 16, then lane ^ 32)
  // without a round trip through the LDS crossbar.
  float bm = sv[0];
#pragma unroll
  for (int r = 1; r < R; ++r) bm = fmaxf(bm, sv[r]);
  {
    const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
    bm = fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
    const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
    bm = fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
  }
  if constexpr (kRaw) bm *= c;
  // A column that has seen nothing (m = -inf) moves to its first finite tile
  // max; one whose tile is all -inf (kMayBeEmpty) keeps its empty state.
  move = bm > m + kLazyMax;
  const float alpha = move ? fast_exp2(m - bm) : 1.f;
  if (move) m = bm;
  float mref = m;
  if constexpr (kMayBeEmpty) mref = (m == kNegInf) ? 0.f : m;
#pragma unroll
  for (int r = 0; r < R; ++r) pw[r] = kRaw ? fast_exp2(fmaf(sv[r], c, -mref)) : fast_exp2(sv[r] - mref);
  if constexpr (kSumL) {
    float sum = (pw[0] + pw[1]) + (pw[2] + pw[3]);
#pragma unroll
    for (int r = 4; r < R; r += 4) sum += (pw[r] + pw[r + 1]) + (pw[r + 2] + pw[r + 3]);
    l = fmaf(l, alpha, sum);
  }
  return alpha;
}

template <int R, bool kMayBeEmpty, bool kSumL = true, bool kRaw = false>
__device__ __attribute__((always_inline)) inline void softmax_core(const float (&sv)[R], f32x4_t (&acc)[8],
                                                                   float& m, float& l, int c4, float (&pw)[R],
                                                                   float c = 1.f) {
  bool move;
  const float alpha = softmax_weights<R, kMayBeEmpty, kSumL, kRaw>(sv, m, l, pw, move, c);
  // Rescale o only where a column's reference moved.
  if (__any(move)) {
    float ar[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * c4 + r, kWave);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[jj][r] *= ar[r];
  }
}

// The softmax part of the one-tile step: from the raw q.k scores sc of lane
// (n16, c4) (column n16, slots 4*c4 .. +3), mask, update the state and
// return p as bf16 head / remainder A operands of the 16-slot p.v.
template <bool kMayBeEmpty>
__device__ __attribute__((always_inline)) inline void softmax_step(const f32x4_t& sc, f32x4_t (&acc)[8], float& m,
                                                                   float& l, int vq, float scale_log2, int c4,
                                                                   s16x4_t& phi, s16x4_t& plo) {
  // Scores in base 2, masked past the column's limit ([Slides] quiz "逻辑顺序没错…").
  float sv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) sv[r] = (4 * c4 + r < vq) ? sc[r] * scale_log2 : kNegInf;
  float pw[4];
  softmax_core<4, kMayBeEmpty>(sv, acc, m, l, c4, pw);
  uint32_t hi0, hi1, lo0, lo1;
  split_pair(pw[0], pw[1], hi0, lo0);
  split_pair(pw[2], pw[3], hi1, lo1);
  phi = __builtin_bit_cast(s16x4_t, make_uint2(hi0, hi1));
  plo = __builtin_bit_cast(s16x4_t, make_uint2(lo0, lo1));
}

template <bool kMayBeEmpty>
__device__ __attribute__((always_inline)) inline void tile_update(const TileReads& rd, const bf16x8_t (&qv)[4],
                                                                  f32x4_t (&acc)[8], float& m, float& l, int vq,
                                                                  float scale_log2, int n16, int c4) {
  f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4_t kv = *reinterpret_cast<const PA_LDS u32x4_t*>(rd.k + 16 * k_pos(4 * i + c4, n16));
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kv), qv[i], sc, 0, 0, 0);
  }
  s16x4_t phi, plo;
  softmax_step<kMayBeEmpty>(sc, acc, m, l, vq, scale_log2, c4, phi, plo);

  wave_lds_order();  // this tile's V is in LDS
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int chunk = rd.vchunk(jj);
    const s16x4_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PA_LDS s16x4_t*)(rd.v + 16 * chunk));
    acc[jj] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, vb, acc[jj], 0, 0, 0);
    acc[jj] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, vb, acc[jj], 0, 0, 0);
  }
}

// The same step for NS sets of 16 columns at once (NS query-token groups of
// one wave): each K and V operand is read from LDS once and feeds NS sets of
// MFMAs, and the NS dependency chains interleave.
template <int NS, bool kMayBeEmpty>
__device__ __attribute__((always_inline)) inline void tile_update_sets(const TileReads& rd,
                                                                       const bf16x8_t (&qv)[NS][4],
                                                                       f32x4_t (&acc)[NS][8], float (&m)[NS],
                                                                       float (&l)[NS], const int (&vq)[NS],
                                                                       float scale_log2, int n16, int c4) {
  f32x4_t sc[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) sc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4_t kv = *reinterpret_cast<const PA_LDS u32x4_t*>(rd.k + 16 * k_pos(4 * i + c4, n16));
#pragma unroll
    for (int j = 0; j < NS; ++j)
      sc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kv), qv[j][i], sc[j], 0, 0, 0);
  }
  s16x4_t phi[NS], plo[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) softmax_step<kMayBeEmpty>(sc[j], acc[j], m[j], l[j], vq[j], scale_log2, c4, phi[j], plo[j]);

  wave_lds_order();  // this tile's V is in LDS
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int chunk = rd.vchunk(jj);
    const s16x4_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PA_LDS s16x4_t*)(rd.v + 16 * chunk));
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      acc[j][jj] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi[j], vb, acc[j][jj], 0, 0, 0);
      acc[j][jj] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo[j], vb, acc[j][jj], 0, 0, 0);
    }
  }
}

// Two fp32 values rounded to bf16 (to nearest, ties to even; one
// v_cvt_pk_bf16_f32), packed low then high.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ inline uint32_t pack_bf16_rn(float x0, float x1) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){x0, x1}, bf16x2_t));
}

// Head and remainder of two weights: hi = bf16(x) rounded to nearest, and
// lo = bf16(x - hi) rounded to nearest (x - hi is exact in fp32), so
// |x - hi - lo| <= 2^-9 |x - hi| <= 2^-18 |x|.
__device__ inline void split_pair_rn(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16_rn(x0, x1);
  lo = pack_bf16_rn(x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xffff0000u));
}

// The step for two consecutive tiles a and b (32 slots) and NS sets of 16
// columns.  q.k runs per tile as above, and the softmax takes the lane's 8
// scores (slots 4*c4 .. +3 of a, then of b).  p.v runs on
// v_mfma_f32_16x16x32_bf16, which does twice the work of the 16-slot
// instruction per issue: its K index 8*c4 + i stands for slot 4*c4 + i of
// tile a (i < 4) or of tile b (i >= 4).  It forms o transposed, o^T += V^T
// p^T: the A operand is the two transposing V reads (tile a, then tile b)
// of the lane side by side (16 dims by the 32 slots) and the B operand the
// lane's 8 weights in slot order (column n16).  Lane (n16, c4) so holds
// column n16 at dims 16*jj + 4*c4 .. +3 (acc[j][jj]): the column whose
// scores, max and alpha it already has, and a rescale is one multiply per
// element with no exchange between lanes.
//
// In the default form the V reads are issued with the K reads, before the
// softmax, whose latency hides theirs, and the rescale (rare under the lazy
// reference) runs on a branch that carries its own copy of the p.v
// products: with one copy after the join the compiler moved the 32
// accumulators to other registers on the common path every step.  The
// one-rounding form keeps one copy and late V reads, which hold it at three
// workgroups per CU.
//
// Default weights: p is split into a head and a remainder rounded to
// nearest (split_pair_rn), which keeps them within 2^-18 of p, and l is
// summed in fp32 per lane.  mask = false (the same in every lane): the
// caller has checked that both tiles lie wholly inside every column's
// limit; then no slot is masked, no column is empty, and the scores go in
// unscaled (scale_log2 >= 0 required), which saves a multiply, a compare
// and a select per score.
//
// kOneRounding (PA_FLAG_BF16_WEIGHTS): p is rounded once to bf16 (to
// nearest) and the softmax denominator is summed by the matrix core from the
// same rounded weights: lacc[j] += ones * p~^T, one extra MFMA per pair,
// holding the l of column n16 in every element.  o / l is then an exact
// weighted mean of V with weights p~ / sum p~, each p~ within 2^-9 of p
// relative, and rounding to nearest leaves no common sign to the errors, so
// they partly cancel over the history; p.v and l take 9 MFMAs per set
// instead of 16, with no split of p.  That form has one softmax path (the
// mask applied by selects where needed; two took its kernel past 256
// registers), with the scale kept at least FLT_MIN so that a masked -inf
// stays -inf (a zero scale then still gives equal weights: the scaled
// scores round to 0).
template <int NS, bool kMayBeEmpty, bool kOneRounding>
__device__ __attribute__((always_inline)) inline void pair_update_sets(const TileReads& ra, const TileReads& rb,
                                                                       const bf16x8_t (&qv)[NS][4],
                                                                       f32x4_t (&acc)[NS][8], f32x4_t (&lacc)[NS],
                                                                       float (&m)[NS], float (&l)[NS],
                                                                       const int (&vqa)[NS], const int (&vqb)[NS],
                                                                       float scale_log2, int n16, int c4, bool mask) {
  wave_lds_order();  // both tiles' K and V are in LDS
  f32x4_t sa[NS], sb[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    sa[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    sb[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // V^T operand jj: dims 16*jj .. +15 by the 32 slots.
  constexpr bool kEarlyV = !kOneRounding;
  auto read_vt = [&](int jj) {
    const s16x4_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PA_LDS s16x4_t*)(ra.v + 16 * ra.vchunk(jj)));
    const s16x4_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PA_LDS s16x4_t*)(rb.v + 16 * rb.vchunk(jj)));
    return __builtin_bit_cast(bf16x8_t, make_uint4(__builtin_bit_cast(uint2, va).x, __builtin_bit_cast(uint2, va).y,
                                                   __builtin_bit_cast(uint2, vb).x, __builtin_bit_cast(uint2, vb).y));
  };
  bf16x8_t vt[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4_t ka = *reinterpret_cast<const PA_LDS u32x4_t*>(ra.k + 16 * k_pos(4 * i + c4, n16));
    const u32x4_t kb = *reinterpret_cast<const PA_LDS u32x4_t*>(rb.k + 16 * k_pos(4 * i + c4, n16));
    if constexpr (kEarlyV) {
      vt[2 * i] = read_vt(2 * i);
      vt[2 * i + 1] = read_vt(2 * i + 1);
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      sa[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka), qv[j][i], sa[j], 0, 0, 0);
      sb[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kb), qv[j][i], sb[j], 0, 0, 0);
    }
  }

  bf16x8_t phi[NS], plo[NS];
  float alpha[NS];
  bool move[NS];
  if constexpr (kOneRounding) {
    const float c = fmaxf(scale_log2, __FLT_MIN__);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      float sv[8], pw[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sv[r] = sa[j][r];
        sv[4 + r] = sb[j][r];
        if (mask) {
          sv[r] = (4 * c4 + r < vqa[j]) ? sv[r] : kNegInf;
          sv[4 + r] = (4 * c4 + r < vqb[j]) ? sv[4 + r] : kNegInf;
        }
      }
      float unused = 0.f;
      alpha[j] = softmax_weights<8, kMayBeEmpty, false, true>(sv, m[j], unused, pw, move[j], c);
      phi[j] = __builtin_bit_cast(bf16x8_t, make_uint4(pack_bf16_rn(pw[0], pw[1]), pack_bf16_rn(pw[2], pw[3]),
                                                       pack_bf16_rn(pw[4], pw[5]), pack_bf16_rn(pw[6], pw[7])));
    }
  } else {
    auto weights = [&](int j, const float (&pw)[8]) {
      uint32_t h[4], lo[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) split_pair_rn(pw[2 * q], pw[2 * q + 1], h[q], lo[q]);
      phi[j] = __builtin_bit_cast(bf16x8_t, make_uint4(h[0], h[1], h[2], h[3]));
      plo[j] = __builtin_bit_cast(bf16x8_t, make_uint4(lo[0], lo[1], lo[2], lo[3]));
    };
    if (mask) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        float sv[8], pw[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sv[r] = (4 * c4 + r < vqa[j]) ? sa[j][r] * scale_log2 : kNegInf;
          sv[4 + r] = (4 * c4 + r < vqb[j]) ? sb[j][r] * scale_log2 : kNegInf;
        }
        alpha[j] = softmax_weights<8, kMayBeEmpty>(sv, m[j], l[j], pw, move[j]);
        weights(j, pw);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        float sv[8], pw[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sv[r] = sa[j][r];
          sv[4 + r] = sb[j][r];
        }
        alpha[j] = softmax_weights<8, false, true, true>(sv, m[j], l[j], pw, move[j], scale_log2);
        weights(j, pw);
      }
    }
  }

  auto products = [&] {
    if constexpr (kOneRounding) {
      const bf16x8_t ones =
          __builtin_bit_cast(bf16x8_t, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
#pragma unroll
      for (int j = 0; j < NS; ++j) lacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, phi[j], lacc[j], 0, 0, 0);
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      if constexpr (!kEarlyV) vt[jj] = read_vt(jj);
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        acc[j][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[jj], phi[j], acc[j][jj], 0, 0, 0);
        if constexpr (!kOneRounding)
          acc[j][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[jj], plo[j], acc[j][jj], 0, 0, 0);
      }
    }
  };
  bool moved = false;
#pragma unroll
  for (int j = 0; j < NS; ++j) moved = moved || move[j];
  auto rescale = [&] {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) acc[j][jj] *= alpha[j];
      if constexpr (kOneRounding) lacc[j] *= alpha[j];
    }
  };
  if constexpr (kOneRounding) {
    if (__any(moved)) rescale();
    products();
  } else if (__any(moved)) {
    rescale();
    products();
  } else {
    products();
  }
}

}  // namespace mfma
}  // namespace pa
