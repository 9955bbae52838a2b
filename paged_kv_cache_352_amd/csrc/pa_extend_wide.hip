// Several query tokens per request on the 32x32 matrix-core tiles: the
// shared-tile kernel for query groups that give each wave 32 columns.
//
// [Slides]  = "PagedAttention：让 KV cache 按需生长"
// [Budgets] = "内存预算约束下的语言模型服务：注意力、分页与调度"
// [Serving] = "PagedAttention 与在线推理：KV 分页、共享及调度的联合分析"
//
// What is computed is the causal form of paged_attn_extend ([Serving] §5):
// the T new tokens are the last T positions of the n-token history, token i
// attends positions 0 .. n-T+i; each block is found through the table
// ([Slides] "读 token 6，先查表，再找偏移"), slots past a column's limit are
// masked ([Slides] quiz "逻辑顺序没错，为什么 attention 输出还是错？"), and the
// history folds into the online-softmax state (m, l, o) of [Budgets] eq. (4).
//
// A workgroup of 4 waves walks one split of one (request, KV head) history,
// 32 slots per step; each wave owns 32 columns, the (token, head) pairs of
// 32/G query tokens of the G-head group.  Each step's 32 K and V slot rows
// are loaded once (every wave fetches 8 rows: two 4-row groups of 16-byte
// lanes; 16 rows in the four-part form below), written to a double-buffered
// LDS tile, and after one barrier every wave folds the whole step into its
// own columns.  The products are taken
// transposed so that a lane owns one column throughout:
//
//   scores  S^T = K Q^T on v_mfma_f32_32x32x16_bf16: A = K (32 slots x 16
//           dims, from LDS), B = Q^T (16 dims x 32 columns, in registers),
//           8 MFMAs over d = 128.  Lane l gets column l%32 for the 16 slots
//           8*(r/4) + 4*(l/32) + r%4, r = 0..15, so the column max is a max
//           over its 16 values and one v_permlane32_swap with the lane 32
//           away, which holds the other 16 slots.
//   p.v     O^T += V^T P^T: A = V^T (32 dims x 16 slots), read from the
//           row-major V tile by ds_read_b64_tr_b16, B = P^T (16 slots x 32
//           columns).  B's K index 8*(l/32) + i of lane l stands for slot
//           i < 4 ? 4*(l/32) + i : 8 + 4*(l/32) + i - 4 of the 16-slot half,
//           which is exactly the order of the lane's own score registers
//           8*kb .. 8*kb+7, so the weights feed p.v without leaving the lane;
//           A reads the same slot order.  The accumulators hold o^T of the
//           lane's own column (dims 32*mb + 8*(r/4) + 4*(l/32) + r%4), so a
//           rescale needs the lane's own factor only.
//
// Weights as in the 16-column kernel: by default each p is a bf16 head plus a
// bf16 remainder, both rounded to nearest (within 2^-18 of p), through two
// MFMAs, and l is summed in fp32; with PA_FLAG_BF16_WEIGHTS each p is rounded
// once to bf16 and l is summed on the matrix core from the same rounded
// weights.  The running max is the lazy reference of the 16-column kernel
// (moved only when a step's max exceeds it by more than kLazyMax, base 2).
//
// Query groups wider than 128 columns run on the ping-pong form below: 8 such
// waves per workgroup, two per SIMD, kept one phase apart so that the matrix
// products of one overlap the softmax of the other.  Its per-column
// arithmetic is the same, step for step, so both forms give the same bits.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "pa_mfma_common.h"

namespace pa {
namespace {

using namespace mfma;

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kWaves = kSharedTileWaves;
constexpr int kStep = 32;                        // slots per step
constexpr int kStepBytes = kStep * kHeadDim * 2;  // one K or V step in LDS: 8 KiB

// K step in LDS: slot t, 16-byte chunk k at 256*t + 16*(k ^ (t % 16)); the
// q.k reads (32 lanes: 32 slots, one chunk each) then meet 16 different
// chunks in every 16-lane group.  V step: the 32-byte pair of chunks k/2 at
// 256*t + 32*((k/2) ^ g(t)) + 16*(k % 2), g(t) = 2*(t % 4) + (t / 4) % 2.  A
// transposing read takes, in each half-wave, two neighbouring pairs (32
// dims) of 4 slots t = 4i .. 4i+3, 8 bytes per lane: g gives those 4 slots
// the even (or odd) values, so the two pairs land on all 8 32-byte bank
// groups once.  (With g(t) = t % 8 they met only 4 of them, two ways each:
// about 32 conflict cycles per 32-slot step and wave, though removing them
// did not change the measured times.)
__device__ inline int kw_pos(int k, int t) { return k ^ (t & 15); }
__device__ inline int vw_perm(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }
__device__ inline int vw_pos(int k, int t) { return (((k >> 1) ^ vw_perm(t)) << 1) | (k & 1); }

// kParts = 2 or 4: one workgroup takes all splits of its (request, KV head),
// one part of waves per split, each part with its own LDS steps and all
// passing the same barriers; at the end the other parts hand their states to
// the first, which merges them as the merge kernel would (M, then the
// 2^(m_p - M) weights folded in split order) and writes the output, so no
// partial state goes through memory and no merge kernel runs.  Two parts
// (two splits) have 4 waves of 32 columns each, as the one-split form, and
// give bitwise the result of two workgroups and the merge kernel.  Four
// parts (four splits, up to 64 columns: 9-16 tokens of a 4-head group) have
// 2 waves each, so every wave loads 16 rows of each step and the workgroup
// holds 8 waves and four parts' double-buffered steps (128 KiB of LDS).
// Measured on 32 x 4096 tokens with 16 tokens of 4-head groups against two
// halves of four 16-column waves (pa_extend_mfma.hip): 95.3 against
// 101.8-103.7 us, each wave's step on the 32x32 tiles doing a 16-column
// wave's work twice over with fewer vector instructions per score, and half
// as many steps and barriers.  kColsArg = 3 (four parts of three waves, up to
// 96 columns: 17-24 tokens of a 4-head group) puts 12 waves, three per SIMD,
// in the workgroup, held to 168 registers: q is read from LDS for every
// product (24 KiB, written once by the first part) instead of 32 registers,
// each wave loads 3 row groups of a step (the last wave 2), and the next
// step is requested right after the current one is written to LDS, so one
// set of row registers serves both.  The states are handed over in two
// rounds.  Against two halves of four 32-column waves, the fourth of them
// idle at 24 tokens, every SIMD then runs three waves over a quarter of the
// history each instead of two over a half (or none): 32 x 4096 tokens,
// T = 18-24, 111.7-115.2 against 117.6-123.9 us.
template <int G, int B, bool kOneRounding, bool kStream, int kParts = 1, int kColsArg = 0>
__global__ __launch_bounds__(kWave * (kColsArg ? kColsArg : (kParts == 4 ? 2 : kWaves)) * kParts,
                             kParts > 1 ? 1 : 2) void extend_wide_kernel(DecodeArgs a) {
  constexpr bool kJoined = kParts > 1;  // the splits are parts of this workgroup
  static_assert(kParts == 1 || kParts == 2 || kParts == 4, "one, two or four splits per workgroup");
  static_assert(!kJoined || kStream, "parts: one workgroup per (request, KV head)");
  constexpr int kCW = kColsArg ? kColsArg : (kParts == 4 ? 2 : kWaves);  // column waves per split
  constexpr int kRG = (8 + kCW - 1) / kCW;  // 4-row groups of a step each wave loads (the last wave may load fewer)
  constexpr bool kQLds = kCW == 3;           // q read from LDS each step (registers for 12 waves)
  static_assert(G >= 1 && G <= 16, "32 columns hold 32/G whole query tokens");
  static_assert(B >= 4 && B <= 64 && (B & (B - 1)) == 0, "block size: a power of two from 4 to 64");
  constexpr int TC = 32 / G;        // query tokens per wave
  constexpr int TW = kCW * TC;      // query tokens per workgroup
  // [part][buffer][K, V][step bytes]
  __shared__ __attribute__((aligned(16))) uint8_t steps_all[kParts][2][2][kStepBytes];
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[kQLds ? kCW * 32 * 256 : 16];

  const int lane = threadIdx.x & (kWave - 1);
  // The wave index, in a scalar register (block offsets and table lanes
  // derived from it must be scalar).
  const int wt = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int grp = kJoined ? wt / kCW : 0;  // the part: the first kCW waves take split 0, and so on
  const int w = kJoined ? wt % kCW : wt;
  auto& steps = steps_all[grp];
  const int col = lane & 31;  // this lane's column
  const int h = lane >> 5;    // which half of the column's slots it holds
  const int n16 = lane & 15;
  const int c4 = lane >> 4;

  int item = xcd_remap(blockIdx.x, gridDim.x);
  int p = grp;
  if constexpr (!kJoined) {
    p = item % a.P;
    item /= a.P;
  }
  const int tw = item % a.TG;
  item /= a.TG;
  const int s = item % a.S;
  const int kvh = item / a.S;

  const int n_raw = a.lens[s];
  bool bad = n_raw < 0 || (int64_t)n_raw > (int64_t)a.MB * B;
  const int n = bad ? 0 : n_raw;
  const int nb = (n + B - 1) / B;
  // Column col is query token tq, head kvh*G + col%G, and may see the first
  // lim positions; the workgroup needs the tiles up to its last token's limit.
  const int tq = tw * TW + w * TC + col / G;
  const int lim = tq < a.T ? min(n, max(0, n - a.T + 1 + tq)) : n;
  const int lim_hi = min(n, max(0, n - a.T + min(a.T, tw * TW + TW)));
  const int nt = (lim_hi + kTile - 1) / kTile;  // 16-slot tiles
  const int u0 = p * (a.tps / kTile);
  const int u1 = min(nt, u0 + a.tps / kTile);
  // A wave whose tokens all lie past T (T not a multiple of the workgroup's
  // tokens) still loads and writes its rows of every step and passes every
  // barrier, but skips the arithmetic: nothing of it is stored, and its SIMD
  // goes to the other workgroup's wave.
  const bool idle = tw * TW + w * TC >= a.T;

  // q^T as the B operand of S^T = K q^T: lane l holds column col over dims
  // 16*kk + 8*h .. +8.  A negative scale enters as q negated (exact in bf16)
  // and the scale's magnitude, so scores are scaled by c >= 0.
  const bool neg_scale = a.scale_log2 < 0.f;
  const float c_log2 = neg_scale ? -a.scale_log2 : a.scale_log2;
  const uint32_t qsign = neg_scale ? 0x80008000u : 0u;
  bf16x8_t qv[kQLds ? 1 : 8];
  const int q_base = 256 * (w * 32 + col);
  {
    const bool live = tq < a.T;  // columns past T get q = 0 and are never stored
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (((int64_t)s * a.T + min(tq, a.T - 1)) * a.Hq + (int64_t)kvh * G + col % G) * kHeadDim;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      uint4 v = *reinterpret_cast<const uint4*>(qp + 16 * kk + 8 * h);
      v = make_uint4(v.x ^ qsign, v.y ^ qsign, v.z ^ qsign, v.w ^ qsign);
      if (!live) v = make_uint4(0, 0, 0, 0);
      if constexpr (kQLds) {
        if (grp == 0) *reinterpret_cast<uint4*>(q_lds + q_base + 16 * kw_pos(2 * kk + h, col)) = v;
      } else {
        qv[kk] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
    if constexpr (kQLds) __syncthreads();
  }

  // This wave loads slot rows 4g + c4 of every step, row groups g = kRG*w + i
  // below 8 (8w + 4i + c4 with four waves): lane l takes bytes 16*n16 .. +16
  // of KV head kvh.  A row group wholly past the
  // history, past the split, or in a prefetch slot past the chunk (`none`)
  // goes through a descriptor of size 0: zeros, no memory read, and no table
  // entry at or past ceil(n / B) addresses the pool.
  const int row_bytes = a.Hkv * kHeadDim * 2;
  const uint32_t blk_bytes = (uint32_t)B * (uint32_t)row_bytes;
  const uint32_t voff = (uint32_t)(c4 * row_bytes + (kvh * kHeadDim + 8 * n16) * 2);
  const char* kpool = static_cast<const char*>(a.k_pool);
  const char* vpool = static_cast<const char*>(a.v_pool);
  const int32_t* trow = a.tables + (int64_t)s * a.MB;
  auto pool_block = [&](int pb) {
    if (pb < 0 || pb >= a.NB) {  // outside the pool: never dereferenced, result poisoned
      bad = true;
      pb = 0;
    }
    return pb;
  };
  struct Rows {
    uint4 k[kRG], v[kRG];
  };
  // Step starting at tile t: slots 16t .. 16t+31; `te` ends the chunk (and
  // the split): a second tile at or past it is not part of the step.
  auto load_step = [&](int t, Rows& r, int eb, int tab, int te, bool none) {
#pragma unroll
    for (int i = 0; i < kRG; ++i) {
      const int g = min(kRG * w + i, 7);  // the row group (past 7: none, the last wave's spare slot)
      const int tok = kTile * t + 4 * g;  // first slot of the row group
      const bool live = !none && kRG * w + i < 8 && tok < n && (4 * g < kTile || t + 1 < te);
      const int pb = live ? pool_block(__builtin_amdgcn_readlane(tab, tok / B - eb)) : 0;
      const int soff = live ? (tok % B) * row_bytes : 0;
      const uint32_t size = live ? blk_bytes : 0u;
      r.k[i] = load_kv16<kStream>(block_rsrc(kpool + (int64_t)pb * blk_bytes, size), voff, soff);
      r.v[i] = load_kv16<kStream>(block_rsrc(vpool + (int64_t)pb * blk_bytes, size), voff, soff);
    }
  };

  float m = kNegInf;  // reference max (base 2) of this lane's column
  float l = 0.f;      // two roundings: partial l over this lane's 16 slots of each step
  f32x16_t lacc = {}; // one rounding: l of the column (every element), from the rounded weights
  f32x16_t acc[4];    // o^T of the column: dims 32*mb + 8*(r/4) + 4*h + r%4
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x16_t{};

  // LDS offsets this lane writes (rows 4g + c4, chunk n16) and reads.
  int wk_off[kRG], wv_off[kRG];
#pragma unroll
  for (int i = 0; i < kRG; ++i) {
    const int r = 4 * min(kRG * w + i, 7) + c4;
    wk_off[i] = 256 * r + 16 * kw_pos(n16, r);
    wv_off[i] = 256 * r + 16 * vw_pos(n16, r);
  }
  // q.k A operand: slot col, chunk 2*kk + h.
  const int rk_base = 256 * col;
  // p.v A operand: lane (group g16 = lane/16, j = lane%16) reads slot
  // 16*kb + 8*sec + 4*h + j/4, dims 32*mb + 16*(g16%2) + 4*(j%4) .. +3; the
  // slot's position in its 8-row swizzle group, (4*h + j/4) % 8, does not
  // depend on kb or sec, so one offset per mb serves all four reads.
  int rv_off[4];
  {
    const int j = lane & 15;
    const int rr = 4 * h + j / 4;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int pair = 2 * mb + ((lane >> 4) & 1);
      rv_off[mb] = 256 * rr + 32 * (pair ^ vw_perm(rr)) + 8 * (j & 3);
    }
  }

  auto process = [&](int t, const Rows& r, int te, auto&& after_write) {
    const int buf = (t >> 1) & 1;
    uint8_t* kb_ = &steps[buf][0][0];
    uint8_t* vb_ = &steps[buf][1][0];
    const int valid = n - kTile * t;  // slots of the step inside the history
#pragma unroll
    for (int i = 0; i < kRG; ++i)
      if (kRG * w + i < 8) *reinterpret_cast<uint4*>(kb_ + wk_off[i]) = r.k[i];
    if (valid >= kStep) {  // the whole step lies inside the history (all but the last)
#pragma unroll
      for (int i = 0; i < kRG; ++i)
        if (kRG * w + i < 8) *reinterpret_cast<uint4*>(vb_ + wv_off[i]) = r.v[i];
    } else {
      // V past the history may hold anything (NaN): zeroed, since a zero
      // weight times NaN would still be NaN.
#pragma unroll
      for (int i = 0; i < kRG; ++i) {
        if (kRG * w + i >= 8) continue;
        const int row = 4 * (kRG * w + i) + c4;
        *reinterpret_cast<uint4*>(vb_ + wv_off[i]) = row < valid ? r.v[i] : make_uint4(0, 0, 0, 0);
      }
    }
    after_write();
    __syncthreads();
    if (idle || t >= te) return;

    // S^T = K q^T over d = 128.
    f32x16_t sc = {};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const u32x4_t kv = *reinterpret_cast<const PA_LDS u32x4_t*>((const PA_LDS uint8_t*)kb_ + rk_base +
                                                                  16 * kw_pos(2 * kk + h, col));
      bf16x8_t qk;
      if constexpr (kQLds)
        qk = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const PA_LDS u32x4_t*>(
                                              (const PA_LDS uint8_t*)q_lds + q_base + 16 * kw_pos(2 * kk + h, col)));
      else
        qk = qv[kk];
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kv), qk, sc, 0, 0, 0);
    }

    // Slots of this step the column may see: below its limit, and in the
    // second tile only while that tile is part of the split.
    int vq = lim - kTile * t;
    if (t + 1 >= te) vq = min(vq, kTile);
    // Below the diagonal every slot counts for every column: the scores go
    // in unscaled and unmasked.
    const bool mask = !__all(vq >= kStep);
    float sv[16];
    if (mask) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int slot = 8 * (rr >> 2) + 4 * h + (rr & 3);
        sv[rr] = slot < vq ? sc[rr] : kNegInf;
      }
    } else {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sv[rr] = sc[rr];
    }
    // Column max: the lane's 16 slots, then the other 16 in the lane 32 away.
    float bm = fmaxf(fmaxf(sv[0], sv[1]), sv[2]);
#pragma unroll
    for (int rr = 3; rr < 15; rr += 2) bm = fmaxf(fmaxf(bm, sv[rr]), sv[rr + 1]);
    bm = fmaxf(bm, sv[15]);
    {
      const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
      bm = fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
    }
    // The scale enters once: c * max s = max c*s for c >= 0 (rounding
    // included), and each weight is 2^fma(s, c, -m).  c is kept at least
    // FLT_MIN so that a masked -inf stays -inf (a zero scale then still gives
    // equal weights: the scaled scores round to about 0).
    const float c = fmaxf(c_log2, __FLT_MIN__);
    bm *= c;
    const bool move = bm > m + kLazyMax;
    const float alpha = move ? fast_exp2(m - bm) : 1.f;
    if (move) m = bm;
    const float mref = m == kNegInf ? 0.f : m;  // a column with nothing valid yet keeps weights 0
    float pw[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) pw[rr] = fast_exp2(fmaf(sv[rr], c, -mref));
    if (__any(move)) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) acc[mb][rr] *= alpha;
      if constexpr (kOneRounding) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) lacc[rr] *= alpha;
      }
    }

    // P^T operands: weights 8*kb .. 8*kb+7 of this lane, in register order.
    bf16x8_t phi[2], plo[2] = {};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (kOneRounding) {
          hi[q] = pack_bf16_rn(pw[8 * kb + 2 * q], pw[8 * kb + 2 * q + 1]);
        } else {
          split_pair_rn(pw[8 * kb + 2 * q], pw[8 * kb + 2 * q + 1], hi[q], lo[q]);
        }
      }
      phi[kb] = __builtin_bit_cast(bf16x8_t, make_uint4(hi[0], hi[1], hi[2], hi[3]));
      if constexpr (!kOneRounding) plo[kb] = __builtin_bit_cast(bf16x8_t, make_uint4(lo[0], lo[1], lo[2], lo[3]));
    }
    if constexpr (kOneRounding) {
      const bf16x8_t ones =
          __builtin_bit_cast(bf16x8_t, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) lacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, phi[kb], lacc, 0, 0, 0);
    } else {
      float sum = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) sum += (pw[4 * q] + pw[4 * q + 1]) + (pw[4 * q + 2] + pw[4 * q + 3]);
      l = fmaf(l, alpha, sum);
    }

    // O^T += V^T P^T.
    const PA_LDS uint8_t* vrd = (const PA_LDS uint8_t*)vb_;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (PA_LDS s16x4_t*)(vrd + rv_off[mb] + 256 * (kTile * kb)));
        const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (PA_LDS s16x4_t*)(vrd + rv_off[mb] + 256 * (kTile * kb + 8)));
        const bf16x8_t va = __builtin_bit_cast(
            bf16x8_t, make_uint4(__builtin_bit_cast(uint2, v0).x, __builtin_bit_cast(uint2, v0).y,
                                 __builtin_bit_cast(uint2, v1).x, __builtin_bit_cast(uint2, v1).y));
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, phi[kb], acc[mb], 0, 0, 0);
        if constexpr (!kOneRounding) acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, plo[kb], acc[mb], 0, 0, 0);
      }
    }
  };

  // Table entries 64 at a time into one register (one per lane): chunks of
  // 64 tiles for B >= 16, 4*B tiles below.  Within a chunk the next step is
  // requested before the current one is used.
  constexpr int kChunkTiles = B >= kTile ? kWave : 4 * B;
  static_assert(kChunkTiles % 2 == 0, "steps of two tiles stay inside one chunk");
  constexpr int kDepth = 2;
  if constexpr (kJoined) {
    // All parts pass the same barriers: chunks and steps are counted on the
    // first split's range (never shorter than the others'); a part past its
    // own range loads nothing (size-0 descriptors) and skips the arithmetic.
    const int c_u1 = min(nt, a.tps / kTile);
    for (int cb = 0; cb < c_u1; cb += kChunkTiles) {
      const int tb = u0 + cb;
      const int te = min(u1, tb + kChunkTiles);
      const int ce = min(c_u1, cb + kChunkTiles) - cb;
      const int eb = (kTile * tb) / B;
      const int tab = tb < te ? trow[min(eb + lane, nb - 1)] : 0;
      if constexpr (kQLds) {
        // One set of row registers: the next step is requested right after
        // the current one is written to LDS, before the barrier.
        Rows cur;
        load_step(max(tb, min(tb, te - 1)), cur, eb, tab, te, tb >= te);
        for (int t = 0; t < ce; t += 2) {
          const int tn = tb + t + 2;
          process(tb + t, cur, te, [&] { load_step(max(tb, min(tn, te - 1)), cur, eb, tab, te, tn >= te); });
        }
        continue;
      }
      Rows ring[kDepth];
      load_step(max(tb, min(tb, te - 1)), ring[0], eb, tab, te, tb >= te);
      for (int t = 0; t < ce; t += 2 * kDepth) {
#pragma unroll
        for (int b = 0; b < kDepth; ++b) {
          const int tn = tb + t + 2 * (b + 1);
          load_step(max(tb, min(tn, te - 1)), ring[(b + 1) % kDepth], eb, tab, te, tn >= te);
          __builtin_amdgcn_sched_barrier(0);
          process(tb + t + 2 * b, ring[b], te, [] {});
          if (t + 2 * b + 2 >= ce) break;
        }
      }
    }
  } else {
    for (int tb = u0; tb < u1; tb += kChunkTiles) {
      const int te = min(u1, tb + kChunkTiles);
      const int eb = (kTile * tb) / B;
      const int tab = trow[min(eb + lane, nb - 1)];
      Rows ring[kDepth];
      load_step(tb, ring[0], eb, tab, te, false);
      for (int t = tb; t < te; t += 2 * kDepth) {
#pragma unroll
        for (int b = 0; b < kDepth; ++b) {
          const int tn = t + 2 * (b + 1);  // the step to prefetch; past the chunk: loads that fetch nothing
          load_step(min(tn, te - 1), ring[(b + 1) % kDepth], eb, tab, te, tn >= te);
          __builtin_amdgcn_sched_barrier(0);  // issue the prefetch before the current step's math
          process(t + 2 * b, ring[b], te, [] {});
          if (t + 2 * b + 2 >= te) break;
        }
      }
    }
  }

  // The column's l: the two lanes holding its halves.
  float lc;
  if constexpr (kOneRounding) {
    lc = lacc[0];
  } else {
    lc = l + __shfl_xor(l, 32, kWave);
  }
  bad = __syncthreads_or(bad);  // any wave that met an entry outside the pool

  const float nan = __builtin_nanf("");
  if constexpr (kParts == 4) {
    // Parts 1-3 hand their states to part 0, lane for lane, through the
    // steps' LDS (in two rounds of two accumulator blocks when one does not
    // fit); part 0 merges the four as the merge kernel does (M, then
    // 2^(m_p - M) weights folded in split order, o * (1 / L)) and writes the
    // output.
    float* xs = reinterpret_cast<float*>(&steps_all[0][0][0][0]);
    constexpr bool kOneRound = (kParts - 1) * kCW * kWave * (2 + 64) * 4 <= (int)sizeof(steps_all);
    constexpr int kRounds = kOneRound ? 1 : 2;
    constexpr int kMB = 4 / kRounds;  // accumulator blocks per round
    constexpr int kSlot = 2 + 16 * kMB;
    static_assert((kParts - 1) * kCW * kWave * kSlot * 4 <= (int)sizeof(steps_all), "the states fit the steps");
    float wq[kParts];
    float inv = 0.f;
    bool empty = true;
    const int64_t row = ((int64_t)s * a.T + tq) * a.Hq + kvh * G + col % G;
    float* dst = a.out + row * kHeadDim + 4 * h;
#pragma unroll
    for (int round = 0; round < kRounds; ++round) {
      if (round > 0) __syncthreads();  // the previous round's values have been read
      if (grp > 0) {
        const int slot = (((grp - 1) * kCW + w) * kWave + lane) * kSlot;
        if (round == 0) {
          xs[slot] = m;
          xs[slot + 1] = lc;
        }
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) xs[slot + 2 + 16 * mb + r] = acc[kMB * round + mb][r];
      }
      __syncthreads();
      if (grp == 0 && tq < a.T) {
        if (round == 0) {
          float mv[kParts], lv[kParts];
          mv[0] = bad ? 0.f : m;
          lv[0] = bad ? nan : lc;
#pragma unroll
          for (int q = 1; q < kParts; ++q) {
            const int slot = (((q - 1) * kCW + w) * kWave + lane) * kSlot;
            mv[q] = bad ? 0.f : xs[slot];
            lv[q] = bad ? nan : xs[slot + 1];
          }
          float M = kNegInf;
#pragma unroll
          for (int q = 0; q < kParts; ++q) M = fmaxf(M, mv[q]);
          empty = M == kNegInf;
          float L = 0.f;
#pragma unroll
          for (int q = 0; q < kParts; ++q) {
            wq[q] = empty ? 0.f : fast_exp2(mv[q] - M);
            L = fmaf(wq[q], lv[q], L);
          }
          inv = 1.f / L;
        }
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float x = 0.f;
              x = fmaf(wq[0], acc[kMB * round + mb][4 * q4 + e], x);
#pragma unroll
              for (int q = 1; q < kParts; ++q) {
                const int slot = (((q - 1) * kCW + w) * kWave + lane) * kSlot;
                x = fmaf(wq[q], xs[slot + 2 + 16 * mb + 4 * q4 + e], x);
              }
              o[e] = empty ? 0.f : x * inv;
            }
            *reinterpret_cast<float4*>(dst + 32 * (kMB * round + mb) + 8 * q4) = make_float4(o[0], o[1], o[2], o[3]);
          }
      }
    }
    return;
  } else if constexpr (kJoined) {
    // The second half's state goes to the first, lane for lane (both halves
    // hold the same columns in the same lanes), through the steps' LDS (free
    // after the barrier above), in two rounds of two accumulator blocks.  The
    // first half merges as the merge kernel does (M, then 2^(m_p - M)
    // weights folded in split order, o * (1 / L); an entry outside the pool
    // gives NaN) and writes the output.
    float* xs = reinterpret_cast<float*>(&steps_all[0][0][0][0]);
    constexpr int kSlot = 2 + 32;
    static_assert(kWaves * kWave * kSlot * 4 <= (int)sizeof(steps_all), "the handed-over states fit the steps");
    const int slot = (w * kWave + lane) * kSlot;
    float w0 = 0.f, w1 = 0.f, inv = 0.f;
    bool empty = true;
    const int64_t row = ((int64_t)s * a.T + tq) * a.Hq + kvh * G + col % G;
    float* dst = a.out + row * kHeadDim + 4 * h;
#pragma unroll
    for (int round = 0; round < 2; ++round) {
      if (round > 0) __syncthreads();  // the first round's values have been read
      if (grp == 1) {
        if (round == 0) {
          xs[slot] = m;
          xs[slot + 1] = lc;
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) xs[slot + 2 + 16 * mb + r] = acc[2 * round + mb][r];
      }
      __syncthreads();
      if (grp == 0 && tq < a.T) {
        if (round == 0) {
          const float m0 = bad ? 0.f : m, m1 = bad ? 0.f : xs[slot];
          const float l0 = bad ? nan : lc, l1 = bad ? nan : xs[slot + 1];
          float M = kNegInf;
          M = fmaxf(M, m0);
          M = fmaxf(M, m1);
          empty = M == kNegInf;
          if (!empty) {
            w0 = fast_exp2(m0 - M);
            w1 = fast_exp2(m1 - M);
            float L = 0.f;
            L = fmaf(w0, l0, L);
            L = fmaf(w1, l1, L);
            inv = 1.f / L;
          }
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float x = 0.f;
              x = fmaf(w0, acc[2 * round + mb][4 * q + e], x);
              x = fmaf(w1, xs[slot + 2 + 16 * mb + 4 * q + e], x);
              o[e] = empty ? 0.f : x * inv;
            }
            *reinterpret_cast<float4*>(dst + 32 * (2 * round + mb) + 8 * q) = make_float4(o[0], o[1], o[2], o[3]);
          }
      }
    }
    return;
  }
  if (tq < a.T) {
    const int64_t row = ((int64_t)s * a.T + tq) * a.Hq + kvh * G + col % G;
    if (a.P == 1) {
      const float inv = lc > 0.f ? 1.f / lc : 0.f;
      float* dst = a.out + row * kHeadDim + 4 * h;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 o = bad ? make_float4(nan, nan, nan, nan)
                               : make_float4(acc[mb][4 * q] * inv, acc[mb][4 * q + 1] * inv,
                                             acc[mb][4 * q + 2] * inv, acc[mb][4 * q + 3] * inv);
          *reinterpret_cast<float4*>(dst + 32 * mb + 8 * q) = o;
        }
    } else {
      const int64_t slot = row * a.P + p;
      float* dst = a.ws_o + slot * kHeadDim + 4 * h;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<float4*>(dst + 32 * mb + 8 * q) =
              make_float4(acc[mb][4 * q], acc[mb][4 * q + 1], acc[mb][4 * q + 2], acc[mb][4 * q + 3]);
      if (h == 0) {
        a.ws_m[slot] = bad ? 0.f : m;
        a.ws_l[slot] = bad ? nan : lc;
      }
    }
  }
}


// The ping-pong form, for query groups of more than 128 columns: 8 waves of
// 32 columns each (256 columns: the (token, head) pairs of 256/G query
// tokens), all folding the same 32-slot steps.  The hardware places waves w
// and w+4 of a workgroup on the same SIMD; waves 0-3 (group A) and 4-7 (group
// B) run one phase apart, so that on every SIMD one wave issues matrix
// products while the other runs vector work:
//
//   phase 2j:    A: M(j)      B: V(j-1)
//   phase 2j+1:  A: V(j)      B: M(j)
//
// M(j) takes q.k of step j and p.v of step j-1; V(x) takes the softmax of
// step x, the LDS write of this wave's rows of step j+1 and the request of
// step j+4.  A workgroup barrier ends every phase.  Step k sits in LDS buffer
// k % 3 from phase 2k-2 (written) to 2k+3 (its V read by B), so three
// buffers (48 KiB) hold every step in use.  Both groups pass the same
// barriers in their own copy of the loop.
//
// The scheduler could move vector work across a barrier into the other
// phase (it did: the softmax sank into the next matrix phase); each barrier
// is therefore fenced for the scheduler and the state live across it is
// pinned with empty asm statements, so every instruction stays in its phase.
template <int G, int B, bool kOneRounding, bool kStream>
__global__ __launch_bounds__(kWave * kPingPongWaves, 1) void extend_pingpong_kernel(DecodeArgs a) {
  static_assert(G >= 1 && G <= 16, "32 columns hold 32/G whole query tokens");
  static_assert(B >= 4 && B <= 64 && (B & (B - 1)) == 0, "block size: a power of two from 4 to 64");
  constexpr int TC = 32 / G;                // query tokens per wave
  constexpr int TW = kPingPongWaves * TC;   // query tokens per workgroup
  constexpr int kBufs = 3;
  // [buffer][K, V][step bytes]
  __shared__ __attribute__((aligned(16))) uint8_t steps[kBufs][2][kStepBytes];

  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const bool late = w >= kPingPongWaves / 2;  // group B
  const int col = lane & 31;
  const int h = lane >> 5;
  const int n16 = lane & 15;
  const int c4 = lane >> 4;

  int item = xcd_remap(blockIdx.x, gridDim.x);
  const int p = item % a.P;
  item /= a.P;
  const int tw = item % a.TG;
  item /= a.TG;
  const int s = item % a.S;
  const int kvh = item / a.S;

  const int n_raw = a.lens[s];
  bool bad = n_raw < 0 || (int64_t)n_raw > (int64_t)a.MB * B;
  const int n = bad ? 0 : n_raw;
  const int tq = tw * TW + w * TC + col / G;
  const int lim = tq < a.T ? min(n, max(0, n - a.T + 1 + tq)) : n;
  const int lim_hi = min(n, max(0, n - a.T + min(a.T, tw * TW + TW)));
  const int nt = (lim_hi + kTile - 1) / kTile;  // 16-slot tiles
  const int u0 = p * (a.tps / kTile);
  const int u1 = min(nt, u0 + a.tps / kTile);
  const int nsteps = u1 > u0 ? (u1 - u0 + 1) / 2 : 0;  // step k: tiles u0+2k, u0+2k+1 (if < u1)
  const int base_slot = kTile * u0;
  // A wave whose tokens all lie past T loads, writes and passes every barrier
  // but skips its matrix and vector work (nothing of it is stored); it runs a
  // loop copy of its own, so the others' copies carry no test for it.
  const bool idle = tw * TW + w * TC >= a.T;

  const bool neg_scale = a.scale_log2 < 0.f;
  const float c_log2 = neg_scale ? -a.scale_log2 : a.scale_log2;
  const uint32_t qsign = neg_scale ? 0x80008000u : 0u;
  bf16x8_t qv[8];
  {
    const bool live = tq < a.T;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (((int64_t)s * a.T + min(tq, a.T - 1)) * a.Hq + (int64_t)kvh * G + col % G) * kHeadDim;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      uint4 v = *reinterpret_cast<const uint4*>(qp + 16 * kk + 8 * h);
      v = make_uint4(v.x ^ qsign, v.y ^ qsign, v.z ^ qsign, v.w ^ qsign);
      if (!live) v = make_uint4(0, 0, 0, 0);
      qv[kk] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // This wave loads slot rows 4w .. 4w+3 of every step (one 16-byte lane of
  // K and of V each; a row group never straddles a block, B >= 4).  The
  // block comes from the table through the constant address space, so it is
  // a scalar load, requested at the start of the vector phase that uses it.
  // A vector load of table entries kept across loop iterations made the
  // compiler wait for every K/V load in flight before each LDS write.
  const int row_bytes = a.Hkv * kHeadDim * 2;
  const uint32_t blk_bytes = (uint32_t)B * (uint32_t)row_bytes;
  const uint32_t voff = (uint32_t)(c4 * row_bytes + (kvh * kHeadDim + 8 * n16) * 2);
  const char* kpool = static_cast<const char*>(a.k_pool);
  const char* vpool = static_cast<const char*>(a.v_pool);
  typedef const __attribute__((address_space(4))) int32_t ctab_t;
  ctab_t* ctab = (ctab_t*)(a.tables + (int64_t)s * a.MB);  // read-only for the whole launch
  // Whether this wave's row group of step k holds history: inside the split,
  // inside the history, and (rows 16-31) in a second tile of the split.
  auto rows_live = [&](int k) {
    const int tok = base_slot + kStep * k + 4 * w;
    return k < nsteps && tok < n && (4 * w < kTile || u0 + 2 * k + 1 < u1);
  };
  auto table_entry = [&](int k) { return rows_live(k) ? ctab[(base_slot + kStep * k + 4 * w) / B] : 0; };
  struct Ld {
    uint4 k, v;
  };
  // A dead row group, or an entry outside the pool (which poisons the
  // output), loads through a descriptor of size 0: zeros, no memory read.
  auto load_step = [&](int k, int e, Ld& r) {
    const bool live = rows_live(k);
    const bool in_pool = e >= 0 && e < a.NB;
    if (live && !in_pool) bad = true;
    const bool fetch = live && in_pool;
    const int tok = base_slot + kStep * k + 4 * w;
    const int soff = fetch ? (tok % B) * row_bytes : 0;
    const char* kb = kpool + (fetch ? (int64_t)e * blk_bytes : 0);
    const char* vb = vpool + (fetch ? (int64_t)e * blk_bytes : 0);
    r.k = load_kv16<kStream>(block_rsrc(kb, fetch ? blk_bytes : 0u), voff, soff);
    r.v = load_kv16<kStream>(block_rsrc(vb, fetch ? blk_bytes : 0u), voff, soff);
  };

  const int wrow = 4 * w + c4;
  const int wk_off = 256 * wrow + 16 * kw_pos(n16, wrow);
  const int wv_off = 256 * wrow + 16 * vw_pos(n16, wrow);
  // V rows past the history may hold anything (NaN): written as zeros, since
  // a zero weight times NaN would still be NaN.
  auto write_step = [&](int k, const Ld& r, uint8_t* kb_, uint8_t* vb_) {
    const int valid = n - base_slot - kStep * k;
    *reinterpret_cast<uint4*>(kb_ + wk_off) = r.k;
    *reinterpret_cast<uint4*>(vb_ + wv_off) = wrow < valid ? r.v : make_uint4(0, 0, 0, 0);
  };

  float m = kNegInf;   // reference max (base 2) of this lane's column
  float l = 0.f;       // two roundings: partial l over this lane's 16 slots of each step
  f32x16_t lacc = {};  // one rounding: l of the column, from the rounded weights
  f32x16_t acc[4];     // o^T of the column: dims 32*mb + 8*(r/4) + 4*h + r%4
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x16_t{};
  f32x16_t sc = {};               // scores of the step between its M and V phases
  bf16x8_t phi[2] = {}, plo[2] = {};  // weights between the V phase and the next M phase

  const int rk_base = 256 * col;
  int rv_off[4];
  {
    const int j = lane & 15;
    const int rr = 4 * h + j / 4;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int pair = 2 * mb + ((lane >> 4) & 1);
      rv_off[mb] = 256 * rr + 32 * (pair ^ vw_perm(rr)) + 8 * (j & 3);
    }
  }
  const float c = fmaxf(c_log2, __FLT_MIN__);

  // M(j): q.k of step j (K in kb_; all 8 reads issued first), then p.v of
  // step j-1 (V in vb_).
  auto mphase = [&](int j, const uint8_t* kb_, const uint8_t* vb_) {
    if (j < nsteps) {
      u32x4_t kr[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        kr[kk] = *reinterpret_cast<const PA_LDS u32x4_t*>((const PA_LDS uint8_t*)kb_ + rk_base +
                                                          16 * kw_pos(2 * kk + h, col));
      f32x16_t z = {};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kr[kk]), qv[kk], z, 0, 0, 0);
      sc = z;
    }
    if (j > 0 && j <= nsteps) {
      if constexpr (kOneRounding) {
        const bf16x8_t ones =
            __builtin_bit_cast(bf16x8_t, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) lacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, phi[kb], lacc, 0, 0, 0);
      }
      const PA_LDS uint8_t* vrd = (const PA_LDS uint8_t*)vb_;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (PA_LDS s16x4_t*)(vrd + rv_off[mb] + 256 * (kTile * kb)));
          const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (PA_LDS s16x4_t*)(vrd + rv_off[mb] + 256 * (kTile * kb + 8)));
          const bf16x8_t va = __builtin_bit_cast(
              bf16x8_t, make_uint4(__builtin_bit_cast(uint2, v0).x, __builtin_bit_cast(uint2, v0).y,
                                   __builtin_bit_cast(uint2, v1).x, __builtin_bit_cast(uint2, v1).y));
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, phi[kb], acc[mb], 0, 0, 0);
          if constexpr (!kOneRounding)
            acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, plo[kb], acc[mb], 0, 0, 0);
        }
      }
    }
  };

  // Softmax of step x into the p.v operands (the same arithmetic as the
  // 4-wave kernel, so the two give bitwise equal outputs).
  auto softmax = [&](int x) {
    int vq = lim - base_slot - kStep * x;
    if (u0 + 2 * x + 1 >= u1) vq = min(vq, kTile);
    const bool mask = !__all(vq >= kStep);
    float sv[16];
    if (mask) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int slot = 8 * (rr >> 2) + 4 * h + (rr & 3);
        sv[rr] = slot < vq ? sc[rr] : kNegInf;
      }
    } else {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sv[rr] = sc[rr];
    }
    float bm = fmaxf(fmaxf(sv[0], sv[1]), sv[2]);
#pragma unroll
    for (int rr = 3; rr < 15; rr += 2) bm = fmaxf(fmaxf(bm, sv[rr]), sv[rr + 1]);
    bm = fmaxf(bm, sv[15]);
    {
      const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
      bm = fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
    }
    bm *= c;
    const bool move = bm > m + kLazyMax;
    const float alpha = move ? fast_exp2(m - bm) : 1.f;
    if (move) m = bm;
    const float mref = m == kNegInf ? 0.f : m;
    float pw[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) pw[rr] = fast_exp2(fmaf(sv[rr], c, -mref));
    if (__any(move)) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) acc[mb][rr] *= alpha;
      if constexpr (kOneRounding) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) lacc[rr] *= alpha;
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (kOneRounding) {
          hi[q] = pack_bf16_rn(pw[8 * kb + 2 * q], pw[8 * kb + 2 * q + 1]);
        } else {
          split_pair_rn(pw[8 * kb + 2 * q], pw[8 * kb + 2 * q + 1], hi[q], lo[q]);
        }
      }
      phi[kb] = __builtin_bit_cast(bf16x8_t, make_uint4(hi[0], hi[1], hi[2], hi[3]));
      if constexpr (!kOneRounding) plo[kb] = __builtin_bit_cast(bf16x8_t, make_uint4(lo[0], lo[1], lo[2], lo[3]));
    }
    if constexpr (!kOneRounding) {
      float sum = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) sum += (pw[4 * q] + pw[4 * q + 1]) + (pw[4 * q + 2] + pw[4 * q + 3]);
      l = fmaf(l, alpha, sum);
    }
  };

  // Phase boundaries.  After an M phase the scores are live, after a V phase
  // the weights; the accumulators and the running state always.
  auto pin_common = [&] {
    if constexpr (!kOneRounding) asm volatile("" : "+v"(l));
    if constexpr (kOneRounding) asm volatile("" : "+v"(lacc));
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) asm volatile("" : "+v"(acc[mb]));
    asm volatile("" : "+v"(m));
  };
  auto pin_scores = [&] {
    asm volatile("" : "+v"(sc));
    pin_common();
  };
  auto pin_weights = [&] {
    asm volatile("" : "+v"(phi[0]), "+v"(phi[1]));
    if constexpr (!kOneRounding) asm volatile("" : "+v"(plo[0]), "+v"(plo[1]));
    pin_common();
  };
  auto barrier_after_m = [&] {
    pin_scores();
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    pin_scores();
  };
  auto barrier_after_v = [&] {
    pin_weights();
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    pin_weights();
  };

  // Prologue: steps 0-2 requested, step 0 written, step 3 requested into the
  // freed registers.  Step k's registers are ring[k % 3].
  Ld ring[3];
  load_step(0, table_entry(0), ring[0]);
  load_step(1, table_entry(1), ring[1]);
  load_step(2, table_entry(2), ring[2]);
  if (nsteps > 0) write_step(0, ring[0], &steps[0][0][0], &steps[0][1][0]);
  load_step(3, table_entry(3), ring[0]);
  __syncthreads();

  // Iterations j = 0 .. nsteps, three per trip so that buffer and register
  // indices are compile-time; a trip runs all three (steps past the end do
  // nothing), which keeps the compiler's count of loads in flight exact: an
  // early exit from the unrolled trip made it wait for every load in flight.
  auto run = [&](auto late_group, auto idle_wave) {
    constexpr bool kLate = decltype(late_group)::value;
    constexpr bool kIdle = decltype(idle_wave)::value;
    for (int j0 = 0; j0 <= nsteps; j0 += kBufs) {
#pragma unroll
      for (int b = 0; b < kBufs; ++b) {
        const int j = j0 + b;
        const uint8_t* kcur = &steps[b][0][0];
        const uint8_t* vprev = &steps[(b + kBufs - 1) % kBufs][1][0];
        uint8_t* knext = &steps[(b + 1) % kBufs][0][0];
        uint8_t* vnext = &steps[(b + 1) % kBufs][1][0];
        Ld& rn = ring[(b + 1) % kBufs];
        auto vphase = [&](int x) {
          const int e = table_entry(j + 4);  // scalar load, used at the end of the phase
          if constexpr (!kIdle)
            if (x >= 0 && x < nsteps) softmax(x);
          if (j + 1 < nsteps) write_step(j + 1, rn, knext, vnext);
          load_step(j + 4, e, rn);
        };
        if constexpr (kLate) {
          vphase(j - 1);
          barrier_after_v();
          if constexpr (!kIdle) mphase(j, kcur, vprev);
          barrier_after_m();
        } else {
          if constexpr (!kIdle) mphase(j, kcur, vprev);
          barrier_after_m();
          vphase(j);
          barrier_after_v();
        }
      }
    }
  };
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;
  if (late) {
    if (idle)
      run(yes{}, yes{});
    else
      run(yes{}, no{});
  } else {
    if (idle)
      run(no{}, yes{});
    else
      run(no{}, no{});
  }

  float lc;
  if constexpr (kOneRounding) {
    lc = lacc[0];
  } else {
    lc = l + __shfl_xor(l, 32, kWave);
  }
  bad = __syncthreads_or(bad);

  const float nan = __builtin_nanf("");
  if (tq < a.T) {
    const int64_t row = ((int64_t)s * a.T + tq) * a.Hq + kvh * G + col % G;
    if (a.P == 1) {
      const float inv = lc > 0.f ? 1.f / lc : 0.f;
      float* dst = a.out + row * kHeadDim + 4 * h;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 o = bad ? make_float4(nan, nan, nan, nan)
                               : make_float4(acc[mb][4 * q] * inv, acc[mb][4 * q + 1] * inv,
                                             acc[mb][4 * q + 2] * inv, acc[mb][4 * q + 3] * inv);
          *reinterpret_cast<float4*>(dst + 32 * mb + 8 * q) = o;
        }
    } else {
      const int64_t slot = row * a.P + p;
      float* dst = a.ws_o + slot * kHeadDim + 4 * h;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<float4*>(dst + 32 * mb + 8 * q) =
              make_float4(acc[mb][4 * q], acc[mb][4 * q + 1], acc[mb][4 * q + 2], acc[mb][4 * q + 3]);
      if (h == 0) {
        a.ws_m[slot] = bad ? 0.f : m;
        a.ws_l[slot] = bad ? nan : lc;
      }
    }
  }
}

template <int G, int B, bool kOneRounding>
void launch_gbr(const DecodeArgs& a, hipStream_t stream) {
  const int items = a.Hkv * a.S * a.P * a.TG;
  if (use_pingpong(PA_BF16, G, a.T)) {
    if (a.TG == 1)
      hipLaunchKernelGGL((extend_pingpong_kernel<G, B, kOneRounding, true>), dim3(items),
                         dim3(kWave * kPingPongWaves), 0, stream, a);
    else
      hipLaunchKernelGGL((extend_pingpong_kernel<G, B, kOneRounding, false>), dim3(items),
                         dim3(kWave * kPingPongWaves), 0, stream, a);
    return;
  }
  if (shared_tile_quarters(PA_BF16, G, a.T, a.P)) {
    if (shared_tile_sets(PA_BF16, G, a.T) == 2)
      hipLaunchKernelGGL((extend_wide_kernel<G, B, kOneRounding, true, 4, 3>), dim3(items / 4), dim3(4 * kWave * 3),
                         0, stream, a);
    else
      hipLaunchKernelGGL((extend_wide_kernel<G, B, kOneRounding, true, 4>), dim3(items / 4), dim3(4 * kWave * 2), 0,
                         stream, a);
    return;
  }
  if (shared_tile_halves(PA_BF16, G, a.T, a.P)) {
    hipLaunchKernelGGL((extend_wide_kernel<G, B, kOneRounding, true, 2>), dim3(items / 2),
                       dim3(2 * kWave * kWaves), 0, stream, a);
    return;
  }
  if (a.TG == 1)
    hipLaunchKernelGGL((extend_wide_kernel<G, B, kOneRounding, true>), dim3(items), dim3(kWave * kWaves), 0, stream,
                       a);
  else
    hipLaunchKernelGGL((extend_wide_kernel<G, B, kOneRounding, false>), dim3(items), dim3(kWave * kWaves), 0, stream,
                       a);
}

template <int G, int B>
hipError_t launch_gb(const DecodeArgs& a, hipStream_t stream) {
  if (a.bf16_weights)
    launch_gbr<G, B, true>(a, stream);
  else
    launch_gbr<G, B, false>(a, stream);
  return hipGetLastError();
}

template <int B>
hipError_t launch_b(const DecodeArgs& a, int G, hipStream_t stream) {
  switch (G) {
    case 1: return launch_gb<1, B>(a, stream);
    case 2: return launch_gb<2, B>(a, stream);
    case 4: return launch_gb<4, B>(a, stream);
    case 8: return launch_gb<8, B>(a, stream);
    case 16: return launch_gb<16, B>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_extend_wide(const DecodeArgs& a, int B, int G, hipStream_t stream) {
  switch (B) {
    case 4: return launch_b<4>(a, G, stream);
    case 8: return launch_b<8>(a, G, stream);
    case 16: return launch_b<16>(a, G, stream);
    case 32: return launch_b<32>(a, G, stream);
    case 64: return launch_b<64>(a, G, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
