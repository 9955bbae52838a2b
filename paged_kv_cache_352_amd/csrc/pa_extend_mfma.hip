// Several query tokens per request on the matrix cores, with each K/V tile
// shared by the waves of a workgroup.
//
// [Slides]  = "PagedAttention：让 KV cache 按需生长"
// [Budgets] = "内存预算约束下的语言模型服务：注意力、分页与调度"
// [Serving] = "PagedAttention 与在线推理：KV 分页、共享及调度的联合分析"
//
// What is computed is the causal form of paged_attn_extend ([Serving] §5:
// speculative verification and prompt chunks read the same paged history as
// a decode step): the T new tokens are the last T positions of the n-token
// history, token i attends positions 0 .. n-T+i, each block is found through
// the table, slots past a column's limit are masked, and blocks fold into the
// (m, l, o) state of [Budgets] eq. (4); splits of the history are merged
// afterwards as for the decode.
//
// When the (token, head) pairs of a request's KV head outnumber the 16
// columns of two column sets of one wave, the decode layout would stream
// the history once per 32 columns.  Here a workgroup of 4 waves takes 4
// column sets, one per wave, which is how it runs: up to 4 sets of 16 columns
// fit one workgroup (16 tokens of a 4-head group) and the history is read
// once.  More tokens, two sets per wave, go to the 32-column kernel in
// pa_extend_wide.hip, which takes the same columns per wave on the 32x32
// tiles; the kSets = 2 form below stays as the reference of that layout (each
// K and V operand a wave reads from LDS feeds all of its sets).  The
// workgroup walks one split of the history tile by
// tile: every tile's K and V are loaded once, each wave fetching one group
// of 4 slot rows (16-byte lanes along a row, as in the decode kernel), and
// written to a double-buffered LDS tile in the swizzled layout.  Tiles go
// two at a time: after one workgroup barrier every wave runs the q.k /
// softmax / p.v step for its own columns on both tiles, p.v on the 32-deep
// MFMA (twice the work per issue of the 16-deep one).  With two LDS buffers
// one barrier per pair suffices: a wave overwrites buffer b only after the
// barrier of the next pair, which no wave passes before it has finished
// reading b.  Each wave owns its columns, so no state is merged inside the
// workgroup, except in the two-split form (kHalves below), whose two 4-wave
// halves walk one split each and merge their states at the end.
//
// The weights p enter p.v in one of two forms.  By default each is a bf16
// head plus a bf16 remainder, both rounded to nearest, through two MFMAs
// (weights within 2^-18 of p), and l is summed in fp32 by the vector ALU.
// With PA_FLAG_BF16_WEIGHTS each is rounded once to bf16 and l is summed by
// one more MFMA from the same rounded weights, so o / l stays a weighted
// mean of V: a third less matrix-core work per pair, weights within 2^-9.
#include <hip/hip_runtime.h>

#include "pa_mfma_common.h"

namespace pa {
namespace {

using namespace mfma;

constexpr int kWaves = kSharedTileWaves;  // = row groups of 4 slots per 16-slot tile
static_assert(kWaves * 4 == kTile, "each wave loads one 4-row group of a tile");
constexpr int kDepth = 2;  // tile pairs in flight per wave (this lane's K and V rows of two tiles each)

// kSets: 16-column sets per wave (1 or 2); each K and V operand read from
// LDS feeds all of them.  kOneRounding: p rounded once to bf16 and l summed
// on the matrix core from the rounded weights (PA_FLAG_BF16_WEIGHTS), else p
// as a bf16 head plus remainder and l summed in fp32 by the vector ALU.
// kHalves (two splits, one set per wave): one workgroup of 8 waves takes
// both splits of its (request, KV head), waves 0-3 the first and 4-7 the
// second, each half with its own LDS tiles; both pass the same barriers, and
// at the end the second half hands its state to the first through LDS, which
// merges the two as the merge kernel would (the same arithmetic, in split
// order, so the output is bitwise that of two workgroups and the merge
// kernel) and writes the output.  Against two workgroups of 4 waves on a CU
// it saves the partial states' round trip through memory and the merge
// kernel's launch.
template <int G, int kSets, int B, bool kOneRounding, bool kStream, bool kHalves = false>
__global__ __launch_bounds__(kWave * kWaves * (kHalves ? 2 : 1), kHalves ? 1 : 2) void extend_shared_kernel(DecodeArgs a) {
  static_assert(!kHalves || (kSets == 1 && kStream), "halves: one set per wave, one workgroup per request");
  static_assert(G >= 1 && G <= 16, "the query group must fit the 16 columns of one MFMA tile");
  static_assert(B >= 4 && B <= 64 && (B & (B - 1)) == 0, "block size: a power of two from 4 to 64");
  constexpr int TC = G >= 16 ? 1 : 16 / G;  // query tokens per 16-column set
  constexpr int TS = kSets * TC;            // query tokens per wave
  constexpr int TW = kWaves * TS;           // query tokens per workgroup
  // [half][buffer][tile a, tile b][K, V][tile bytes]
  __shared__ __attribute__((aligned(16))) uint8_t tiles_all[kHalves ? 2 : 1][2][2][2][kVtBytes];

  const int lane = threadIdx.x & (kWave - 1);
  // The wave index, in a scalar register: the compiler cannot see that it is
  // uniform, and block offsets and table lanes derived from it must be scalar.
  const int wt = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int grp = kHalves ? wt / kWaves : 0;  // kHalves: waves 0-3 take split 0, waves 4-7 split 1
  const int w = kHalves ? wt % kWaves : wt;
  auto& tiles = tiles_all[grp];
  const int n16 = lane & 15;
  const int c4 = lane >> 4;

  int item = xcd_remap(blockIdx.x, gridDim.x);
  int p = grp;
  if constexpr (!kHalves) {
    p = item % a.P;
    item /= a.P;
  }
  const int tw = item % a.TG;  // which TW query tokens of the request
  item /= a.TG;
  const int s = item % a.S;
  const int kvh = item / a.S;

  const int n_raw = a.lens[s];
  bool bad = n_raw < 0 || (int64_t)n_raw > (int64_t)a.MB * B;
  const int n = bad ? 0 : n_raw;
  const int nb = (n + B - 1) / B;
  // Column n16 of set j of wave w is query token tq[j], head kvh*G + n16%G,
  // and may see the first lim[j] positions; the workgroup needs the tiles up
  // to its last token's limit.
  int tq[kSets], lim[kSets];
#pragma unroll
  for (int j = 0; j < kSets; ++j) {
    tq[j] = tw * TW + w * TS + j * TC + n16 / G;
    lim[j] = tq[j] < a.T ? min(n, max(0, n - a.T + 1 + tq[j])) : n;
  }
  const int lim_hi = min(n, max(0, n - a.T + min(a.T, tw * TW + TW)));
  const int nt = (lim_hi + kTile - 1) / kTile;
  // A wave whose tokens all lie past T loads and writes its rows and passes
  // every barrier, but skips the arithmetic (nothing of it is stored).
  const bool idle = tw * TW + w * TS >= a.T;
  const int u0 = p * (a.tps / kTile);
  const int u1 = min(nt, u0 + a.tps / kTile);  // the same range for every wave

  // q enters the matrix core as given; with a negative scale it enters
  // negated (exact in bf16) and the magnitude of the scale is used, so the
  // scores are scaled by c >= 0 and keep their order: (-q).k * |c| = q.k * c.
  const bool neg_scale = a.scale_log2 < 0.f;
  const float c_log2 = neg_scale ? -a.scale_log2 : a.scale_log2;
  const uint32_t qsign = neg_scale ? 0x80008000u : 0u;
  bf16x8_t qv[kSets][4];
#pragma unroll
  for (int j = 0; j < kSets; ++j) {
    const bool live = tq[j] < a.T;  // columns past T get q = 0 and are never stored
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (((int64_t)s * a.T + min(tq[j], a.T - 1)) * a.Hq + (int64_t)kvh * G + n16 % G) * kHeadDim;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 v = *reinterpret_cast<const uint4*>(qp + 32 * i + 8 * c4);
      v = make_uint4(v.x ^ qsign, v.y ^ qsign, v.z ^ qsign, v.w ^ qsign);
      if (!live) v = make_uint4(0, 0, 0, 0);
      qv[j][i] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // This wave loads slot rows 4w .. 4w+3 of every tile: lane l takes row
  // 4w + c4, bytes 16*n16 .. +16 (KV head kvh).
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
  // Rows past the history (only in the last tile), and the loads of `none`
  // (a pair's second tile past the range, the prefetch slot past a chunk's
  // last pair), go through a descriptor of size 0: the hardware returns
  // zeros and reads no memory, the instruction count (and so every wait)
  // stays the same, and no table entry at or past ceil(n / B) addresses the
  // pool.  Those rows are zeroed or masked.  kStream: one workgroup covers all query tokens of
  // its (request, KV head) (a.TG == 1), so each K/V byte is read once and the
  // loads carry the non-temporal hint; otherwise several workgroups read the
  // same history, and it is left to the caches (measured on the 512-token
  // chunk: 414 vs 440 us without and with the hint).
  auto load_rows = [&](int u, uint4& k, uint4& v, int eb, int tab, bool none) {
    const int tok = kTile * u + 4 * w;
    const bool live = !none && tok < n;
    const uint32_t size = live ? blk_bytes : 0u;
    if constexpr (B >= kTile) {
      const int pb = live ? pool_block(__builtin_amdgcn_readlane(tab, (kTile * u) / B - eb)) : 0;
      const int soff = ((kTile * u) % B + 4 * w) * row_bytes;
      k = load_kv16<kStream>(block_rsrc(kpool + (int64_t)pb * blk_bytes, size), voff, soff);
      v = load_kv16<kStream>(block_rsrc(vpool + (int64_t)pb * blk_bytes, size), voff, soff);
    } else {
      const int pb = live ? pool_block(__builtin_amdgcn_readlane(tab, tok / B - eb)) : 0;
      const int soff = live ? (tok % B) * row_bytes : 0;
      k = load_kv16<kStream>(block_rsrc(kpool + (int64_t)pb * blk_bytes, size), voff, soff);
      v = load_kv16<kStream>(block_rsrc(vpool + (int64_t)pb * blk_bytes, size), voff, soff);
    }
  };

  float m[kSets];
  float l[kSets];       // two roundings: partial l of column n16 over this lane's slots
  f32x4_t lacc[kSets];  // one rounding: l of column n16 (in every element), in the layout of o^T
  f32x4_t acc[kSets][8];  // o^T: column n16 at dims 16*jj + 4*c4 .. +3
#pragma unroll
  for (int j = 0; j < kSets; ++j) {
    m[j] = kNegInf;
    l[j] = 0.f;
    lacc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) acc[j][jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const TileReads rd0(tiles[0][0][0], tiles[0][0][1], n16, c4);
  const int r_own = 4 * w + c4;                        // the slot row this lane writes
  const int wk_off = 256 * r_own + 16 * k_pos(n16, r_own);  // its swizzled byte offsets in a K
  const int wv_off = 256 * r_own + 16 * v_pos(n16, r_own);  // and in a V tile

  // This lane's rows of two consecutive tiles.
  struct Rows {
    uint4 ka, va, kb, vb;
  };
  // none: the prefetch slot past a chunk's last pair.  A second tile past the
  // range (an odd tile count) fetches nothing and is masked below.
  auto load_pair = [&](int t, Rows& r, int eb, int tab, int te, bool none) {
    load_rows(t, r.ka, r.va, eb, tab, none);
    load_rows(min(t + 1, te - 1), r.kb, r.vb, eb, tab, none || t + 1 >= te);
  };

  // Tiles t and t+1: write this lane's rows into buffer (t/2) & 1, wait for
  // the other waves' rows, then fold both tiles into this wave's columns.
  auto process = [&](int t, const Rows& r, int te) {
    const int buf = (t >> 1) & 1;
    const int tb_loaded = min(t + 1, te - 1);
    uint8_t* base = &tiles[buf][0][0][0];
    *reinterpret_cast<uint4*>(base + wk_off) = r.ka;
    *reinterpret_cast<uint4*>(base + kVtBytes + wv_off) = r_own < n - t * kTile ? r.va : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(base + 2 * kVtBytes + wk_off) = r.kb;
    *reinterpret_cast<uint4*>(base + 3 * kVtBytes + wv_off) =
        r_own < n - tb_loaded * kTile ? r.vb : make_uint4(0, 0, 0, 0);
    __syncthreads();
    if (idle || t >= te) return;
    TileReads ra = rd0, rb = rd0;
    ra.k += buf * (4 * kVtBytes);
    ra.v += buf * (4 * kVtBytes);
    rb.k += buf * (4 * kVtBytes) + 2 * kVtBytes;
    rb.v += buf * (4 * kVtBytes) + 2 * kVtBytes;
    int vqa[kSets], vqb[kSets];
#pragma unroll
    for (int j = 0; j < kSets; ++j) {
      vqa[j] = lim[j] - t * kTile;
      vqb[j] = t + 1 < te ? lim[j] - (t + 1) * kTile : 0;  // no tile b past the range
    }
    // Below the diagonal (both tiles inside every column's limit, as for all
    // but the last pairs of a chunk) nothing is masked and no column is
    // empty: the step without masks takes the scores unscaled.
    bool full = true;
#pragma unroll
    for (int j = 0; j < kSets; ++j) full = full && vqb[j] >= kTile;
    const bool mask = !__all(full);
    pair_update_sets<kSets, true, kOneRounding>(ra, rb, qv, acc, lacc, m, l, vqa, vqb, c_log2, n16, c4, mask);
  };

  // Table entries are read 64 at a time into one register (one per lane), as
  // in the decode kernel: chunks of 64 tiles for B >= 16, 4*B tiles below
  // (an even count, so a pair never straddles two chunks).  Within a chunk
  // the next pair is requested before the current one is used.
  constexpr int kChunkTiles = B >= kTile ? kWave : 4 * B;
  static_assert(kChunkTiles % 2 == 0, "pairs of tiles stay inside one chunk");
  if constexpr (kHalves) {
    // Both halves pass the same barriers: chunks and pairs are counted on the
    // first split's range (never shorter than the second's); a half past its
    // own range loads nothing (size-0 descriptors) and skips the arithmetic.
    const int c_u1 = min(nt, a.tps / kTile);
    for (int cb = 0; cb < c_u1; cb += kChunkTiles) {
      const int tb = u0 + cb;
      const int te = min(u1, tb + kChunkTiles);  // te <= tb: nothing of this half's own
      const int ce = min(c_u1, cb + kChunkTiles) - cb;
      const int eb = (kTile * tb) / B;
      const int tab = tb < te ? trow[min(eb + lane, nb - 1)] : 0;
      Rows ring[kDepth];
#pragma unroll
      for (int b = 0; b + 1 < kDepth; ++b)
        load_pair(max(tb, min(tb + 2 * b, te - 1)), ring[b], eb, tab, te, tb + 2 * b >= te);
      for (int t = 0; t < ce; t += 2 * kDepth) {
#pragma unroll
        for (int b = 0; b < kDepth; ++b) {
          constexpr int kNext = kDepth - 1;
          const int tn = tb + t + 2 * (b + kNext);
          load_pair(max(tb, min(tn, te - 1)), ring[(b + kNext) % kDepth], eb, tab, te, tn >= te);
          __builtin_amdgcn_sched_barrier(0);
          process(tb + t + 2 * b, ring[b], te);
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
#pragma unroll
      for (int b = 0; b + 1 < kDepth; ++b) load_pair(min(tb + 2 * b, te - 1), ring[b], eb, tab, te, tb + 2 * b >= te);
      for (int t = tb; t < te; t += 2 * kDepth) {
#pragma unroll
        for (int b = 0; b < kDepth; ++b) {
          constexpr int kNext = kDepth - 1;
          const int tn = t + 2 * (b + kNext);  // the pair to prefetch; past the chunk: loads that fetch nothing
          load_pair(min(tn, te - 1), ring[(b + kNext) % kDepth], eb, tab, te, tn >= te);
          __builtin_amdgcn_sched_barrier(0);  // issue the prefetch before the current pair's math
          process(t + 2 * b, ring[b], te);
          if (t + 2 * b + 2 >= te) break;
        }
      }
    }
  }

  // The full l of column n16 in every lane of it (the accumulators hold o^T:
  // lane (n16, c4) has column n16 at dims 16*jj + 4*c4 .. +3).
  float lc[kSets];
#pragma unroll
  for (int j = 0; j < kSets; ++j) {
    if constexpr (kOneRounding) {
      lc[j] = lacc[j][0];
    } else {
      lc[j] = l[j] + __shfl_xor(l[j], 16, kWave);  // the four lanes of column n16
      lc[j] += __shfl_xor(lc[j], 32, kWave);
    }
  }
  bad = __syncthreads_or(bad);  // any wave that met an entry outside the pool

  const float nan = __builtin_nanf("");
  if constexpr (kHalves) {
    // The second half's state goes to the first through LDS, lane for lane
    // (both halves hold the same columns in the same lanes), into the tiles'
    // space, free after the barrier above.  The first half merges the two
    // as the merge kernel does (M, then 2^(m_p - M) weights folded in split
    // order, o * (1 / L); an entry outside the pool gives NaN) and writes
    // the output.
    constexpr int kSlot = 2 + 32;  // m, l and o^T of one lane
    static_assert(kWaves * kWave * kSlot * 4 <= (int)sizeof(tiles_all), "the handed-over states fit the tiles");
    float* xs = reinterpret_cast<float*>(&tiles_all[0][0][0][0][0]);
    const int slot = (w * kWave + lane) * kSlot;
    if (grp == 1) {
      xs[slot] = m[0];
      xs[slot + 1] = lc[0];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) xs[slot + 2 + 4 * jj + r] = acc[0][jj][r];
    }
    __syncthreads();
    if (grp == 0 && tq[0] < a.T) {
      const float mv[2] = {bad ? 0.f : m[0], bad ? 0.f : xs[slot]};
      const float lv[2] = {bad ? nan : lc[0], bad ? nan : xs[slot + 1]};
      float M = kNegInf;
      M = fmaxf(M, mv[0]);
      M = fmaxf(M, mv[1]);
      const int64_t row = ((int64_t)s * a.T + tq[0]) * a.Hq + kvh * G + n16 % G;
      float* dst = a.out + row * kHeadDim + 4 * c4;
      if (M == kNegInf) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) *reinterpret_cast<f32x4_t*>(dst + 16 * jj) = f32x4_t{0.f, 0.f, 0.f, 0.f};
      } else {
        const float w0 = fast_exp2(mv[0] - M), w1 = fast_exp2(mv[1] - M);
        float L = 0.f;
        L = fmaf(w0, lv[0], L);
        L = fmaf(w1, lv[1], L);
        const float inv = 1.f / L;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          f32x4_t o;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float x = 0.f;
            x = fmaf(w0, acc[0][jj][r], x);
            x = fmaf(w1, xs[slot + 2 + 4 * jj + r], x);
            o[r] = x * inv;
          }
          *reinterpret_cast<f32x4_t*>(dst + 16 * jj) = o;
        }
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < kSets; ++j) {
    if (tq[j] >= a.T) continue;
    const int64_t row = ((int64_t)s * a.T + tq[j]) * a.Hq + kvh * G + n16 % G;
    if (a.P == 1) {
      const float inv = lc[j] > 0.f ? 1.f / lc[j] : 0.f;
      float* dst = a.out + row * kHeadDim + 4 * c4;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const f32x4_t o = acc[j][jj] * inv;
        *reinterpret_cast<f32x4_t*>(dst + 16 * jj) = bad ? f32x4_t{nan, nan, nan, nan} : o;
      }
    } else {
      const int64_t slot = row * a.P + p;
      float* dst = a.ws_o + slot * kHeadDim + 4 * c4;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) *reinterpret_cast<f32x4_t*>(dst + 16 * jj) = acc[j][jj];
      if (c4 == 0) {
        a.ws_m[slot] = bad ? 0.f : m[j];
        a.ws_l[slot] = bad ? nan : lc[j];
      }
    }
  }
}

template <int G, int B, bool kOneRounding>
void launch_gbr(const DecodeArgs& a, hipStream_t stream) {
  const int items = a.Hkv * a.S * a.P * a.TG;
  // One column set per wave is chosen only while one workgroup holds all T
  // tokens (a.TG == 1); two sets per wave go to the 32-column kernel
  // (pa_extend_wide.hip) instead.
  if (shared_tile_halves(PA_BF16, G, a.T, a.P)) {
    hipLaunchKernelGGL((extend_shared_kernel<G, 1, B, kOneRounding, true, true>), dim3(items / 2),
                       dim3(2 * kWave * kWaves), 0, stream, a);
    return;
  }
  hipLaunchKernelGGL((extend_shared_kernel<G, 1, B, kOneRounding, true>), dim3(items), dim3(kWave * kWaves), 0,
                     stream, a);
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

hipError_t launch_extend_shared(const DecodeArgs& a, int B, int G, hipStream_t stream) {
  // Two 16-column sets per wave: the same columns as one 32-column set of the
  // 32x32 kernel, which measured 6 % faster on a 512-token chunk (fewer
  // vector instructions per score; see pa_extend_wide.hip).  A four-split
  // plan of one set per wave runs there too, as four parts of two 32-column
  // waves in one workgroup.
  if (shared_tile_sets(PA_BF16, G, a.T) == 2 || shared_tile_quarters(PA_BF16, G, a.T, a.P))
    return launch_extend_wide(a, B, G, stream);
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
