// Paged-attention decode for bf16 K/V on the CDNA4 matrix cores.
//
// [Slides]  = "PagedAttention：让 KV cache 按需生长"
// [Budgets] = "内存预算约束下的语言模型服务：注意力、分页与调度"
//
// Same contract as the vector-ALU kernel in pa_decode.hip ([Slides]
// "分页以后，attention 仍然按完整历史归一化": look up each logical block,
// load its K/V tile, mask slots past the length, fold the block into the
// running (m, l, o) state of [Budgets] eq. (4); partial states over disjoint
// block sets are merged).  What changes is where the arithmetic runs: the two
// contractions of the GQA group, q.k and p.v, are MFMA instructions, which
// leaves the vector ALU only the softmax of four scores per lane.
//
// Work decomposition.  The history is cut into 16-slot tiles (the M
// dimension of the q.k MFMA), whatever the block size B (a power of two from
// 4 to 64: a tile is part of one block, or spans 16/B blocks).  One workgroup
// of W waves per (request s, KV head g, split p); the split's tiles are dealt
// to the waves in turn (wave w takes tiles w, w + W, ...), each wave keeps
// its own (m, l, o), and the W states are merged through LDS at the end.
// Which tiles a wave takes depends only on the split, not on the length, so
// its first table entries and first tile are requested before the length
// has arrived.  With one split the workgroup writes the
// final output; with several it writes its merged state and a second kernel
// merges the splits.
//
// Loads.  One tile of one KV head is 16 slot rows of 256 bytes, Hkv*256
// bytes apart in the [block, slot, KV head, dim] pool ([Slides] "把 token 6
// 变成真正的内存地址").  Each 16-byte load instruction of a wave covers a group
// of 4 whole rows (lane l: row 4*i + l/16, bytes 16*(l%16)), so every row is
// fetched as full cache lines by one instruction; B >= 4 keeps each group in
// one block.  The loads are buffer loads: a descriptor for the block
// (uniform, in SGPRs) plus constant 32-bit lane offsets, with the
// non-temporal hint, since every K/V byte is read once.  The next tile's K
// and V are in flight while the current one is processed.  Each wave stages
// its K and V tiles in its own LDS in the swizzled layouts of
// pa_mfma_common.h (k_pos, v_pos), which keep the row-wise writes and the
// operand reads below free of bank conflicts.
//
// Math for one wave and one 16-slot tile, head dim 128; lane l is
// (n = l%16, c = l/16):
//
//   q.k  four v_mfma_f32_16x16x32_bf16 with A = the K tile (M = 16 slots,
//        K = 32 dims; lane l reads slot n, dims 32*i + 8*c .. +8 from LDS)
//        and B = q of the group (N = 16 query heads, zero beyond G; lane l
//        holds head n over the same dims), so the products pair up whatever
//        order the hardware sums them in.  The result leaves lane l with the
//        scores of head n for slots 4c .. 4c+3.
//   p.v  that is exactly the A layout (M = 16 heads, K = 16 slots, 4 slots
//        per lane) of v_mfma_f32_16x16x16_bf16, so the weights feed p.v
//        without crossing lanes.  Its B operand needs V with slots along K:
//        ds_read_b64_tr_b16 reads the row-major V tile transposed, handing
//        lane (n, c) the dims 16*j + n of slots 4c .. 4c+3.  p is split into
//        a bf16 head and a bf16 remainder (p = hi + lo to about 2^-16
//        relative) and both go through the matrix core, so p.v keeps
//        fp32-class accuracy.  The eight accumulators hold o for heads
//        4c .. 4c+3, dims 16*j + n.
//
// Softmax state: lane l keeps m (the running max, base 2) of head n and a
// partial l over its own four slots of every tile; the partials of the four
// lanes of a head are summed once at the end.  The accumulators are rescaled
// only in tiles where some head's max moved.
//
// Several query tokens (the causal variant).  A verification step or a
// prompt chunk brings T new tokens per request, already appended as the last
// T positions of the history; token i attends positions 0 .. n-T+i
// ([Serving] §5 sets speculative decoding beside paging).  The 16 columns of
// the MFMA tile then hold (token, head) pairs: 16/G tokens of the G-head
// group per column set, and a wave keeps one or two sets (NS), so up to
// 32/G tokens cost one pass over the history; each K and V operand read from
// LDS feeds both sets.  Each column carries its own length limit; a column
// whose limit lies before a tile sees only -inf there, and its state stays
// empty (m = -inf, l = 0, o = 0) until a tile reaches it.  Still more tokens
// go to the shared-tile kernel (pa_extend_mfma.hip).
#include <hip/hip_runtime.h>

#include "pa_mfma_common.h"

namespace pa {
namespace {

using namespace mfma;

// K/V tiles in flight per wave.
constexpr int kDepth = 2;

struct Tile {
  uint4 k[4];
  uint4 v[4];
};

// NS: 16-column sets per wave (2 only with several query tokens: each K and
// V operand a wave reads from LDS then feeds both sets).  kAppend: the step's
// new token is appended in the same launch (one query token only).
template <int G, bool kCausal, int NS, int W, int B, bool kAppend = false>
__global__ __launch_bounds__(kWave * W) void decode_mfma_kernel(DecodeArgs a) {
  static_assert(G >= 1 && G <= 16, "the query group must fit the 16 columns of one MFMA tile");
  static_assert(B >= 4 && B <= 64 && (B & (B - 1)) == 0, "block size: a power of two from 4 to 64");
  static_assert(NS == 1 || (NS == 2 && kCausal), "two column sets only for several query tokens");
  static_assert(!(kAppend && kCausal), "the fused append is for one query token");
  constexpr int TC = kCausal ? (G >= 16 ? 1 : 16 / G) : 1;  // query tokens per column set
  constexpr int NC = G * TC;                                  // MFMA columns in use per set
  __shared__ __attribute__((aligned(16))) uint8_t vt_all[W][kVtBytes];
  __shared__ __attribute__((aligned(16))) uint8_t kt_all[W][kVtBytes];
  __shared__ float red_m[W][16];
  __shared__ float red_l[W][16];
  // o per wave and column; rows padded by 4 floats so that the four lane groups of a
  // store land in different banks
  __shared__ __attribute__((aligned(16))) float red_o[W][NC][kHeadDim + 4];

  const int lane = threadIdx.x & (kWave - 1);
  // The wave index, in a scalar register: the compiler cannot see that it is
  // uniform, and block offsets and table lanes derived from it must be scalar.
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int n16 = lane & 15;
  const int c4 = lane >> 4;

  int item = a.plain_order ? (int)blockIdx.x : xcd_remap(blockIdx.x, gridDim.x);
  const int p = item % a.P;
  item /= a.P;
  int tg = 0;  // which NS*TC query tokens of the request this item takes
  if constexpr (kCausal) {
    tg = item % a.TG;
    item /= a.TG;
  }
  int s = item % a.S;
  int kvh = item / a.S;
  if (a.plain_order && a.order) {
    // Requests in the caller's order (longest first from paged_attn_order),
    // the KV heads of one request side by side.  An entry outside [0, S)
    // stands for its own position.
    const int r = item / a.Hkv;
    kvh = item % a.Hkv;
    const int so = a.order[r];
    s = so >= 0 && so < a.S ? so : r;
  }

  // Column n16 of set j is query token tq[j], head kvh*G + n16%G.
  int tq[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) tq[j] = (tg * NS + j) * TC + n16 / G;

  // q of each column over the dims this lane contributes, as MFMA B operands.
  bf16x8_t qv[NS][4];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    // every lane loads (no divergent loads), then columns without a query are zeroed
    const bool live = n16 < NC && tq[j] < a.T;
    const int row = kCausal ? min(tq[j], a.T - 1) : 0;
    const int hq = kCausal ? n16 % G : (n16 < G ? n16 : G - 1);
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (((int64_t)s * a.T + row) * a.Hq + (int64_t)kvh * G + hq) * kHeadDim;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 v = *reinterpret_cast<const uint4*>(qp + 32 * i + 8 * c4);
      if (!live) v = make_uint4(0, 0, 0, 0);
      qv[j][i] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // The length of the request, then (below) its first table entries and
  // first tile: the length is read with a vector (buffer) load so that it
  // is in flight together with the entries instead of waiting behind them.
  const int n_raw = __builtin_amdgcn_readfirstlane(
      (int)__builtin_amdgcn_raw_buffer_load_b32(block_rsrc(reinterpret_cast<const char*>(a.lens), (uint32_t)a.S * 4u),
                                                0, s * 4, 0));

  // Fused append ([Slides] "写满一块，再拿下一块"): the new token of request s
  // goes to logical position pos.  This lane keeps 16 bytes of its K and V
  // (dims 8*n16 .. +8 of KV head kvh), which replace the pool's row for pos
  // wherever a tile holds it, so this step never reads the slot it writes;
  // the work item whose split holds pos writes the row into the pool for
  // the steps that follow.  The result is bit for bit that of kv_append
  // followed by the decode.
  int pos = -1;
  uint4 k_in = make_uint4(0, 0, 0, 0), v_in = make_uint4(0, 0, 0, 0);
  if constexpr (kAppend) {
    pos = a.positions[s];
    const int64_t src = ((int64_t)s * a.Hkv + kvh) * kHeadDim + 8 * n16;
    k_in = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k_new) + src);
    v_in = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.v_new) + src);
  }

  // Byte offsets inside a block (a block is at most a few hundred KiB, so 32
  // bits suffice).  A load is a block descriptor (uniform, in SGPRs) plus the
  // lane's offset (slot c4 of the row group, KV head kvh, dims 8*n16) plus
  // the uniform offset of the row group's first slot.
  const int row_bytes = a.Hkv * kHeadDim * 2;
  const uint32_t blk_bytes = (uint32_t)B * (uint32_t)row_bytes;
  const uint32_t voff = (uint32_t)(c4 * row_bytes + (kvh * kHeadDim + 8 * n16) * 2);
  const char* kpool = static_cast<const char*>(a.k_pool);
  const char* vpool = static_cast<const char*>(a.v_pool);
  const int32_t* trow = a.tables + (int64_t)s * a.MB;

  // The split's tiles are dealt to the waves in turn: the k-th tile of wave
  // w is u0 + w + W*k.  Table entries are read 64 at a time into one
  // register: lane j holds entry j % E of the wave's tile kb + j / E, with
  // E = 16/B entries per tile below B = 16 (one per 4-row group's block
  // pair or quad) and one above.
  constexpr int E = B >= kTile ? 1 : kTile / B;
  constexpr int kChunk = kWave / E;  // wave tiles per register of entries
  const int u0 = p * (a.tps / kTile);
  auto wave_tile = [&](int k) { return u0 + w + W * k; };
  auto lane_entry = [&](int kb) { return (kTile * wave_tile(kb + lane / E)) / B + lane % E; };

  // Issue the 8 16-byte loads of the K and V rows of the wave's k-th tile:
  // row group i is slots 16*u + 4*i .. +3.  With B >= 16 the tile lies
  // inside one block; with B < 16 each row group has its own block.  Once
  // the length is known, a row group wholly past the history is loaded
  // through a descriptor of size 0: the hardware returns zeros for it and
  // reads no memory (its rows are masked anyway), and no table entry at or
  // past ceil(n / B) addresses the pool.  With `none` the whole tile is
  // such a load: the prefetch slot past a wave's last tile keeps the same
  // instruction count, so every wait still covers exactly the tile it
  // needs, but fetches nothing (an earlier form re-loaded the last tile
  // there, which with non-temporal loads went back to memory: 1.17x the
  // algorithmic bytes on 256 requests of 2-513 tokens, 1.05x at 1025).  A
  // speculative load (issued before the length is known) clamps a block id
  // outside the pool to block 0 without judging it: it is judged once the
  // length says whether the tile is part of the history.
  bool bad = false;
  auto pool_block = [&](int pb, bool judge) {
    if (pb < 0 || pb >= a.NB) {  // outside the pool: never dereferenced, result poisoned
      bad = bad || judge;
      pb = 0;
    }
    return pb;
  };
  int n = 0;
  auto load_tile = [&](int k, int kb, Tile& t, int tab, bool spec, bool none = false) {
    const int u = wave_tile(k);
    if constexpr (B >= kTile) {
      const int pb = pool_block(__builtin_amdgcn_readlane(tab, k - kb), !spec && !none);
      const char* kb_ptr = kpool + (int64_t)pb * blk_bytes;
      const char* vb_ptr = vpool + (int64_t)pb * blk_bytes;
      const int row0 = (kTile * u) % B;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool live = !none && (spec || kTile * u + 4 * i < n);
        t.k[i] = load_kv16<true>(block_rsrc(kb_ptr, live ? blk_bytes : 0u), voff, (row0 + 4 * i) * row_bytes);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool live = !none && (spec || kTile * u + 4 * i < n);
        t.v[i] = load_kv16<true>(block_rsrc(vb_ptr, live ? blk_bytes : 0u), voff, (row0 + 4 * i) * row_bytes);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = kTile * u + 4 * i;
        const bool live = !none && (spec || tok < n);
        const int pb = pool_block(__builtin_amdgcn_readlane(tab, (k - kb) * E + (live ? (4 * i) / B : 0)),
                                  !spec && live);
        const int soff = live ? (tok % B) * row_bytes : 0;
        const uint32_t size = live ? blk_bytes : 0u;
        t.k[i] = load_kv16<true>(block_rsrc(kpool + (int64_t)pb * blk_bytes, size), voff, soff);
        t.v[i] = load_kv16<true>(block_rsrc(vpool + (int64_t)pb * blk_bytes, size), voff, soff);
      }
    }
  };

  // The first register of entries and the wave's first tile depend only on
  // the split, not on the length: request them before the length arrives,
  // so a work item waits for two dependent reads (entries, then tile)
  // instead of three.  Entries read past the history are never used.
  Tile ring[kDepth];
  int tab = trow[min(lane_entry(0), a.MB - 1)];
  load_tile(0, 0, ring[0], tab, true);

  bad = n_raw < 0 || (int64_t)n_raw > (int64_t)a.MB * B;
  n = bad ? 0 : n_raw;
  const int nb = (n + B - 1) / B;  // blocks holding the history
  // Column n16 of set j may see the first lim[j] positions.  The item needs
  // the tiles up to its last token's limit.
  int lim[NS];
  int lim_hi = n;
#pragma unroll
  for (int j = 0; j < NS; ++j) lim[j] = n;
  if constexpr (kCausal) {
#pragma unroll
    for (int j = 0; j < NS; ++j) lim[j] = tq[j] < a.T ? min(n, max(0, n - a.T + 1 + tq[j])) : n;
    lim_hi = min(n, max(0, n - a.T + min(a.T, (tg + 1) * NS * TC)));
  }
  const int nt = (lim_hi + kTile - 1) / kTile;  // 16-slot tiles this item reads
  const int u1 = min(nt, u0 + a.tps / kTile);
  const int K = u1 > u0 + w ? (u1 - u0 - w + W - 1) / W : 0;  // this wave's tiles
  if (K > 0) {
    // judge the entries the speculative first tile used
    if constexpr (B >= kTile) {
      pool_block(__builtin_amdgcn_readlane(tab, 0), true);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (kTile * wave_tile(0) + 4 * i < n) pool_block(__builtin_amdgcn_readlane(tab, (4 * i) / B), true);
    }
  }

  if constexpr (kAppend) {
    // The work item whose split holds pos writes the new row (16 lanes of
    // wave 0, 16 bytes each of K and V); a position or block outside the
    // table or the pool is skipped, as kv_append skips it.
    const bool mine = a.P == 1 || pos / a.tps == p;
    if (mine && w == 0 && c4 == 0 && pos >= 0 && (int64_t)pos < (int64_t)a.MB * B) {
      const int blk = trow[pos / B];
      if (blk >= 0 && blk < a.NB) {
        const int64_t dst = (((int64_t)blk * B + pos % B) * a.Hkv + kvh) * kHeadDim + 8 * n16;
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(const_cast<void*>(a.k_pool)) + dst) = k_in;
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(const_cast<void*>(a.v_pool)) + dst) = v_in;
      }
    }
  }

  float m[NS];         // running max (base 2) of column n16
  float l[NS];         // partial sum over this lane's slots
  f32x4_t acc[NS][8];  // o: columns 4*c4 + r, dims 16*jj + n16
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    m[j] = kNegInf;
    l[j] = 0.f;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) acc[j][jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Writes: slot 4*i + c4, chunk n16 of this wave's tile; reads as in TileReads.
  uint8_t* vt = vt_all[w];
  uint8_t* kt = kt_all[w];
  const TileReads rd(kt, vt, n16, c4);

  auto process = [&](int u, Tile& cur) {
    const int valid = n - u * kTile;  // >= 1
    wave_lds_order();  // the previous tile's reads of this LDS come first
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * i + c4;
      *reinterpret_cast<uint4*>(kt + 256 * r + 16 * k_pos(n16, r)) = cur.k[i];
      *reinterpret_cast<uint4*>(vt + 256 * r + 16 * v_pos(n16, r)) = cur.v[i];
    }
    // V rows past the length are zeroed (their weights are 0, but 0 * NaN
    // would not be): only in the history's last tile, the same in every lane.
    if (valid < kTile) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * i + c4;
        if (r >= valid) *reinterpret_cast<uint4*>(vt + 256 * r + 16 * v_pos(n16, r)) = make_uint4(0, 0, 0, 0);
      }
    }
    if constexpr (kAppend) {
      // The token this step appends: its row of the tile holding pos (the
      // same test in every lane) is written over with the new K and V, by
      // the 16 lanes that wrote that row; V stays zero past the length.
      const int r = pos - u * kTile;
      if (r >= 0 && r < kTile) {
        if (c4 == (r & 3)) {
          *reinterpret_cast<uint4*>(kt + 256 * r + 16 * k_pos(n16, r)) = k_in;
          if (r < valid) *reinterpret_cast<uint4*>(vt + 256 * r + 16 * v_pos(n16, r)) = v_in;
        }
      }
    }
    wave_lds_order();
    // Mask past the length or, for several query tokens, past this column's
    // own position (then a column may have no valid slot yet).
    if constexpr (NS == 1) {
      tile_update<kCausal>(rd, qv[0], acc[0], m[0], l[0], kCausal ? lim[0] - u * kTile : valid, a.scale_log2, n16, c4);
    } else {
      int vq[NS];
#pragma unroll
      for (int j = 0; j < NS; ++j) vq[j] = lim[j] - u * kTile;
      tile_update_sets<NS, true>(rd, qv, acc, m, l, vq, a.scale_log2, n16, c4);
    }
  };

  // The wave's tiles are walked one register of table entries at a time.
  // Within a register kDepth tiles are in flight: tile k + kDepth - 1 is
  // loaded before tile k is processed (the load index is clamped, never
  // conditional, so the wait before each tile covers only that tile's loads).
  for (int kb = 0; kb < K; kb += kChunk) {
    const int ke = min(K, kb + kChunk);
    if (kb > 0) {
      tab = trow[min(lane_entry(kb), nb - 1)];
      load_tile(kb, kb, ring[0], tab, false);
    }
#pragma unroll
    for (int b = 1; b + 1 < kDepth; ++b) load_tile(min(kb + b, ke - 1), kb, ring[b], tab, false, kb + b >= ke);
    for (int k = kb; k < ke; k += kDepth) {
#pragma unroll
      for (int b = 0; b < kDepth; ++b) {
        const int kn = k + b + kDepth - 1;  // the tile to prefetch; past the run: a load that fetches nothing
        load_tile(min(kn, ke - 1), kb, ring[(b + kDepth - 1) % kDepth], tab, false, kn >= ke);
        __builtin_amdgcn_sched_barrier(0);  // issue the prefetch before the current tile's math
        process(wave_tile(k + b), ring[b]);
        if (k + b + 1 >= ke) break;
      }
    }
  }

  // Merge the W wave states ([Budgets] eq. (4) applied across disjoint block
  // sets): M = max m_w, L = sum 2^(m_w - M) l_w, O = sum 2^(m_w - M) o_w;
  // one column set after the other through the same LDS.  Each wave leaves
  // its m, l and unscaled o there; one barrier later every thread finishes
  // two adjacent outputs of one column.
  const float nan = __builtin_nanf("");
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    // Full l of column n16 in this wave: sum the partials of its four lanes.
    float lj = l[j];
    lj += __shfl_xor(lj, 16, kWave);
    lj += __shfl_xor(lj, 32, kWave);
    if (j > 0) __syncthreads();  // the previous set's outputs have been read
    if (c4 == 0) {
      red_m[w][n16] = m[j];
      red_l[w][n16] = lj;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hg = 4 * c4 + r;
      if (hg < NC) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) red_o[w][hg][16 * jj + n16] = acc[j][jj][r];
      }
    }
    if (j == 0) {
      bad = __syncthreads_or(bad);  // any wave that met an entry outside the pool
    } else {
      __syncthreads();
    }

    // NC * 128 outputs (column hg = query token (tg*NS + j)*TC + hg/G, head
    // kvh*G + hg%G), two adjacent dims per thread.
    for (int idx = threadIdx.x; idx < NC * (kHeadDim / 2); idx += kWave * W) {
      const int hg = idx / (kHeadDim / 2);
      const int d = 2 * (idx % (kHeadDim / 2));
      const int t_out = (tg * NS + j) * TC + hg / G;
      if (kCausal && t_out >= a.T) break;  // idx only grows: every later output is past T too
      float M = kNegInf;
#pragma unroll
      for (int v = 0; v < W; ++v) M = fmaxf(M, red_m[v][hg]);
      float L = 0.f, O0 = 0.f, O1 = 0.f;
#pragma unroll
      for (int v = 0; v < W; ++v) {
        const float mv = red_m[v][hg];
        // scale of wave v's state (0 for a wave that saw no valid slot)
        const float f = mv == kNegInf ? 0.f : fast_exp2(mv - M);
        if (mv != kNegInf) L = fmaf(f, red_l[v][hg], L);
        const float2 o = *reinterpret_cast<const float2*>(&red_o[v][hg][d]);
        O0 = fmaf(o.x, f, O0);
        O1 = fmaf(o.y, f, O1);
      }
      const int64_t row = ((int64_t)s * a.T + t_out) * a.Hq + kvh * G + hg % G;  // [S, T, Hq] row
      if (a.P == 1) {
        const float2 r = bad ? make_float2(nan, nan)
                             : (L > 0.f ? make_float2(O0 / L, O1 / L) : make_float2(0.f, 0.f));
        *reinterpret_cast<float2*>(a.out + row * kHeadDim + d) = r;
      } else {
        const int64_t slot = row * a.P + p;
        *reinterpret_cast<float2*>(a.ws_o + slot * kHeadDim + d) = make_float2(O0, O1);
        if (d == 0) {
          a.ws_m[slot] = bad ? 0.f : M;
          a.ws_l[slot] = bad ? nan : L;
        }
      }
    }
  }
}

// Workgroups of this kernel resident at once on MI355X: 256 CUs, two each
// (172-181 VGPRs per wave).
constexpr int kResidentItems = 2 * 256;

template <int G, bool kCausal, int B>
hipError_t launch_gb(const DecodeArgs& args, hipStream_t stream) {
  const int items = args.Hkv * args.S * args.P * (kCausal ? args.TG : 1);
  // Which items an XCD runs.  Grouped (xcd_remap), each XCD takes a
  // contiguous range, which is one KV head of every request; in launch order
  // the XCDs take items in turn, so every XCD sees every KV head, one head
  // after the other over the launch.  Measured on one box (non-temporal
  // loads): grouped is faster while the items fit in one round of resident
  // workgroups (32 x 4096: 82.6-86.7 vs 91.4 us; 64 x 2048: 88.5 vs 93.4 us),
  // launch order once they take more (168 x 1025 tokens: 62.5 vs 64.2 us per
  // layer; 256 requests of 1-513 tokens: 54.2 vs 56.7 us; 128 requests of
  // 1-4096 tokens: 210.9 vs 211.6 us; 128 x 1024 tokens, exactly two rounds:
  // 92.0 vs 91.8 us).
  DecodeArgs a = args;
  a.plain_order = items > kResidentItems;
  // dims->order acts only in launch order (more than one round): within one
  // round every item is resident from the start.
  if constexpr (!kCausal) {
    if (a.k_new) {
      hipLaunchKernelGGL((decode_mfma_kernel<G, false, 1, kMfmaWaves, B, true>), dim3(items),
                         dim3(kWave * kMfmaWaves), 0, stream, a);
      return hipGetLastError();
    }
  }
  if constexpr (kCausal) {
    if (decode_column_sets(PA_BF16, G, a.T) == 2) {
      hipLaunchKernelGGL((decode_mfma_kernel<G, true, 2, kMfmaWaves, B>), dim3(items), dim3(kWave * kMfmaWaves), 0,
                         stream, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((decode_mfma_kernel<G, kCausal, 1, kMfmaWaves, B>), dim3(items), dim3(kWave * kMfmaWaves), 0,
                     stream, a);
  return hipGetLastError();
}

template <bool kCausal, int B>
hipError_t launch_b(const DecodeArgs& a, int G, hipStream_t stream) {
  switch (G) {
    case 1: return launch_gb<1, kCausal, B>(a, stream);
    case 2: return launch_gb<2, kCausal, B>(a, stream);
    case 4: return launch_gb<4, kCausal, B>(a, stream);
    case 8: return launch_gb<8, kCausal, B>(a, stream);
    case 16: return launch_gb<16, kCausal, B>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool kCausal>
hipError_t launch_c(const DecodeArgs& a, int B, int G, hipStream_t stream) {
  switch (B) {
    case 4: return launch_b<kCausal, 4>(a, G, stream);
    case 8: return launch_b<kCausal, 8>(a, G, stream);
    case 16: return launch_b<kCausal, 16>(a, G, stream);
    case 32: return launch_b<kCausal, 32>(a, G, stream);
    case 64: return launch_b<kCausal, 64>(a, G, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, int B, int G, bool causal, hipStream_t stream) {
  return causal ? launch_c<true>(a, B, G, stream) : launch_c<false>(a, B, G, stream);
}

}  // namespace pa
