// Paged-attention decode: one query token per request, exact softmax
// attention over the request's history, read through its block table.
//
// [Slides]  = "PagedAttention：让 KV cache 按需生长"
// [Budgets] = "内存预算约束下的语言模型服务：注意力、分页与调度"
//
// What is computed ([Slides] "分页以后，attention 仍然按完整历史归一化"): for
// each logical block of the request, look up its physical block, load the
// K/V tile, mask slots at or past the length, score, and fold the block into
// a running (m, l, o) state with the update of [Budgets] eq. (4).  Long
// histories are cut into contiguous ranges of logical blocks ("splits"); each
// range is reduced to its own (m, l, o), and the states are merged
// ([Slides] quiz "逻辑顺序没错…": mergeable state, not averaged softmaxes):
// by the waves of one workgroup through LDS for groups of up to 4 splits
// (float32), and by a second kernel across groups and for the matrix-core
// kernels' splits.
//
// This file holds the float32 path (bf16 K/V go to the matrix-core kernel in
// pa_decode_mfma.hip) and the split merge both paths share.
//
// Mapping to CDNA4 (vector ALU):
//   * one 64-lane wave per work item (request s, KV head g, split p); the G
//     query heads of the GQA group share every K/V byte the wave loads; the
//     waves of up to 4 consecutive splits form one workgroup and merge their
//     states in LDS, so a request cut into at most 4 splits needs no second
//     kernel and more splits leave a quarter as many partial states;
//   * a K or V tile of one (block, KV head) is B rows of d contiguous
//     elements, rows Hkv*d apart.  Lane (r, c) loads 16 bytes — dims
//     [c*E, c*E+E) of row i*RPL + r — so a wave instruction reads RPL whole
//     rows, each as one contiguous run;
//   * q.k partial sums are reduced across the LPR lanes of a row with
//     cross-lane shuffles; the running max is reduced across rows;
//   * scores are kept in base 2 (scale*log2(e) folded into q) so every
//     exponential is a single v_exp_f32;
//   * work items are numbered KV-head-major and handed out XCD by XCD, so
//     the waves that read one KV head's blocks (a shared prefix, say) sit on
//     the same L2.
//
// Several query tokens per request (the causal variant): T new tokens,
// already the last T positions of the history, token i attending positions
// 0 .. n-T+i ([Serving] §5: speculative verification and prompt chunks read
// the same paged history).  A wave then keeps C = 8 (token, head) columns —
// 8/G tokens of its group — each with its own length limit; a column that
// has seen no valid position yet keeps the empty state (m = -inf, l = 0,
// o = 0).  Further tokens go to further work items.
#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kWave = 64;
constexpr float kNegInf = -__builtin_huge_valf();

// A 16-byte K/V load; kStream marks it non-temporal (each byte is read once
// per decode step: one query token, one work item per split of the history).
// The several-token form leaves it to the caches, since its token groups
// read the same history.
typedef unsigned int u32x4_native __attribute__((ext_vector_type(4)));

template <bool kStream>
__device__ inline uint4 load_row16(const void* p) {
  if constexpr (kStream) {
    const u32x4_native v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_native*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  }
  return *reinterpret_cast<const uint4*>(p);
}

template <typename T>
struct Vec16;  // how a 16-byte load unpacks into float32

template <>
struct Vec16<float> {
  static constexpr int kElems = 4;
  __device__ static inline void unpack(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
};

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, kWave); }

// Workgroups are dispatched to the 8 XCDs round-robin; renumber them so that
// consecutive logical work items share an XCD (and its L2).
__device__ inline int xcd_remap(int bid, int nwg) {
  const int x = bid % kNumXcd, k = bid / kNumXcd;
  const int q = nwg / kNumXcd, rem = nwg % kNumXcd;
  return x * q + min(x, rem) + k;
}

// W waves per workgroup, one split each; their W states are merged through
// LDS at the end.
template <typename T, int G, bool kCausal, int B, int W>
__global__ __launch_bounds__(kWave * W) void decode_split_kernel(DecodeArgs a) {
  constexpr int TC = kCausal ? (G >= 8 ? 1 : 8 / G) : 1;  // query tokens per work item
  constexpr int C = G * TC;                                // (token, head) columns
  constexpr int E = Vec16<T>::kElems;  // elements per 16-byte load
  constexpr int LPR = kHeadDim / E;    // lanes per row (32 for fp32)
  constexpr int RPL = kWave / LPR;     // rows per wave load (2 for fp32)
  constexpr int kTile = 16;            // slots processed per step
  constexpr int NL = kTile / RPL;      // loads per tile (8 for fp32)
  static_assert(B % RPL == 0, "block size must be a multiple of the rows one wave load covers");

  const int lane = threadIdx.x % kWave;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int c = lane % LPR;
  const int r = lane / LPR;

  // The workgroup takes group pg of W consecutive splits (a.P groups per
  // request, KV head and token group); its wave w runs split pg*W + w.
  int item = xcd_remap(blockIdx.x, gridDim.x);
  const int pg = item % a.P;
  const int p = pg * W + w;
  item /= a.P;
  int tg = 0;  // which TC query tokens of the request this item takes
  if constexpr (kCausal) {
    tg = item % a.TG;
    item /= a.TG;
  }
  const int s = item % a.S;
  const int kvh = item / a.S;

  const int n_raw = a.lens[s];
  bool bad = n_raw < 0 || (int64_t)n_raw > (int64_t)a.MB * B;  // outside what the table can describe
  const int n = bad ? 0 : n_raw;
  // Column g is query token tg*TC + g/G, head kvh*G + g%G; it may see the
  // first lim[g] positions.  The item needs the tiles up to its last token's.
  int lim[C];
  int lim_hi = n;
#pragma unroll
  for (int g = 0; g < C; ++g) lim[g] = n;
  if constexpr (kCausal) {
#pragma unroll
    for (int g = 0; g < C; ++g) {
      const int tq = tg * TC + g / G;
      lim[g] = tq < a.T ? min(n, max(0, n - a.T + 1 + tq)) : n;
    }
    lim_hi = min(n, max(0, n - a.T + min(a.T, tg * TC + TC)));
  }
  const int nt = (lim_hi + kTile - 1) / kTile;  // 16-slot tiles this item reads
  const int u0 = p * (a.tps / kTile);
  const int u1 = min(nt, u0 + a.tps / kTile);

  // q of the C columns, dims [c*E, c*E+E), pre-scaled into base 2.
  float qf[C][E];
  {
#pragma unroll
    for (int g = 0; g < C; ++g) {
      const int row = kCausal ? min(tg * TC + g / G, a.T - 1) : 0;  // a column past T repeats the last token
      const T* qp = static_cast<const T*>(a.q) +
                    (((int64_t)s * a.T + row) * a.Hq + (int64_t)kvh * G + g % G) * kHeadDim + c * E;
      const uint4 w = *reinterpret_cast<const uint4*>(qp);
      Vec16<T>::unpack(w, qf[g]);
#pragma unroll
      for (int e = 0; e < E; ++e) qf[g][e] *= a.scale_log2;
    }
  }

  float m[C], l[C], o[C][E];
#pragma unroll
  for (int g = 0; g < C; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[g][e] = 0.f;
  }

  const int64_t row_stride = (int64_t)a.Hkv * kHeadDim;  // elements between slots
  const int64_t blk_stride = (int64_t)B * row_stride;     // elements between blocks
  const int64_t lane_off = (int64_t)kvh * kHeadDim + c * E;
  const T* kbase = static_cast<const T*>(a.k_pool) + lane_off;
  const T* vbase = static_cast<const T*>(a.v_pool) + lane_off;
  const int32_t* trow = a.tables + (int64_t)s * a.MB;

  for (int u = u0; u < u1; ++u) {
    // Row pair i of tile u is slots 16*u + RPL*i + (0 .. RPL-1); B is a
    // multiple of RPL, so a pair lies in one block.  A pair past the history
    // reads the history's last block instead (masked below), so no table
    // entry at or past ceil(n / B) is read.
    uint4 kraw[NL], vraw[NL];
    auto pool_block = [&](int pb) {
      if (pb < 0 || pb >= a.NB) {  // a table entry outside the pool: poison, never dereference
        bad = true;
        pb = 0;
      }
      return pb;
    };
    if constexpr (B >= kTile) {  // the whole tile lies in one block: one table read
      const int pb = pool_block(trow[(kTile * u) / B]);
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int64_t off = (int64_t)pb * blk_stride + (int64_t)((kTile * u) % B + RPL * i + r) * row_stride;
        kraw[i] = load_row16<!kCausal>(kbase + off);
        vraw[i] = load_row16<!kCausal>(vbase + off);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int tok = kTile * u + RPL * i;
        const bool live = tok < n;
        const int pb = pool_block(trow[(live ? tok : n - 1) / B]);
        const int64_t off = (int64_t)pb * blk_stride + (int64_t)((live ? tok % B : 0) + r) * row_stride;
        kraw[i] = load_row16<!kCausal>(kbase + off);
        vraw[i] = load_row16<!kCausal>(vbase + off);
      }
    }

    // Scores of this lane's NL slots for the C columns (base 2).
    float sc[NL][C];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      float kf[E];
      Vec16<T>::unpack(kraw[i], kf);
#pragma unroll
      for (int g = 0; g < C; ++g) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc = fmaf(qf[g][e], kf[e], acc);
        sc[i][g] = acc;
      }
    }
#pragma unroll
    for (int mask = 1; mask < LPR; mask <<= 1)
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int g = 0; g < C; ++g) sc[i][g] += shfl_xor(sc[i][g], mask);

    // Mask slots at or past the length ([Slides] quiz "逻辑顺序没错…" step 1),
    // and, for several query tokens, past each column's own position.
    const bool tail = (u + 1) * kTile > n;
    bool valid[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int slot = kTile * u + i * RPL + r;
      valid[i] = slot < n;
#pragma unroll
      for (int g = 0; g < C; ++g) sc[i][g] = slot < lim[g] ? sc[i][g] : kNegInf;
    }

    // [Budgets] eq. (4): new running max, rescale factor, block weights.
#pragma unroll
    for (int g = 0; g < C; ++g) {
      float bm = sc[0][g];
#pragma unroll
      for (int i = 1; i < NL; ++i) bm = fmaxf(bm, sc[i][g]);
#pragma unroll
      for (int mask = LPR; mask < kWave; mask <<= 1) bm = fmaxf(bm, shfl_xor(bm, mask));
      const float mn = fmaxf(m[g], bm);  // decode: finite, slot 0 of tile u < nt is valid
      float alpha, mref = mn;
      if constexpr (kCausal) {
        // a column may have seen nothing yet (mn = -inf): keep its empty state
        alpha = (m[g] == mn) ? 1.f : fast_exp2(m[g] - mn);
        mref = (mn == kNegInf) ? 0.f : mn;
      } else {
        alpha = fast_exp2(m[g] - mn);
      }
      m[g] = mn;
      l[g] *= alpha;
#pragma unroll
      for (int e = 0; e < E; ++e) o[g][e] *= alpha;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int slot = kTile * u + i * RPL + r;
        const float pw = slot < lim[g] ? fast_exp2(sc[i][g] - mref) : 0.f;
        sc[i][g] = pw;
        l[g] += pw;
      }
    }

    // o += p * v over this lane's slots; unwritten slots never enter (0*NaN = NaN).
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      float vf[E];
      Vec16<T>::unpack(vraw[i], vf);
      if (tail && !valid[i]) {
#pragma unroll
        for (int e = 0; e < E; ++e) vf[e] = 0.f;
      }
#pragma unroll
      for (int g = 0; g < C; ++g)
#pragma unroll
        for (int e = 0; e < E; ++e) o[g][e] = fmaf(sc[i][g], vf[e], o[g][e]);
    }
  }

  // Rows hold disjoint slot subsets under the same running max: sum them.
#pragma unroll
  for (int mask = LPR; mask < kWave; mask <<= 1) {
#pragma unroll
    for (int g = 0; g < C; ++g) {
      l[g] += shfl_xor(l[g], mask);
#pragma unroll
      for (int e = 0; e < E; ++e) o[g][e] += shfl_xor(o[g][e], mask);
    }
  }

  // Merge the W split states ([Budgets] eq. (4) across disjoint block sets,
  // in split order): M = max m_w, L = sum 2^(m_w - M) l_w,
  // O = sum 2^(m_w - M) o_w.  A wave whose split holds no tile keeps m = -inf
  // and drops out; with one group of splits the result is the output, else
  // the group's partial state for the merge kernel.
  __shared__ float red_m[W][C];
  __shared__ float red_l[W][C];
  __shared__ float red_o[W][C][kHeadDim];
  if (r == 0) {
#pragma unroll
    for (int g = 0; g < C; ++g) {
#pragma unroll
      for (int e = 0; e < E; ++e) red_o[w][g][c * E + e] = o[g][e];
      if (c == 0) {
        red_m[w][g] = m[g];
        red_l[w][g] = l[g];
      }
    }
  }
  bad = __syncthreads_or(bad);  // any wave that met an entry outside the pool

  const float nan = __builtin_nanf("");
  for (int idx = threadIdx.x; idx < C * kHeadDim; idx += kWave * W) {
    const int g = idx / kHeadDim;
    const int d = idx % kHeadDim;
    const int t_out = tg * TC + g / G;
    if (kCausal && t_out >= a.T) break;  // idx only grows: every later column is past T too
    float M = kNegInf;
#pragma unroll
    for (int v = 0; v < W; ++v) M = fmaxf(M, red_m[v][g]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int v = 0; v < W; ++v) {
      const float mv = red_m[v][g];
      const float f = mv == kNegInf ? 0.f : fast_exp2(mv - M);
      L = fmaf(f, red_l[v][g], L);
      O = fmaf(f, red_o[v][g][d], O);
    }
    const int64_t row = ((int64_t)s * a.T + t_out) * a.Hq + kvh * G + g % G;  // [S, T, Hq] row
    if (a.P == 1) {
      a.out[row * kHeadDim + d] = bad ? nan : (L > 0.f ? O / L : 0.f);
    } else {
      const int64_t slot = row * a.P + pg;
      a.ws_o[slot * kHeadDim + d] = O;
      if (d == 0) {
        a.ws_m[slot] = bad ? 0.f : M;
        a.ws_l[slot] = bad ? nan : L;
      }
    }
  }
}

// Merge of the split states of one (request, query token, head) per half
// wave:
//   M = max_p m_p, L = sum_p 2^(m_p - M) l_p, O = sum_p 2^(m_p - M) o_p, out = O / L.
// Empty splits carry m = -inf, l = 0 and drop out; all empty gives 0.  Each
// lane takes four consecutive dims (16-byte loads and stores), a workgroup
// of four waves takes kMergeRows rows.  With kP > 0 (exactly kP splits)
// every load of the row is issued before the first is used, so a row costs
// one trip to memory instead of one per split; kP = 0 takes any count.  The
// arithmetic is the same in both forms, in split order.
constexpr int kMergeRows = 8;
template <int kP>
__global__ __launch_bounds__(kWave * 4) void decode_merge_kernel(DecodeArgs a) {
  const int64_t rows = (int64_t)a.S * a.T * a.Hq;
  const int64_t sh = (int64_t)blockIdx.x * kMergeRows + (threadIdx.x >> 5);  // (s * T + t) * Hq + h
  if (sh >= rows) return;
  const int lane = threadIdx.x & 31;
  const int P = kP > 0 ? kP : a.P;
  const float* ms = a.ws_m + sh * P;
  const float* ls = a.ws_l + sh * P;
  const float4* os = reinterpret_cast<const float4*>(a.ws_o + sh * P * kHeadDim) + lane;
  float4* dst = reinterpret_cast<float4*>(a.out + sh * kHeadDim) + lane;
  float M = kNegInf, L = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  auto fold = [&](float w, float lp, const float4& v) {
    L = fmaf(w, lp, L);
    o.x = fmaf(w, v.x, o.x);
    o.y = fmaf(w, v.y, o.y);
    o.z = fmaf(w, v.z, o.z);
    o.w = fmaf(w, v.w, o.w);
  };
  if constexpr (kP > 0) {
    float mv[kP], lv[kP];
    float4 ov[kP];
#pragma unroll
    for (int p = 0; p < kP; ++p) {
      mv[p] = ms[p];
      lv[p] = ls[p];
      ov[p] = os[p * (kHeadDim / 4)];
    }
#pragma unroll
    for (int p = 0; p < kP; ++p) M = fmaxf(M, mv[p]);
    if (M == kNegInf) {
      *dst = make_float4(0.f, 0.f, 0.f, 0.f);
      return;
    }
#pragma unroll
    for (int p = 0; p < kP; ++p) fold(fast_exp2(mv[p] - M), lv[p], ov[p]);
  } else {
#pragma unroll 8
    for (int p = 0; p < P; ++p) M = fmaxf(M, ms[p]);
    if (M == kNegInf) {
      *dst = make_float4(0.f, 0.f, 0.f, 0.f);
      return;
    }
#pragma unroll 4
    for (int p = 0; p < P; ++p) fold(fast_exp2(ms[p] - M), ls[p], os[p * (kHeadDim / 4)]);
  }
  const float inv = 1.f / L;
  *dst = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
}

template <typename T, int G, bool kCausal, int B>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  const int items = a.Hkv * a.S * a.P * (kCausal ? a.TG : 1);
  switch (a.W) {
    case 1: hipLaunchKernelGGL((decode_split_kernel<T, G, kCausal, B, 1>), dim3(items), dim3(kWave), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<T, G, kCausal, B, 2>), dim3(items), dim3(kWave * 2), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_split_kernel<T, G, kCausal, B, 4>), dim3(items), dim3(kWave * 4), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, bool kCausal, int B>
hipError_t launch_group(const DecodeArgs& a, int G, hipStream_t stream) {
  switch (G) {
    case 1: return launch_typed<T, 1, kCausal, B>(a, stream);
    case 2: return launch_typed<T, 2, kCausal, B>(a, stream);
    case 4: return launch_typed<T, 4, kCausal, B>(a, stream);
    case 8: return launch_typed<T, 8, kCausal, B>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool kCausal>
hipError_t launch_valu(const DecodeArgs& a, int B, int G, hipStream_t stream) {
  switch (B) {
    case 4: return launch_group<float, kCausal, 4>(a, G, stream);
    case 8: return launch_group<float, kCausal, 8>(a, G, stream);
    case 16: return launch_group<float, kCausal, 16>(a, G, stream);
    case 32: return launch_group<float, kCausal, 32>(a, G, stream);
    case 64: return launch_group<float, kCausal, 64>(a, G, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t decode_workspace_floats(int64_t rows, int P) { return (size_t)rows * P * (kHeadDim + 2); }

hipError_t launch_decode(const DecodeArgs& a, pa_dtype dtype, int B, int G, hipStream_t stream) {
  // bf16: q.k and p.v on the matrix cores; fp32: the vector-ALU kernel.
  const bool causal = a.T > 1;
  hipError_t e;
  if (use_shared_tile(dtype, G, a.T)) {
    e = launch_extend_shared(a, B, G, stream);
    if (shared_tile_parts(dtype, G, a.T, a.P) > 1) return e;  // the splits merged in the kernel
  } else if (dtype == PA_BF16)
    e = launch_decode_mfma(a, B, G, causal, stream);
  else
    e = causal ? launch_valu<true>(a, B, G, stream) : launch_valu<false>(a, B, G, stream);
  if (e != hipSuccess || a.P == 1) return e;
  if (!a.ws_o || !a.ws_m || !a.ws_l) return hipErrorInvalidValue;  // a merge reads the split workspace
  const int64_t rows = (int64_t)a.S * a.T * a.Hq;
  const dim3 grid((unsigned)((rows + kMergeRows - 1) / kMergeRows)), block(kWave * 4);
  switch (a.P) {
    case 2: hipLaunchKernelGGL(decode_merge_kernel<2>, grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL(decode_merge_kernel<3>, grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL(decode_merge_kernel<4>, grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL(decode_merge_kernel<0>, grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace pa
