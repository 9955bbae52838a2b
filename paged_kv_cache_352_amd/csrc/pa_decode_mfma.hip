// Paged-attention decode for bf16 K/V on the CDNA4 matrix cores.
//
// [Slides]  = "PagedAttention：让 KV cache 按需生长"
// [Budgets] = "内存预算约束下的语言模型服务：注意力、分页与调度"
//
// Same contract as the vector-ALU kernel in pa_decode.hip ([Slides]
// "分页以后，attention 仍然按完整历史归一化": look up each logical block,
// load its K/V tile, mask slots past the length, fold the block into the
// running (m, l, o) state of [Budgets] eq. (4); splits of a long history are
// merged afterwards).  What changes is where the arithmetic runs: the two
// contractions of the GQA group, q.k and p.v, are MFMA instructions, which
// leaves the vector ALU only the softmax of four scores per lane.
//
// One 64-lane wave per (request s, KV head g, split p).  Lane l is (n = l%16,
// c = l/16).  For one 16-slot block and head dim 128:
//
//   q.k  four v_mfma_f32_16x16x32_bf16 with A = the K tile (M = 16 slots,
//        K = 32 dims) and B = q of the group (N = 16 query heads, zero beyond
//        G).  Lane l loads 16 bytes of K: slot n, dims 32*i + 8*c .. +8, and
//        holds q of head n over the same dims, so the products pair up
//        whatever order the hardware sums them in.  The result leaves lane l
//        with the scores of head n for slots 4c .. 4c+3.
//   p.v  that is exactly the A layout (M = 16 heads, K = 16 slots, 4 slots
//        per lane) of v_mfma_f32_16x16x16_bf16, so the weights feed p.v
//        without crossing lanes.  The B operand needs V with slots along K;
//        V arrives slot-major, so each wave transposes its 4 KiB V tile
//        through LDS (16-bit writes, 64-bit reads).  p is split into a bf16
//        head and a bf16 remainder (p = hi + lo to about 2^-16 relative) and
//        both go through the matrix core, so p.v keeps fp32-class accuracy.
//        The eight accumulators hold o for heads 4c .. 4c+3, dims 16*j + n.
//
// Softmax state: lane l keeps m (the running max, base 2) of head n and a
// partial l over its own four slots of every block; the partials of the four
// lanes of a head are summed once at the end.  The accumulators are rescaled
// only in blocks where some head's max moved.  The next block's K and V are
// loaded before the current block is processed.
#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kWave = 64;
constexpr int kB = 16;  // block size this kernel is built for
constexpr float kNegInf = -__builtin_huge_valf();

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// V^T tile in LDS: element (dim d, slot t) at byte
//   (d / 8) * kGroupBytes + (d % 8) * 32 + 2 * t.
// Each run of 8 dims is padded by 32 bytes so that the four lane groups of a
// transposing write land in different banks.
constexpr int kGroupBytes = 8 * kB * 2 + 32;  // 288
constexpr int kVtBytes = (128 / 8) * kGroupBytes;  // 4608

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

struct Tile {
  uint4 k[4];
  uint4 v[4];
};

template <int G>
__global__ __launch_bounds__(kWave) void decode_mfma_kernel(DecodeArgs a) {
  static_assert(G >= 1 && G <= 16, "the query group must fit the 16 columns of one MFMA tile");
  __shared__ __attribute__((aligned(16))) uint8_t vt[kVtBytes];

  const int lane = threadIdx.x;
  const int n16 = lane & 15;
  const int c4 = lane >> 4;

  int item = xcd_remap(blockIdx.x, gridDim.x);
  const int p = item % a.P;
  item /= a.P;
  const int s = item % a.S;
  const int kvh = item / a.S;

  const int n_raw = a.lens[s];
  bool bad = n_raw < 0 || n_raw > a.MB * kB;
  const int n = bad ? 0 : n_raw;
  const int nb = (n + kB - 1) / kB;
  const int j0 = p * a.bps;
  const int j1 = min(nb, j0 + a.bps);

  // q of head kvh*G + n16 over the dims this lane contributes, as MFMA B operands.
  bf16x8_t qv[4];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((int64_t)s * a.Hq + (int64_t)kvh * G) * kHeadDim;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (n16 < G) w = *reinterpret_cast<const uint4*>(qp + n16 * kHeadDim + 32 * i + 8 * c4);
      qv[i] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  // Element offset of this lane's 16 bytes inside a block: slot n16, head kvh, dims 8*c4 (+32*i).
  const int64_t row_stride = (int64_t)a.Hkv * kHeadDim;
  const int64_t blk_stride = (int64_t)kB * row_stride;
  const int64_t lane_off = (int64_t)n16 * row_stride + (int64_t)kvh * kHeadDim + 8 * c4;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k_pool) + lane_off;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v_pool) + lane_off;
  const int32_t* trow = a.tables + (int64_t)s * a.MB;

  // Issue the 8 16-byte loads of the K and V tile of physical block pb.
  auto load_tile = [&](int pb, Tile& t) {
    if (pb < 0 || pb >= a.NB) {  // outside the pool: never dereferenced, result poisoned
      bad = true;
      pb = 0;
    }
    const uint16_t* kb = kbase + (int64_t)pb * blk_stride;
    const uint16_t* vb = vbase + (int64_t)pb * blk_stride;
#pragma unroll
    for (int i = 0; i < 4; ++i) t.k[i] = *reinterpret_cast<const uint4*>(kb + 32 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) t.v[i] = *reinterpret_cast<const uint4*>(vb + 32 * i);
  };

  float m = kNegInf;  // running max (base 2) of head n16
  float l = 0.f;      // partial sum over this lane's slots
  f32x4_t acc[8];     // o: heads 4*c4 + r, dims 16*jj + n16
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) acc[jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // LDS addresses: transposing writes (slot n16, dims 32*i + 8*c4 + e) and
  // B-operand reads (slots 4*c4 .. +3, dim 16*jj + n16).
  uint8_t* vt_w = vt + 2 * n16;
  const uint8_t* vt_r = vt + (n16 >> 3) * kGroupBytes + (n16 & 7) * 32 + 8 * c4;

  auto process = [&](int j, Tile& cur) {
    // q.k for the 16 slots of block j.
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, cur.k[i]), qv[i], sc, 0, 0, 0);

    // Transpose V into LDS; slots past the length become zeros so that their
    // (possibly NaN) contents never meet a zero weight.
    const int valid = n - j * kB;  // >= 1
    if (valid < kB && n16 >= valid) {
#pragma unroll
      for (int i = 0; i < 4; ++i) cur.v[i] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint8_t* w = vt_w + (4 * i + c4) * kGroupBytes;
      const uint32_t d[4] = {cur.v[i].x, cur.v[i].y, cur.v[i].z, cur.v[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        *reinterpret_cast<uint16_t*>(w + (2 * e) * 32) = (uint16_t)(d[e] & 0xffffu);
        *reinterpret_cast<uint16_t*>(w + (2 * e + 1) * 32) = (uint16_t)(d[e] >> 16);
      }
    }

    // Scores in base 2, masked past the length ([Slides] quiz "逻辑顺序没错…").
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[r] = (4 * c4 + r < valid) ? sc[r] * a.scale_log2 : kNegInf;

    // [Budgets] eq. (4): block max over the 16 slots of head n16, new running max.
    float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    bm = fmaxf(bm, __shfl_xor(bm, 16, kWave));
    bm = fmaxf(bm, __shfl_xor(bm, 32, kWave));
    const float mn = fmaxf(m, bm);  // finite: slot 0 of a block below nb is valid
    const float alpha = fast_exp2(m - mn);
    m = mn;
    float pw[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pw[r] = fast_exp2(sv[r] - mn);
    l = fmaf(l, alpha, (pw[0] + pw[1]) + (pw[2] + pw[3]));

    uint32_t hi0, hi1, lo0, lo1;
    split_pair(pw[0], pw[1], hi0, lo0);
    split_pair(pw[2], pw[3], hi1, lo1);
    const s16x4_t phi = __builtin_bit_cast(s16x4_t, make_uint2(hi0, hi1));
    const s16x4_t plo = __builtin_bit_cast(s16x4_t, make_uint2(lo0, lo1));

    // Rescale o only where a head's max moved (alpha < 1 somewhere in the wave).
    if (__any(alpha != 1.f)) {
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * c4 + r, kWave);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[jj][r] *= ar[r];
    }

    __syncthreads();  // the transposed tile is visible to every lane
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const s16x4_t vb = *reinterpret_cast<const s16x4_t*>(vt_r + 2 * jj * kGroupBytes);
      acc[jj] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, vb, acc[jj], 0, 0, 0);
      acc[jj] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, vb, acc[jj], 0, 0, 0);
    }
    __syncthreads();  // reads done before the next block overwrites the tile
  };

  // The split is walked in chunks of up to 64 blocks.  One vector load
  // brings a chunk's table entries into a register, one per lane; block j's
  // entry is then read out of lane j - jb.  Within a chunk two tiles are in
  // flight: block j+1 loads while block j is processed (the load index is
  // clamped, never conditional, so the wait before each tile covers only that
  // tile's loads).
  for (int jb = j0; jb < j1; jb += kWave) {
    const int je = min(j1, jb + kWave);
    const int tab = (jb + lane < je) ? trow[jb + lane] : 0;
    Tile t0, t1;
    load_tile(__builtin_amdgcn_readlane(tab, 0), t0);
    for (int j = jb; j < je; j += 2) {
      load_tile(__builtin_amdgcn_readlane(tab, min(j + 1, je - 1) - jb), t1);
      process(j, t0);
      if (j + 1 >= je) break;
      load_tile(__builtin_amdgcn_readlane(tab, min(j + 2, je - 1) - jb), t0);
      process(j + 1, t1);
    }
  }

  // Full l of head n16: sum the partials of the four lanes holding that head.
  l += __shfl_xor(l, 16, kWave);
  l += __shfl_xor(l, 32, kWave);

  const float nan = __builtin_nanf("");
  if (a.P == 1) {
    // out = o / l for the heads this lane's accumulators hold.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hg = 4 * c4 + r;
      const float lh = __shfl(l, hg & 15, kWave);
      if (hg >= G) continue;
      const float inv = lh > 0.f ? 1.f / lh : 0.f;
      float* dst = a.out + ((int64_t)s * a.Hq + kvh * G + hg) * kHeadDim + n16;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) dst[16 * jj] = bad ? nan : acc[jj][r] * inv;
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hg = 4 * c4 + r;
      if (hg >= G) continue;
      const int64_t slot = ((int64_t)s * a.Hq + kvh * G + hg) * a.P + p;
      float* dst = a.ws_o + slot * kHeadDim + n16;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) dst[16 * jj] = acc[jj][r];
    }
    if (c4 == 0 && n16 < G) {
      const int64_t slot = ((int64_t)s * a.Hq + kvh * G + n16) * a.P + p;
      a.ws_m[slot] = bad ? 0.f : m;
      a.ws_l[slot] = bad ? nan : l;
    }
  }
}

template <int G>
hipError_t launch_g(const DecodeArgs& a, hipStream_t stream) {
  const int items = a.Hkv * a.S * a.P;
  hipLaunchKernelGGL((decode_mfma_kernel<G>), dim3(items), dim3(kWave), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, int G, hipStream_t stream) {
  switch (G) {
    case 1: return launch_g<1>(a, stream);
    case 2: return launch_g<2>(a, stream);
    case 4: return launch_g<4>(a, stream);
    case 8: return launch_g<8>(a, stream);
    case 16: return launch_g<16>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
