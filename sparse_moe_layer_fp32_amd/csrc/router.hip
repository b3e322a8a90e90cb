// Router of the MoE layer on gfx950: fp32 logits, sigmoid, bias used for
// selection only, top-k with ties to the lower expert index, gating weights
// renormalised over the selected experts and scaled.
//
// Follows the sglang-jax issue "[Feature] Support Step 3.5 Flash (StepFun)
// Model", "Key difficulties" item 1, and the llm-atlas Step-3.5-Flash card's
// raw config fields need_fp32_gate, moe_router_activation = sigmoid,
// use_moe_router_bias, norm_expert_weight, moe_router_scaling_factor = 3.
//
// fp32 logits on bf16 matrix cores: x is bf16, and every fp32 router weight
// w is split exactly into three bf16 terms w = hi + mid + lo (each step
// rounds the remainder to the nearest bf16; 3 x 8 significand bits cover
// fp32's 24).  Products of bf16 values are exact in fp32 and the MFMA
// accumulates in fp32, so z = x.hi + x.mid + x.lo is an fp32 dot product of
// the fp32 weights, at the bf16 MFMA rate.

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int RT_BM = 64;   // tokens per tile
constexpr int RT_BN = 64;   // experts per tile
constexpr int RT_BK = 64;   // k per step
constexpr int RT_LD = RT_BK + 8;  // padded LDS row (bf16 elements)

__device__ __forceinline__ void split3(float w, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = f32_to_bf16_bits(w);
  const float r1 = w - __uint_as_float(hi << 16);
  mid = f32_to_bf16_bits(r1);
  const float r2 = r1 - __uint_as_float(mid << 16);
  lo = f32_to_bf16_bits(r2);
}

// zpart[t][e][s] = sum over k in split s of x[t][k] * wg[e][k] (the split
// partials of one logit are contiguous, S a power of two <= 32).
// Grid: (ceil(E/64), ceil(T/64), S); 256 threads = 4 waves in a 2x2 layout,
// each wave one 32x32 output block.
__global__ __launch_bounds__(256) void router_gemm_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ wg,
                                                          float* __restrict__ zpart, int T, int H,
                                                          int E, int klen, int nsplit) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][RT_BM][RT_LD];
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][3][RT_BN][RT_LD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int n0 = blockIdx.x * RT_BN;
  const int m0 = blockIdx.y * RT_BM;
  const int s = blockIdx.z;
  const int kbeg = s * klen;
  const int ksteps = klen / RT_BK;

  // A: 64 rows x 64 bf16 = 512 16-byte chunks, 2 per thread.
  const uint16_t* aptr[2];
  bool aval[2];
  int arow[2], acol[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i;
    arow[i] = c >> 3;
    acol[i] = (c & 7) * 8;
    const int t = m0 + arow[i];
    aval[i] = t < T;
    aptr[i] = x + static_cast<int64_t>(aval[i] ? t : 0) * H + kbeg + acol[i];
  }
  // B: 64 experts x 64 fp32 = 1024 16-byte chunks, 4 per thread.
  const float* bptr[4];
  bool bval[4];
  int brow[4], bcol[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    brow[i] = c >> 4;
    bcol[i] = (c & 15) * 4;
    const int e = n0 + brow[i];
    bval[i] = e < E;
    bptr[i] = wg + static_cast<int64_t>(bval[i] ? e : 0) * H + kbeg + bcol[i];
  }

  u32x4 ra[2];
  f32x4 rb[4];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (aval[i]) v = *reinterpret_cast<const u32x4*>(aptr[i] + kt * RT_BK);
      ra[i] = v;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (bval[i]) v = *reinterpret_cast<const f32x4*>(bptr[i] + kt * RT_BK);
      rb[i] = v;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<u32x4*>(&sa[buf][arow[i]][acol[i]]) = ra[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t hi[4], mid[4], lo[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) split3(rb[i][q], hi[q], mid[q], lo[q]);
      uint2 vh = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
      uint2 vm = make_uint2(mid[0] | (mid[1] << 16), mid[2] | (mid[3] << 16));
      uint2 vl = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
      *reinterpret_cast<uint2*>(&sb[buf][0][brow[i]][bcol[i]]) = vh;
      *reinterpret_cast<uint2*>(&sb[buf][1][brow[i]][bcol[i]]) = vm;
      *reinterpret_cast<uint2*>(&sb[buf][2][brow[i]][bcol[i]]) = vl;
    }
  };

  f32x16 acc = {};
  gload(0);
  sstore(0);
  __syncthreads();
  const int fr = lane & 31;
  const int fk = (lane >> 5) * 8;
  for (int kt = 0; kt < ksteps; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ksteps) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < RT_BK / 16; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sa[buf][32 * wm + fr][16 * ks + fk]);
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        const bf16x8 b =
            *reinterpret_cast<const bf16x8*>(&sb[buf][p][32 * wn + fr][16 * ks + fk]);
        acc = mfma32(a, b, acc);
      }
    }
    if (kt + 1 < ksteps) sstore(buf ^ 1);
    __syncthreads();
  }

  const int e = n0 + 32 * wn + fr;
  if (e < E) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = m0 + 32 * wm + mfma32_row(r, lane);
      if (t < T) zpart[(static_cast<int64_t>(t) * E + e) * nsplit + s] = acc[r];
    }
  }
}

// One wave per token.  Lane l holds experts l, l+64, ...; each expert's
// logit is the sum of the split partials in split order, its score the
// fp32 sigmoid, its selection key score + bias.  Keys are packed with the
// expert index into one orderable 64-bit word, (key, 2^32-1-index), so one
// unsigned max picks the largest key and, among equal keys, the lower index.
// k rounds of a wave-wide max (DPP within rows of 16 lanes, then the four
// row results) select the experts in rank order; the winner's lane retires
// it.  Gating weights come from the bias-free scores of the selected set.
constexpr int TK_MAX_SLOTS = 16;  // E <= 1024 = 16 slots x 64 lanes

__device__ __forceinline__ uint32_t orderable(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), CTRL, 0xF,
                                             0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(static_cast<int>(v >> 32),
                                             static_cast<int>(v >> 32), CTRL, 0xF, 0xF, false);
  return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(v), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(v >> 32), lane);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Wave-wide maximum, uniform result.  Within each row of 16 lanes: swap
// neighbours, pairs, mirror halves of 8, mirror the row; then the rows.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  uint64_t o;
  o = dpp64<0xB1>(v);  v = o > v ? o : v;   // quad_perm [1,0,3,2]
  o = dpp64<0x4E>(v);  v = o > v ? o : v;   // quad_perm [2,3,0,1]
  o = dpp64<0x141>(v); v = o > v ? o : v;   // row_half_mirror
  o = dpp64<0x140>(v); v = o > v ? o : v;   // row_mirror
  const uint64_t r0 = readlane64(v, 0), r1 = readlane64(v, 16);
  const uint64_t r2 = readlane64(v, 32), r3 = readlane64(v, 48);
  const uint64_t a = r0 > r1 ? r0 : r1, b = r2 > r3 ? r2 : r3;
  return a > b ? a : b;
}

// Sum of the S partials of one logit, in order (S a power of two <= 32 for
// k splits, or 3 for the weight planes; the partials of one logit are
// contiguous).
__device__ __forceinline__ float sum_splits(const float* p, int S) {
  if (S == 1) return p[0];
  if (S == 2) {
    const float2 a = *reinterpret_cast<const float2*>(p);
    return a.x + a.y;
  }
  if (S == 3) return (p[0] + p[1]) + p[2];  // the three weight planes, hi + mid + lo
  f32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (4 * i < S) v[i] = *reinterpret_cast<const f32x4*>(p + 4 * i);
  float acc = v[0][0];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (4 * i < S)
#pragma unroll
      for (int q = (i == 0 ? 1 : 0); q < 4; ++q) acc += v[i][q];
  return acc;
}

template <int NS>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ zpart, int S,
                                                   int64_t ld, const float* __restrict__ bias,
                                                   int T, int E,
                                                   int k, float scaling, int renorm,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= T) return;

  float z[NS];
  uint64_t key[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int e = lane + 64 * i;
    z[i] = 0.f;
    key[i] = 0;  // below every real key: never selected
    if (e < E) {
      z[i] = sum_splits(zpart + static_cast<int64_t>(t) * ld + static_cast<int64_t>(e) * S, S);
      float kv = sigmoid_f32(z[i]) + (bias ? bias[e] : 0.f);
      if (kv != kv) kv = -INFINITY;  // non-finite input: rank last, stay in range
      key[i] = (static_cast<uint64_t>(orderable(kv)) << 32) |
               (0xFFFFFFFFu - static_cast<uint32_t>(e));
    }
  }

  int my_id = 0;
  float my_s = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < NS; ++i)
      if (key[i] > best) best = key[i];
    const uint64_t win = wave_max_u64(best);
    const int id = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(win));
    const int owner = id & 63, slot = id >> 6;
    float zw = 0.f;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i == slot) {
        zw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z[i]), owner));
        if (lane == owner) key[i] = 0;
      }
    }
    if (lane == j) {
      my_id = id;
      my_s = sigmoid_f32(zw);
    }
  }
  // Sum of the selected scores in slot order (lane 0 .. k-1).
  float sum = 0.f;
  for (int j = 0; j < k; ++j) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), j));
  if (lane < k) {
    const float g = renorm ? my_s / sum : my_s;
    ids[static_cast<int64_t>(t) * k + lane] = my_id;
    w[static_cast<int64_t>(t) * k + lane] = g * scaling;
  }
}

// Few tokens, many partials: one block per token with one thread per expert
// (64 ceil(E / 64) threads), so every logit's partials are requested at
// once.  Each wave selects its own top k (as above); wave 0 then selects
// the top k of the waves' candidates.  Every expert of the global top k is
// in its wave's top k, and the keys and scores are those of topk_kernel, so
// the two kernels give identical results.
constexpr int TKB_MAX_WAVES = kMaxExperts / 64;
constexpr int TKB_PER_LANE = TKB_MAX_WAVES * kMaxTopK / 64;  // merge candidates per lane

__global__ __launch_bounds__(1024) void topk_block_kernel(const float* __restrict__ zpart, int S,
                                                          int64_t ld,
                                                          const float* __restrict__ bias, int T,
                                                          int E, int k, float scaling,
                                                          int renorm, int32_t* __restrict__ ids,
                                                          float* __restrict__ w) {
  __shared__ uint64_t cand_key[TKB_MAX_WAVES][kMaxTopK];
  __shared__ float cand_z[TKB_MAX_WAVES][kMaxTopK];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwaves = blockDim.x >> 6;
  const int t = blockIdx.x;
  const int e = tid;

  float z = 0.f;
  uint64_t key = 0;
  if (e < E) {
    z = sum_splits(zpart + static_cast<int64_t>(t) * ld + static_cast<int64_t>(e) * S, S);
    float kv = sigmoid_f32(z) + (bias ? bias[e] : 0.f);
    if (kv != kv) kv = -INFINITY;
    key = (static_cast<uint64_t>(orderable(kv)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(e));
  }
  for (int j = 0; j < k; ++j) {
    const uint64_t win = wave_max_u64(key);
    float zw = 0.f;
    if (win != 0) {  // 0: this wave has no keys left
      const int owner = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(win)) & 63;
      zw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), owner));
      if (lane == owner) key = 0;
    }
    if (lane == 0) {
      cand_key[wave][j] = win;
      cand_z[wave][j] = zw;
    }
  }
  __syncthreads();
  if (wave != 0) return;

  // Lane l holds candidates l, l + 64, ... of the nwaves * k (wave-major).
  const int ncand = nwaves * k;
  uint64_t ck[TKB_PER_LANE];
  float cz[TKB_PER_LANE];
#pragma unroll
  for (int h = 0; h < TKB_PER_LANE; ++h) {
    const int c = lane + 64 * h;
    ck[h] = 0;
    cz[h] = 0.f;
    if (c < ncand) {
      ck[h] = cand_key[c / k][c % k];
      cz[h] = cand_z[c / k][c % k];
    }
  }
  int my_id = 0;
  float my_s = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int h = 0; h < TKB_PER_LANE; ++h) best = ck[h] > best ? ck[h] : best;
    const uint64_t win = wave_max_u64(best);
    const int id = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(win));
    // The holder of the winning key publishes its logit and retires it.
    float zmine = 0.f;
    bool mine = false;
#pragma unroll
    for (int h = 0; h < TKB_PER_LANE; ++h)
      if (ck[h] == win) {
        zmine = cz[h];
        ck[h] = 0;
        mine = true;
      }
    const uint64_t mask = __ballot(mine);
    const int holder = __builtin_ctzll(mask);
    const float zsel = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(zmine), holder));
    if (lane == j) {
      my_id = id;
      my_s = sigmoid_f32(zsel);
    }
  }
  float sum = 0.f;
  for (int j = 0; j < k; ++j) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), j));
  if (lane < k) {
    const float g = renorm ? my_s / sum : my_s;
    ids[static_cast<int64_t>(t) * k + lane] = my_id;
    w[static_cast<int64_t>(t) * k + lane] = g * scaling;
  }
}

// The three bf16 planes of the router weight for the GEMM form of the
// logits: wsplit[3e + p][h] = plane p of wg[e][h] (split3 above), rows 3E ..
// Np-1 zero.  One thread per 8 consecutive weights.
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ wg, int E,
                                                           int H, int Np,
                                                           uint16_t* __restrict__ wsplit) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int per_row = H / 8;
  const int64_t real = static_cast<int64_t>(E) * per_row;
  const int64_t pad = static_cast<int64_t>(Np - 3 * E) * per_row;
  if (i < real) {
    const int e = static_cast<int>(i / per_row);
    const int h = static_cast<int>(i - static_cast<int64_t>(e) * per_row) * 8;
    const f32x4 w0 = *reinterpret_cast<const f32x4*>(wg + static_cast<int64_t>(e) * H + h);
    const f32x4 w1 = *reinterpret_cast<const f32x4*>(wg + static_cast<int64_t>(e) * H + h + 4);
    uint32_t pl[3][8];
#pragma unroll
    for (int q = 0; q < 8; ++q) split3(q < 4 ? w0[q] : w1[q - 4], pl[0][q], pl[1][q], pl[2][q]);
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      u32x4 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = pl[p][2 * q] | (pl[p][2 * q + 1] << 16);
      *reinterpret_cast<u32x4*>(wsplit + static_cast<int64_t>(3 * e + p) * H + h) = v;
    }
  } else if (i < real + pad) {
    const int64_t j = i - real;
    const int n = 3 * E + static_cast<int>(j / per_row);
    const int h = static_cast<int>(j % per_row) * 8;
    *reinterpret_cast<u32x4*>(wsplit + static_cast<int64_t>(n) * H + h) = u32x4{0u, 0u, 0u, 0u};
  }
}

}  // namespace

hipError_t launch_router_gemm(const uint16_t* x, const float* wg, float* zpart, int T, int H,
                              int E, int S, hipStream_t stream) {
  const dim3 grid((E + RT_BN - 1) / RT_BN, (T + RT_BM - 1) / RT_BM, S);
  router_gemm_kernel<<<grid, 256, 0, stream>>>(x, wg, zpart, T, H, E, H / S, S);
  return hipGetLastError();
}

hipError_t launch_topk(const float* zpart, int S, int64_t ld, const float* bias, int T, int E,
                       int k, float scaling, int renorm, int32_t* ids, float* w,
                       hipStream_t stream) {
  if (T < kTopkBlockTokens) {
    // Few tokens: a block per token spreads the partial sums over more CUs.
    const int threads = (E + 63) / 64 * 64;
    topk_block_kernel<<<T, threads, 0, stream>>>(zpart, S, ld, bias, T, E, k, scaling, renorm,
                                                 ids, w);
    return hipGetLastError();
  }
  const int blocks = (T + 3) / 4;
  const int ns = (E + 63) / 64;
  switch (ns) {
#define MOE_TOPK_CASE(N) \
  case N:                \
    topk_kernel<N><<<blocks, 256, 0, stream>>>(zpart, S, ld, bias, T, E, k, scaling, renorm, ids, \
                                               w); \
    break;
    MOE_TOPK_CASE(1) MOE_TOPK_CASE(2) MOE_TOPK_CASE(3) MOE_TOPK_CASE(4) MOE_TOPK_CASE(5)
    MOE_TOPK_CASE(6) MOE_TOPK_CASE(7) MOE_TOPK_CASE(8) MOE_TOPK_CASE(9) MOE_TOPK_CASE(10)
    MOE_TOPK_CASE(11) MOE_TOPK_CASE(12) MOE_TOPK_CASE(13) MOE_TOPK_CASE(14) MOE_TOPK_CASE(15)
    MOE_TOPK_CASE(16)
#undef MOE_TOPK_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_router_split(const float* wg, int E, int H, int Np, uint16_t* wsplit,
                               hipStream_t stream) {
  const int64_t threads = static_cast<int64_t>(Np - 2 * E) * (H / 8);  // E real rows + pad
  if (threads <= 0) return hipSuccess;
  router_split_kernel<<<static_cast<unsigned>((threads + 255) / 256), 256, 0, stream>>>(
      wg, E, H, Np, wsplit);
  return hipGetLastError();
}

int router_split(int T, int H, int E) {
  // Enough blocks to stream the router weight from many CUs (a few tiles,
  // as in decoding, split k up to 32 ways), few enough partials that the
  // top-k kernel reads little.
  const int tiles = ((T + RT_BM - 1) / RT_BM) * ((E + RT_BN - 1) / RT_BN);
  const int ksteps = H / RT_BK;
  int s = 1;  // a power of two <= 32 that divides the k steps
  while (s < 32 && tiles * s < 256 && ksteps % (2 * s) == 0) s *= 2;
  return s;
}

}  // namespace moe
