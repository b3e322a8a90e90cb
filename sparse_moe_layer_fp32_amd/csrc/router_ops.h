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

#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int RT_BM = 64;   // tokens per tile
constexpr int RT_BN = 64;   // experts per tile
constexpr int RT_BK = 64;   // k per step
constexpr int RT_LD = RT_BK + 8;  // padded LDS row (bf16 elements)
constexpr int kRouterTileSaBytes = 2 * RT_BM * RT_LD * 2;
constexpr int kRouterTileLds = kRouterTileSaBytes + 2 * 3 * RT_BN * RT_LD * 2;

__device__ __forceinline__ void split3(float w, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = f32_to_bf16_bits(w);
  const float r1 = w - __uint_as_float(hi << 16);
  mid = f32_to_bf16_bits(r1);
  const float r2 = r1 - __uint_as_float(mid << 16);
  lo = f32_to_bf16_bits(r2);
}

// zpart[s][t][e] = sum over k in split s of x[t][k] * wg[e][k] (one
// contiguous [T][E] plane per split, S a power of two <= 32).
// One 64 x 64 tile (experts bx, tokens by) of split s; 256 threads = 4 waves
// in a 2x2 layout, each wave one 32x32 output block; smem holds
// kRouterTileLds bytes (two stages of x and of the three weight planes).
__device__ __forceinline__ void router_tile(const uint16_t* __restrict__ x,
                                            const float* __restrict__ wg,
                                            float* __restrict__ zpart, int T, int H, int E,
                                            int klen, int nsplit, int bx, int by, int s,
                                            uint8_t* smem) {
  auto sa = reinterpret_cast<uint16_t(*)[RT_BM][RT_LD]>(smem);
  auto sb = reinterpret_cast<uint16_t(*)[3][RT_BN][RT_LD]>(smem + kRouterTileSaBytes);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int n0 = bx * RT_BN;
  const int m0 = by * RT_BM;
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
      if (t < T) zpart[(static_cast<int64_t>(s) * T + t) * E + e] = acc[r];
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

// Sum of the S <= 32 partials of one logit in order, p0 + p1 + ... (k
// splits, or the three weight planes hi + mid + lo); partial i is at p[i ps].
__device__ __forceinline__ float sum_partials(const float* p, int S, int64_t ps) {
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i)
    if (i < S) {
      v[i] = *p;
      p += ps;
    }
  float acc = v[0];
#pragma unroll
  for (int i = 1; i < 32; ++i)
    if (i < S) acc += v[i];
  return acc;
}

// Top-k of token t by the calling wave (see above).
template <int NS>
__device__ __forceinline__ void topk_wave(const float* __restrict__ zpart, PartialLayout pl,
                                          const float* __restrict__ bias, int E, int k,
                                          float scaling, int renorm, int32_t* __restrict__ ids,
                                          float* __restrict__ w, int t) {
  const int lane = threadIdx.x & 63;
  float z[NS];
  uint64_t key[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int e = lane + 64 * i;
    z[i] = 0.f;
    key[i] = 0;  // below every real key: never selected
    if (e < E) {
      z[i] = sum_partials(zpart + t * pl.ld + e * pl.es, pl.S, pl.ps);
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

// topk_wave with the logits and keys in LDS instead of registers, for any
// E <= kMaxExperts at run time: zl and kl hold this wave's kMaxExperts
// logits and keys.  The partials are read two slots at a time (bounded
// registers).  Keys, scores, the selection and the sums are those of
// topk_wave, so the results are identical.
__device__ __forceinline__ void topk_wave_lds(const float* __restrict__ zpart, PartialLayout pl,
                                              const float* __restrict__ bias, int E, int k,
                                              float scaling, int renorm,
                                              int32_t* __restrict__ ids, float* __restrict__ w,
                                              int t, float* zl, uint64_t* kl) {
  const int lane = threadIdx.x & 63;
  const int ns = (E + 63) / 64;
  for (int i0 = 0; i0 < ns; i0 += 2) {
    float z[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = lane + 64 * (i0 + j);
      z[j] = 0.f;
      if (e < E)
        z[j] = sum_partials(zpart + t * pl.ld + e * pl.es, pl.S, pl.ps);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = lane + 64 * (i0 + j);
      if (i0 + j < ns) {
        uint64_t key = 0;  // below every real key: never selected
        if (e < E) {
          float kv = sigmoid_f32(z[j]) + (bias ? bias[e] : 0.f);
          if (kv != kv) kv = -INFINITY;
          key = (static_cast<uint64_t>(orderable(kv)) << 32) |
                (0xFFFFFFFFu - static_cast<uint32_t>(e));
        }
        zl[e] = z[j];
        kl[e] = key;
      }
    }
  }
  int my_id = 0;
  float my_s = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
    for (int i = 0; i < ns; ++i) {
      const uint64_t v = kl[lane + 64 * i];
      best = v > best ? v : best;
    }
    const uint64_t win = wave_max_u64(best);
    const int id = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(win));
    const float zw = zl[id];
    if (lane == (id & 63)) kl[id] = 0;
    if (lane == j) {
      my_id = id;
      my_s = sigmoid_f32(zw);
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

}  // namespace

}  // namespace moe
