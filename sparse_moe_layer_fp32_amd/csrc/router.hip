// Router kernels of the MoE layer and their launchers: the logits, the
// top-k selection and the weight-plane split.  The per-tile and per-token
// bodies are in router_ops.h, shared with the fused decode kernel.

#include "router_ops.h"

namespace moe {

namespace {

// zpart[t][e][s]: grid (ceil(E/64), ceil(T/64), S) of router_tile.
__global__ __launch_bounds__(256) void router_gemm_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ wg,
                                                          float* __restrict__ zpart, int T, int H,
                                                          int E, int klen, int nsplit) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kRouterTileLds];
  router_tile(x, wg, zpart, T, H, E, klen, nsplit, blockIdx.x, blockIdx.y, blockIdx.z, smem);
}

// One wave per token (topk_wave).
template <int NS>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ zpart,
                                                   PartialLayout pl, const float* __restrict__ bias,
                                                   int T, int E,
                                                   int k, float scaling, int renorm,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  const int t = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= T) return;
  topk_wave<NS>(zpart, pl, bias, E, k, scaling, renorm, ids, w, t);
}

// Few tokens, many partials: one block per token with one thread per expert
// (64 ceil(E / 64) threads), so every logit's partials are requested at
// once.  Each wave selects its own top k (as above); wave 0 then selects
// the top k of the waves' candidates.  Every expert of the global top k is
// in its wave's top k, and the keys and scores are those of topk_kernel, so
// the two kernels give identical results.
constexpr int TKB_MAX_WAVES = kMaxExperts / 64;
constexpr int TKB_PER_LANE = TKB_MAX_WAVES * kMaxTopK / 64;  // merge candidates per lane

__global__ __launch_bounds__(1024) void topk_block_kernel(const float* __restrict__ zpart,
                                                          PartialLayout pl,
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
    z = sum_partials(zpart + t * pl.ld + e * pl.es, pl.S, pl.ps);
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
// logits: wsplit[3e + p][h] = plane p of wg[e][h] (split3), rows 3E ..
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

hipError_t launch_topk(const float* zpart, PartialLayout pl, const float* bias, int T, int E,
                       int k, float scaling, int renorm, int32_t* ids, float* w,
                       hipStream_t stream) {
  if (T < kTopkBlockTokens) {
    // Few tokens: a block per token spreads the partial sums over more CUs.
    const int threads = (E + 63) / 64 * 64;
    topk_block_kernel<<<T, threads, 0, stream>>>(zpart, pl, bias, T, E, k, scaling, renorm,
                                                 ids, w);
    return hipGetLastError();
  }
  const int blocks = (T + 3) / 4;
  const int ns = (E + 63) / 64;
  switch (ns) {
#define MOE_TOPK_CASE(N) \
  case N:                \
    topk_kernel<N><<<blocks, 256, 0, stream>>>(zpart, pl, bias, T, E, k, scaling, renorm, ids, \
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
