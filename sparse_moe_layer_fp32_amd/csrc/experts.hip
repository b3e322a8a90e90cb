// Grouped SwiGLU expert GEMMs of the MoE layer on gfx950 matrix cores.
//
// Each routed expert is a SwiGLU MLP H -> I -> H (sglang-jax issue
// "[Feature] Support Step 3.5 Flash (StepFun) Model", "Model configuration"
// and "Reuse map": SiLU-and-mul with an elementwise clamp branch; llm-atlas
// Step-3.5-Flash card, raw fields moe_intermediate_size 1280 and
// share_expert_dim 1280).  The pairs were sorted by expert, so expert e owns
// rows [offsets[e], offsets[e+1]) of the sorted order; the shared expert is
// one more group whose rows are the tokens themselves.
//
// gate/up: h[r] = SiLU(min(g, L)) * clamp(u, -L, L) with g = W_gate[e] x_r,
//          u = W_up[e] x_r (no clamp when L <= 0); x rows are gathered by
//          token from the sorted pairs; h is stored bf16 in sorted order.
// down:    o[r] = w_r * (W_down[e] h[r]), bf16, sorted order; w_r is the
//          pair's gating weight (1 for the shared expert).
//
// Both are bf16 x bf16 -> fp32 MFMA (v_mfma_f32_32x32x16_bf16) GEMMs over a
// device-side tile list (no host synchronisation): 128-row tiles, 64-deep
// k steps double-buffered through LDS, 4 waves each owning a 64 x 64 block.
// Work units are spread over the XCDs in contiguous ranges and walked in
// groups of 8 row tiles so that co-resident blocks share weight and
// activation tiles in their XCD's L2.

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int BM = 128;      // rows (pairs or tokens) per tile
constexpr int BN = 128;      // B rows per tile
constexpr int BK = 64;       // k per step
constexpr int LD = BK + 8;   // padded LDS row, bf16 elements (144 B)
constexpr int GROUP_M = 8;   // row tiles per scheduling group

struct TileCoord {
  int mt, nt;
};

__device__ __forceinline__ TileCoord tile_of(int u, int ntiles, int NT) {
  const int group = u / (GROUP_M * NT);
  const int first = group * GROUP_M;
  const int gm = min(GROUP_M, ntiles - first);
  const int within = u - group * GROUP_M * NT;
  return {first + within % gm, within / gm};
}

__global__ __launch_bounds__(256) void gateup_kernel(GateUpArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][BM][LD];
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][BN][LD];

  const int ntiles = *a.ntiles;
  const int u = xcd_remap(blockIdx.x, gridDim.x, ntiles * a.NT);
  if (u < 0) return;
  const TileCoord tc = tile_of(u, ntiles, a.NT);
  const int2 tile = a.tiles[tc.mt];
  const int e = tile.x, row0 = tile.y;
  const bool shared = e == a.E;
  const int N = shared ? a.Is : a.I;
  const int i0 = tc.nt * 64;
  if (i0 >= N) return;
  const int rows = shared ? static_cast<int>(min<int64_t>(BM, a.T - row0))
                          : min(BM, a.offsets[e + 1] - row0);
  const int H = a.H;
  const uint16_t* bg = shared ? a.ws_gate : a.w_gate + static_cast<int64_t>(e) * a.I * H;
  const uint16_t* bu = shared ? a.ws_up : a.w_up + static_cast<int64_t>(e) * a.I * H;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int lrow = tid >> 3;
  const int lcol = (tid & 7) * 8;

  const uint16_t* ap[4];
  bool av[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = lrow + 32 * i;
    av[i] = r < rows;
    int64_t token = 0;
    if (av[i]) token = shared ? static_cast<int64_t>(row0 + r) : a.sorted[row0 + r] / a.k;
    token = min<int64_t>(max<int64_t>(token, 0), a.T - 1);  // stays inside x whatever the list holds
    ap[i] = a.x + token * H + lcol;
  }
  const uint16_t* bp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = lrow + 32 * i;
    bp[i] = (r < 64 ? bg + static_cast<int64_t>(i0 + r) * H
                    : bu + static_cast<int64_t>(i0 + r - 64) * H) + lcol;
  }

  u32x4 ra[4], rb[4];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (av[i]) v = *reinterpret_cast<const u32x4*>(ap[i] + k0);
      ra[i] = v;
      rb[i] = *reinterpret_cast<const u32x4*>(bp[i] + k0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(&sa[buf][lrow + 32 * i][lcol]) = ra[i];
      *reinterpret_cast<u32x4*>(&sb[buf][lrow + 32 * i][lcol]) = rb[i];
    }
  };

  const int wm = wid >> 1, wn = wid & 1;
  const int fr = lane & 31;
  const int fk = (lane >> 5) * 8;
  const bool on0 = 64 * wm < rows;
  const bool on1 = 64 * wm + 32 < rows;
  f32x16 accg[2] = {}, accu[2] = {};

  const int ksteps = H / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < ksteps; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ksteps) gload(kt + 1);
    if (on0) {
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int kk = 16 * ks + fk;
        const bf16x8 g = *reinterpret_cast<const bf16x8*>(&sb[buf][32 * wn + fr][kk]);
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(&sb[buf][64 + 32 * wn + fr][kk]);
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&sa[buf][64 * wm + fr][kk]);
        accg[0] = mfma32(a0, g, accg[0]);
        accu[0] = mfma32(a0, v, accu[0]);
        if (on1) {
          const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&sa[buf][64 * wm + 32 + fr][kk]);
          accg[1] = mfma32(a1, g, accg[1]);
          accu[1] = mfma32(a1, v, accu[1]);
        }
      }
    }
    if (kt + 1 < ksteps) sstore(buf ^ 1);
    __syncthreads();
  }

  uint16_t* out = shared ? a.h_shared : a.h_routed;
  const float lim = shared ? a.limit_shared : a.limit;
  const int col = i0 + 32 * wn + fr;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 64 * wm + 32 * mb + mfma32_row(r, lane);
      if (row < rows) {
        const float hv = swiglu_f32(accg[mb][r], accu[mb][r], lim);
        out[static_cast<int64_t>(row0 + row) * N + col] = static_cast<uint16_t>(f32_to_bf16_bits(hv));
      }
    }
  }
}

__global__ __launch_bounds__(256) void down_kernel(DownArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[2][BM][LD];
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][BN][LD];

  const int ntiles = *a.ntiles;
  const int u = xcd_remap(blockIdx.x, gridDim.x, ntiles * a.NT);
  if (u < 0) return;
  const TileCoord tc = tile_of(u, ntiles, a.NT);
  const int2 tile = a.tiles[tc.mt];
  const int e = tile.x, row0 = tile.y;
  const bool shared = e == a.E;
  const int K = shared ? a.Is : a.I;
  const int d0 = tc.nt * BN;
  const int rows = shared ? static_cast<int>(min<int64_t>(BM, a.T - row0))
                          : min(BM, a.offsets[e + 1] - row0);
  const int H = a.H;
  const uint16_t* hsrc = shared ? a.h_shared : a.h_routed;
  const uint16_t* wb = shared ? a.ws_down : a.w_down + static_cast<int64_t>(e) * H * a.I;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int lrow = tid >> 3;
  const int lcol = (tid & 7) * 8;

  const uint16_t* ap[4];
  bool av[4];
  const uint16_t* bp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = lrow + 32 * i;
    av[i] = r < rows;
    ap[i] = hsrc + static_cast<int64_t>(row0 + (av[i] ? r : 0)) * K + lcol;
    bp[i] = wb + static_cast<int64_t>(d0 + r) * K + lcol;
  }

  u32x4 ra[4], rb[4];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (av[i]) v = *reinterpret_cast<const u32x4*>(ap[i] + k0);
      ra[i] = v;
      rb[i] = *reinterpret_cast<const u32x4*>(bp[i] + k0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4*>(&sa[buf][lrow + 32 * i][lcol]) = ra[i];
      *reinterpret_cast<u32x4*>(&sb[buf][lrow + 32 * i][lcol]) = rb[i];
    }
  };

  const int wm = wid >> 1, wn = wid & 1;
  const int fr = lane & 31;
  const int fk = (lane >> 5) * 8;
  const bool on0 = 64 * wm < rows;
  const bool on1 = 64 * wm + 32 < rows;
  f32x16 acc[2][2] = {};

  const int ksteps = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < ksteps; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ksteps) gload(kt + 1);
    if (on0) {
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int kk = 16 * ks + fk;
        const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(&sb[buf][64 * wn + fr][kk]);
        const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(&sb[buf][64 * wn + 32 + fr][kk]);
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&sa[buf][64 * wm + fr][kk]);
        acc[0][0] = mfma32(a0, b0, acc[0][0]);
        acc[0][1] = mfma32(a0, b1, acc[0][1]);
        if (on1) {
          const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&sa[buf][64 * wm + 32 + fr][kk]);
          acc[1][0] = mfma32(a1, b0, acc[1][0]);
          acc[1][1] = mfma32(a1, b1, acc[1][1]);
        }
      }
    }
    if (kt + 1 < ksteps) sstore(buf ^ 1);
    __syncthreads();
  }

  uint16_t* out = shared ? a.o_shared : a.o_routed;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 64 * wm + 32 * mb + mfma32_row(r, lane);
      if (row < rows) {
        const float wt = shared ? 1.0f : a.topk_w[a.sorted[row0 + row]];
        uint16_t* orow = out + static_cast<int64_t>(row0 + row) * H + d0 + 64 * wn + fr;
        orow[0] = static_cast<uint16_t>(f32_to_bf16_bits(acc[mb][0][r] * wt));
        orow[32] = static_cast<uint16_t>(f32_to_bf16_bits(acc[mb][1][r] * wt));
      }
    }
  }
}

// y[t] = o_shared[t] + sum_j o[pos(t, j)] in slot order j = 0..k-1, fp32,
// rounded once to bf16.  One thread per 8 consecutive outputs.
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ o_routed,
                                                      const uint16_t* __restrict__ o_shared,
                                                      const int32_t* __restrict__ pair_pos, int k,
                                                      int64_t T, int H, int P,
                                                      uint16_t* __restrict__ y) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int per_row = H / 8;
  const int64_t t = idx / per_row;
  if (t >= T) return;
  const int d = static_cast<int>(idx - t * per_row) * 8;
  float acc[8];
  if (o_shared) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(o_shared + t * H + d);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] = bf16_lo(v[q]);
      acc[2 * q + 1] = bf16_hi(v[q]);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  }
  for (int j = 0; j < k; ++j) {
    const int64_t pos = min(max(pair_pos[t * k + j], 0), P - 1);
    const u32x4 v = *reinterpret_cast<const u32x4*>(o_routed + pos * H + d);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] += bf16_lo(v[q]);
      acc[2 * q + 1] += bf16_hi(v[q]);
    }
  }
  u32x4 outv;
#pragma unroll
  for (int q = 0; q < 4; ++q) outv[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
  *reinterpret_cast<u32x4*>(y + t * H + d) = outv;
}

}  // namespace

int experts_tile_rows() { return BM; }

int experts_tile_capacity(int64_t T, int P, int E, int with_shared) {
  const int64_t routed = P / BM + std::min<int64_t>(E, P);
  const int64_t sh = with_shared ? (T + BM - 1) / BM : 0;
  return static_cast<int>(routed + sh);
}

hipError_t launch_gateup(const GateUpArgs& a, int tile_capacity, hipStream_t stream) {
  const int64_t units = static_cast<int64_t>(tile_capacity) * a.NT;
  const int64_t grid = (units + kNumXcd - 1) / kNumXcd * kNumXcd;
  if (grid <= 0) return hipSuccess;
  gateup_kernel<<<static_cast<unsigned>(grid), 256, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_down(const DownArgs& a, int tile_capacity, hipStream_t stream) {
  const int64_t units = static_cast<int64_t>(tile_capacity) * a.NT;
  const int64_t grid = (units + kNumXcd - 1) / kNumXcd * kNumXcd;
  if (grid <= 0) return hipSuccess;
  down_kernel<<<static_cast<unsigned>(grid), 256, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_combine(const uint16_t* o_routed, const uint16_t* o_shared,
                          const int32_t* pair_pos, int k, int64_t T, int H, uint16_t* y,
                          hipStream_t stream) {
  const int64_t threads = T * (H / 8);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks <= 0) return hipSuccess;
  combine_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(
      o_routed, o_shared, pair_pos, k, T, H, static_cast<int>(T * k), y);
  return hipGetLastError();
}

}  // namespace moe
