// Grouped SwiGLU expert GEMM kernels, the weighted combine, and their
// launchers.  The tile bodies (mainloop, epilogues, combine row) are in
// expert_tile.h, shared with the fused decode kernel.

#include "expert_tile.h"

namespace moe {

namespace {

template <int MODE, int BM, int BN, int BK, int WM, int WN, int S, int WF = 0, int AV = 0>
__global__ __launch_bounds__(64 * WM * WN) void expert_gemm(ExpertArgs a) {
  using C0 = Cfg<BM, BN, BK, WM, WN, S, 0, AV>;
  using C1 = Cfg<BM, BN, BK, WM, WN, S, WF, AV>;
  constexpr int LDS = C0::LDS_BYTES > C1::LDS_BYTES ? C0::LDS_BYTES : C1::LDS_BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS];

  const int ntiles = MODE == 2 ? static_cast<int>((a.T + BM - 1) / BM) : *a.ntiles;
  const int u = xcd_remap(blockIdx.x, ntiles * a.NT);
  if (u < 0) return;
  const TileCoord tc = MODE == 2 ? tile_of(u, ntiles, a.NT)
                                 : tile_of_expert<BM>(u, a.NT, a.tiles, a.offsets, a.E, a.T);
  int e, row0;
  if (MODE == 2) {
    e = 0;
    row0 = tc.mt * BM;
  } else {
    const int2 tile = a.tiles[tc.mt];
    e = tile.x;
    row0 = tile.y;
  }
  if constexpr (WF == 1) {
    if (e == a.E) {  // shared expert: bf16 weights
      gemm_tile<MODE, BM, BN, BK, WM, WN, S, 0, AV>(a, smem, tc, e, row0);
      return;
    }
  }
  gemm_tile<MODE, BM, BN, BK, WM, WN, S, WF, AV>(a, smem, tc, e, row0);
}

// One thread per 8 consecutive outputs (combine_row).
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ o_routed,
                                                      const uint16_t* __restrict__ o_shared,
                                                      const int32_t* __restrict__ pair_pos, int k,
                                                      int64_t T, int H, int P,
                                                      uint16_t* __restrict__ y) {
  combine_row(o_routed, o_shared, pair_pos, k, T, H, P, y,
              static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x);
}

template <int MODE, int BM, int BN, int BK, int WM, int WN, int S, int WF = 0, int AV = 0>
hipError_t launch_one(const ExpertArgs& a, int tile_capacity, int NT, hipStream_t stream) {
  using C = Cfg<BM, BN, BK, WM, WN, S, WF, AV>;
  const int64_t units = static_cast<int64_t>(tile_capacity) * NT;
  const int64_t grid = (units + kNumXcd - 1) / kNumXcd * kNumXcd;
  if (grid <= 0) return hipSuccess;
  ExpertArgs b = a;
  b.NT = NT;
  expert_gemm<MODE, BM, BN, BK, WM, WN, S, WF, AV>
      <<<static_cast<unsigned>(grid), C::THREADS, 0, stream>>>(b);
  return hipGetLastError();
}

}  // namespace

int experts_tile_rows(int shape) { return shape == kTileBig ? 256 : 64; }

int experts_pick_shape(int64_t T, int P, int E, int H, int I, int Is) {
  // Many rows per active expert: MFMA-bound, big tiles.  Few: the GEMMs
  // stream weights, and small row tiles waste no weight bandwidth.  The big
  // tile also needs whole 128-column h tiles and 256-column output tiles.
  (void)T;
  const bool fits = H % 256 == 0 && I % 128 == 0 && Is % 128 == 0;
  return (fits && P >= 4096 && P >= 16 * std::min(E, P)) ? kTileBig : kTileSmall;
}

int experts_tile_capacity(int64_t T, int P, int E, int with_shared, int shape) {
  const int bm = experts_tile_rows(shape);
  const int64_t routed = P / bm + std::min<int64_t>(E, P);
  const int64_t sh = with_shared ? (T + bm - 1) / bm : 0;
  return static_cast<int>(routed + sh);
}

// Tile shapes.  Big (many rows per expert): 256 x 256, k step 64 (128-byte
// row pieces), 8 waves of 128 x 64 (two per SIMD, so one wave's stalls are
// covered by the other's MFMAs), split ring with A 2-deep and B 3-deep, the
// whole 160 KB of LDS (e4m3 launches too: their B stages are half the size,
// and the shared expert's bf16 tiles in them take the same ring).
// Small (few rows per expert, the GEMMs stream weights): 64 rows, 3-deep
// ring, one block per CU; gate/up 64 h columns (128 weight rows) with k step
// 128, so every weight row is read in 256-byte pieces; down 256 output
// columns, k step 64, 8 waves (128 columns and 4 waves when H is not a
// multiple of 256).  The e4m3 kernels keep 64 x 128 tiles with k step 64.
hipError_t launch_gateup(const ExpertArgs& a, int shape, int tile_capacity, hipStream_t stream,
                         int fp8) {
  const int maxn = std::max(a.I, a.Is);
  if (fp8) {
    if (shape == kTileBig)
      return launch_one<0, 256, 256, 64, 2, 4, 3, 1, 1>(a, tile_capacity, (maxn + 127) / 128,
                                                        stream);
    return launch_one<0, 64, 128, 64, 2, 2, 3, 1>(a, tile_capacity, (maxn + 63) / 64, stream);
  }
  if (shape == kTileBig)
    return launch_one<0, 256, 256, 64, 2, 4, 3, 0, 1>(a, tile_capacity, (maxn + 127) / 128,
                                                      stream);
  return launch_one<0, 64, 128, 128, 2, 2, 3>(a, tile_capacity, (maxn + 63) / 64, stream);
}

hipError_t launch_down(const ExpertArgs& a, int shape, int tile_capacity, hipStream_t stream,
                       int fp8) {
  if (fp8) {
    if (shape == kTileBig)
      return launch_one<1, 256, 256, 64, 2, 4, 3, 1, 1>(a, tile_capacity, a.H / 256, stream);
    return launch_one<1, 64, 128, 64, 2, 2, 3, 1>(a, tile_capacity, a.H / 128, stream);
  }
  if (shape == kTileBig)
    return launch_one<1, 256, 256, 64, 2, 4, 3, 0, 1>(a, tile_capacity, a.H / 256, stream);
  if (a.H % 256 == 0)
    return launch_one<1, 64, 256, 64, 2, 4, 3>(a, tile_capacity, a.H / 256, stream);
  return launch_one<1, 64, 128, 64, 2, 2, 3>(a, tile_capacity, a.H / 128, stream);
}

hipError_t launch_router_logits(const ExpertArgs& a, hipStream_t stream) {
  // Enough 256-row tiles to fill the GPU: 8 waves of 64 x 64, split ring at
  // k step 64; else 64 x 128.
  if (a.T >= 8192)
    return launch_one<2, 256, 128, 64, 4, 2, 3, 0, 1>(a, static_cast<int>((a.T + 255) / 256),
                                                     a.Np / 128, stream);
  return launch_one<2, 64, 128, 64, 2, 2, 3>(a, static_cast<int>((a.T + 63) / 64), a.Np / 128,
                                             stream);
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
