// Grouped SwiGLU expert GEMM kernels, the weighted combine, and their
// launchers.  The tile bodies (mainloop, epilogues, combine row) are in
// expert_tile.h, shared with the fused decode kernel.

#include "expert_tile.h"

namespace moe {

namespace {

// One unit (row tile, column tile) per block.  With e4m3 routed weights
// (WF = 1) the shared expert's bf16 tiles in the same launch take their own
// k step BK0 and ring depth S0, so that both bodies fit the LDS.
template <int MODE, int BM, int BN, int BK, int WM, int WN, int S, int WF = 0, int AV = 0,
          int BK0 = BK, int S0 = S>
__global__ __launch_bounds__(64 * WM * WN) void expert_gemm(ExpertArgs a) {
  static_assert(WF == 1 || (BK0 == BK && S0 == S), "one body without e4m3 weights");
  using C0 = Cfg<BM, BN, BK0, WM, WN, S0, 0, AV>;
  using C1 = Cfg<BM, BN, BK, WM, WN, S, WF, AV>;
  constexpr int LDS = C0::LDS_BYTES > C1::LDS_BYTES ? C0::LDS_BYTES : C1::LDS_BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS];

  const int ntiles = MODE == 2 ? static_cast<int>((a.T + BM - 1) / BM) : *a.ntiles;
  // e4m3 launches: the shared expert's units, the last of the list, keep
  // bf16 weights and stream about 1.7 times the bytes of a routed unit.
  // Dealt over the XCDs and run first, they no longer end one XCD's range
  // as its last blocks (FP8 decode -10%).
  int u;
  if constexpr (WF == 1) {
    const int nvalid = ntiles * a.NT;
    const int nsh = a.Is > 0 ? static_cast<int>((a.T + BM - 1) / BM) * a.NT : 0;
    u = xcd_remap_dealt(blockIdx.x, nvalid, min(nsh, nvalid));
  } else {
    u = xcd_remap(blockIdx.x, ntiles * a.NT);
  }
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
      gemm_tile<MODE, BM, BN, BK0, WM, WN, S0, 0, AV>(a, smem, tc, e, row0);
      return;
    }
  }
  gemm_tile<MODE, BM, BN, BK, WM, WN, S, WF, AV>(a, smem, tc, e, row0);
}

// Barrier that orders LDS accesses only (a full __syncthreads also waits
// for the wave's global stores).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Persistent form of the big tiles: one block per CU takes units (row tile,
// column tile) from its own XCD's queue, the XCD's contiguous share of the
// units in schedule order, and once that is empty from the other XCDs'
// queues, so the XCDs finish together whatever their speeds.  queue[x] is
// XCD x's counter, zero at launch; a block requests its next unit's ticket
// before starting the current tile, so the round trip overlaps the tile.
// No block waits for another.
constexpr int kRemRows = 64;  // rows of the remainder tile (persistent big-tile launches)

template <int MODE, int BM, int BN, int BK, int WM, int WN, int S, int WF, int AV>
__global__ __launch_bounds__(64 * WM * WN) void expert_gemm_persistent(ExpertArgs a,
                                                                        uint32_t* queue) {
  using C0 = Cfg<BM, BN, BK, WM, WN, S, 0, AV>;
  using C1 = Cfg<BM, BN, BK, WM, WN, S, WF, AV>;
  constexpr int LDS = C0::LDS_BYTES > C1::LDS_BYTES ? C0::LDS_BYTES : C1::LDS_BYTES;
  constexpr bool JOIN = MODE == 1;  // the staged down epilogue has barriers
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS];
  // The unit is handed to the block's waves in the LDS's last word: the last
  // weight-ring slot, which no DMA writes before the tile's first k step
  // (after the prologue barrier, by when every wave has read it), and which
  // neither epilogue uses.
  static_assert(S >= 3 && AV == 1 && LDS == C0::LDS_BYTES,
                "split ring: the LDS ends with the last bf16 B slot, free until step 0");
  static_assert(kQueueWords == 2 * kNumXcd, "a queue per XCD and GEMM");
  static_assert(BM * BN * 2 <= LDS - 4, "the staged down tile stays clear of it");
  static_assert(WM * WN == 8 && Cfg<kRemRows, BN, BK, 2, 4, 3>::LDS_BYTES <= LDS - 4,
                "the remainder tile: the same 8 waves, its ring clear of the hand-over word");
  int& s_unit = *reinterpret_cast<int*>(smem + LDS - 4);

  const int total = *a.ntiles * a.NT;
  const int per = (total + kNumXcd - 1) / kNumXcd;
  const int xcc = static_cast<int>(__builtin_amdgcn_s_getreg(kHwRegXccId)) & (kNumXcd - 1);
  auto len_of = [&](int y) { return max(0, min(per, total - y * per)); };
  auto take = [&](int y) {
    const uint32_t t =
        __hip_atomic_fetch_add(queue + y, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return t < static_cast<uint32_t>(len_of(y)) ? y * per + static_cast<int>(t) : -1;
  };
  auto steal = [&] {
    for (int j = 1; j < kNumXcd; ++j) {
      const int y = (xcc + j) & (kNumXcd - 1);
      if (__hip_atomic_load(queue + y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >=
          static_cast<uint32_t>(len_of(y)))
        continue;
      const int u = take(y);
      if (u >= 0) return u;
    }
    return -1;
  };
  if (threadIdx.x == 0) {
    const int u = take(xcc);
    s_unit = u >= 0 ? u : steal();
  }
  __syncthreads();
  int u = s_unit;
  while (u >= 0) {
    int next = -1;
    if (threadIdx.x == 0) next = take(xcc);
    const TileCoord tc = tile_of_expert<BM>(u, a.NT, a.tiles, a.offsets, a.E, a.T);
    const int2 tile = a.tiles[tc.mt];
    const bool bf = WF == 1 && tile.x == a.E;  // shared expert: bf16 weights
    // Gate/up: a tile with at most 64 rows (an expert's remainder) runs as
    // the 64-row single-ring tile over the same BN columns: the A slab it
    // streams per k step shrinks from 256 to 64 rows (the weight slab is the
    // same), and the k order, hence every result, is unchanged (prefill
    // gate/up -3.6%).  Down keeps the big tile: its short units gain nothing
    // and would lose the staged epilogue.
    const int rows = tile.x == a.E ? static_cast<int>(min<int64_t>(BM, a.T - tile.y))
                                   : min(BM, a.offsets[tile.x + 1] - tile.y);
    if (MODE == 0 && rows <= kRemRows) {
      if (bf)
        gemm_tile<MODE, kRemRows, BN, BK, 2, 4, 3, 0, 0, false>(a, smem, tc, tile.x, tile.y);
      else
        gemm_tile<MODE, kRemRows, BN, BK, 2, 4, 3, WF, 0, false>(a, smem, tc, tile.x, tile.y);
    } else if (bf) {
      gemm_tile<MODE, BM, BN, BK, WM, WN, S, 0, AV, true, JOIN>(a, smem, tc, tile.x, tile.y);
    } else {
      gemm_tile<MODE, BM, BN, BK, WM, WN, S, WF, AV, true, JOIN>(a, smem, tc, tile.x, tile.y);
    }
    // LDS-only barriers: the tile's global stores drain on their own.
    lds_barrier();  // every wave is past the tile's last LDS access
    if (threadIdx.x == 0) s_unit = next >= 0 ? next : steal();
    lds_barrier();
    u = s_unit;
  }
}

// One thread per 8 consecutive outputs (combine_row).
template <bool NT>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ o_routed,
                                                      const uint16_t* __restrict__ o_shared,
                                                      const int32_t* __restrict__ pair_pos, int k,
                                                      int64_t T, int H, int P,
                                                      uint16_t* __restrict__ y) {
  combine_row<NT>(o_routed, o_shared, pair_pos, k, T, H, P, y,
                  static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x);
}

template <int MODE, int BM, int BN, int BK, int WM, int WN, int S, int WF = 0, int AV = 0,
          int BK0 = BK, int S0 = S>
hipError_t launch_one(const ExpertArgs& a, int tile_capacity, int NT, hipStream_t stream) {
  using C = Cfg<BM, BN, BK, WM, WN, S, WF, AV>;
  const int64_t units = static_cast<int64_t>(tile_capacity) * NT;
  if (units <= 0) return hipSuccess;
  // e4m3 launches map blocks with xcd_remap_dealt: one more block per XCD
  const int64_t grid = ((units + kNumXcd - 1) / kNumXcd + (WF == 1 ? 1 : 0)) * kNumXcd;
  ExpertArgs b = a;
  b.NT = NT;
  expert_gemm<MODE, BM, BN, BK, WM, WN, S, WF, AV, BK0, S0>
      <<<static_cast<unsigned>(grid), C::THREADS, 0, stream>>>(b);
  return hipGetLastError();
}

template <int MODE, int BM, int BN, int BK, int WM, int WN, int S, int WF, int AV>
hipError_t launch_persistent(const ExpertArgs& a, int NT, uint32_t* queue, hipStream_t stream) {
  using C = Cfg<BM, BN, BK, WM, WN, S, WF, AV>;
  int dev = 0, cus = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  ExpertArgs b = a;
  b.NT = NT;
  expert_gemm_persistent<MODE, BM, BN, BK, WM, WN, S, WF, AV>
      <<<static_cast<unsigned>(std::max(cus, 1)), C::THREADS, 0, stream>>>(b, queue);
  return hipGetLastError();
}

}  // namespace

// From this many tokens on, the combine loads o with the non-temporal hint.
constexpr int64_t kCombineNtTokens = 1024;

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
// Small (few rows per expert, the GEMMs stream weights): 64 rows, one block
// per CU; gate/up 128 h columns (256 weight rows), k step 64, 8 waves, 4-deep
// ring when I and Is are multiples of 128 (else 64 h columns, k step 128, 4
// waves, 3-deep: every weight row read in 256-byte pieces); down 256 output
// columns, k step 64, 8 waves, 3-deep (128 columns and 4 waves when H is not
// a multiple of 256).  The e4m3 kernels: 64 x 256 tiles, 8 waves, k step 128
// with a 3-deep ring (each weight row piece a whole 128-byte line, which
// takes the non-temporal hint; FP8 decode -11% against k step 64), the
// shared expert's bf16 tiles in them at k step 64 with a 4-deep ring (the
// whole 160 KB of LDS); else 64 x 128 at k step 64 with a 3-deep ring.
hipError_t launch_gateup(const ExpertArgs& a, int shape, int tile_capacity, hipStream_t stream,
                         int fp8) {
  const int maxn = std::max(a.I, a.Is);
  if (fp8) {
    if (shape == kTileBig)
      return launch_persistent<0, 256, 256, 64, 2, 4, 3, 1, 1>(a, (maxn + 127) / 128, a.queue,
                                                               stream);
    if (a.I % 128 == 0 && a.Is % 128 == 0)
      return launch_one<0, 64, 256, 128, 2, 4, 3, 1, 0, 64, 4>(a, tile_capacity, maxn / 128,
                                                              stream);
    return launch_one<0, 64, 128, 64, 2, 2, 3, 1>(a, tile_capacity, (maxn + 63) / 64, stream);
  }
  if (shape == kTileBig)
    return launch_persistent<0, 256, 256, 64, 2, 4, 3, 0, 1>(a, (maxn + 127) / 128, a.queue,
                                                             stream);
  if (a.I % 128 == 0 && a.Is % 128 == 0)
    return launch_one<0, 64, 256, 64, 2, 4, 4>(a, tile_capacity, maxn / 128, stream);
  return launch_one<0, 64, 128, 128, 2, 2, 3>(a, tile_capacity, (maxn + 63) / 64, stream);
}

hipError_t launch_down(const ExpertArgs& a, int shape, int tile_capacity, hipStream_t stream,
                       int fp8) {
  if (fp8) {
    if (shape == kTileBig)
      return launch_persistent<1, 256, 256, 64, 2, 4, 3, 1, 1>(a, a.H / 256, a.queue + kNumXcd,
                                                               stream);
    if (a.H % 256 == 0 && a.I % 128 == 0 && a.Is % 128 == 0)
      return launch_one<1, 64, 256, 128, 2, 4, 3, 1, 0, 64, 4>(a, tile_capacity, a.H / 256,
                                                              stream);
    if (a.H % 256 == 0)
      return launch_one<1, 64, 256, 64, 2, 4, 4, 1>(a, tile_capacity, a.H / 256, stream);
    return launch_one<1, 64, 128, 64, 2, 2, 3, 1>(a, tile_capacity, a.H / 128, stream);
  }
  if (shape == kTileBig)
    return launch_persistent<1, 256, 256, 64, 2, 4, 3, 0, 1>(a, a.H / 256, a.queue + kNumXcd,
                                                             stream);
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
  if (T >= kCombineNtTokens)
    combine_kernel<true><<<static_cast<unsigned>(blocks), 256, 0, stream>>>(
        o_routed, o_shared, pair_pos, k, T, H, static_cast<int>(T * k), y);
  else
    combine_kernel<false><<<static_cast<unsigned>(blocks), 256, 0, stream>>>(
        o_routed, o_shared, pair_pos, k, T, H, static_cast<int>(T * k), y);
  return hipGetLastError();
}

}  // namespace moe
