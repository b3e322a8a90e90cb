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
// Mainloop (one template for both GEMMs and both tile shapes):
//  * bf16 x bf16 -> fp32 on v_mfma_f32_32x32x16_bf16; every operand is
//    k-contiguous in memory (weights are out x in), so A and B fragments are
//    plain 16-byte LDS reads.
//  * Tiles are copied HBM -> LDS with global_load_lds_dwordx4 (no VGPR
//    staging): one wave instruction fills 8 rows x 128 bytes; rows are
//    gathered per lane, so the token gather of the gate/up GEMM costs
//    nothing extra.  The 16-byte chunks of a row are XOR-swizzled by
//    (row & 7), which keeps the fragment reads free of bank conflicts.
//  * An S-stage ring: stage kt+S-1 is in flight while stage kt is
//    multiplied; per-wave `s_waitcnt vmcnt` plus a bare s_barrier order the
//    ring (no full fence, which would drain the prefetches).
//  * Work comes from a device-side tile list (no host synchronisation); units
//    are spread over the 8 XCDs in contiguous ranges and walked in groups of
//    8 row tiles so that co-resident blocks share operands in their L2.
//
// Two tile shapes: 256 x 256 (one block per CU, 4 waves of 128 x 128) for
// many rows per expert, and 64 x 128 with a 3-deep ring (two blocks per CU) for few rows per
// expert, where the GEMMs stream weights at HBM rate.

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

constexpr int BK = 64;        // k per stage: one 128-byte row segment
constexpr int GROUP_M = 8;    // row tiles per scheduling group

__device__ __forceinline__ void dma16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((gbl_void*)src, (lds_void*)lds_wave_base, 16, 0, 0);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

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

template <int BM, int BN, int WM, int WN, int S>
struct Cfg {
  static constexpr int NW = WM * WN;
  static constexpr int THREADS = 64 * NW;
  static constexpr int MB = BM / WM / 32;   // 32-row blocks per wave
  static constexpr int NB = BN / WN / 32;   // 32-col blocks per wave
  static constexpr int JA = BM / 8 / NW;    // A DMA instructions per wave per stage
  static constexpr int JB = BN / 8 / NW;    // B DMA instructions per wave per stage
  static constexpr int STAGE_BYTES = (BM + BN) * 128;
  static constexpr int LDS_BYTES = S * STAGE_BYTES;
  static_assert(MB >= 1 && NB >= 1 && JA >= 1 && JB >= 1, "tile shape");
  static_assert(JA + JB <= 63 / (S > 2 ? S - 2 : 1), "vmcnt budget");
};

// MODE 0: gate/up (+ SwiGLU), MODE 1: down (+ gating weight).
template <int MODE, int BM, int BN, int WM, int WN, int S>
__global__ __launch_bounds__(64 * WM * WN) void expert_gemm(ExpertArgs a) {
  using C = Cfg<BM, BN, WM, WN, S>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS_BYTES];

  const int ntiles = *a.ntiles;
  const int u = xcd_remap(blockIdx.x, gridDim.x, ntiles * a.NT);
  if (u < 0) return;
  const TileCoord tc = tile_of(u, ntiles, a.NT);
  const int2 tile = a.tiles[tc.mt];
  const int e = tile.x, row0 = tile.y;
  const bool shared = e == a.E;
  const int H = a.H;

  // Problem shape of this group.
  int K, N;  // reduction length, output columns (h cols or d cols)
  if (MODE == 0) {
    K = H;
    N = shared ? a.Is : a.I;
  } else {
    K = shared ? a.Is : a.I;
    N = H;
  }
  const int n0 = tc.nt * (MODE == 0 ? BN / 2 : BN);  // first output column
  if (n0 >= N) return;
  const int rows = shared ? static_cast<int>(min<int64_t>(BM, a.T - row0))
                          : min(BM, a.offsets[e + 1] - row0);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform

  // ---- DMA source pointers.  Instruction j of wave w fills tile rows
  // [8 (w*J + j), +8); lane l writes row 8(w*J + j) + l/8, physical chunk
  // l % 8, which holds logical chunk (l % 8) ^ (row & 7).
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ lrow;  // logical chunk; every DMA row r has r & 7 == lrow
  // A rows: element offsets from the A base (x, or h), gathered per row.
  const uint16_t* abase;
  if (MODE == 0)
    abase = a.x;
  else
    abase = shared ? a.h_shared : a.h_routed;
  uint32_t aoff[C::JA];
  bool aon[C::JA];  // lanes of rows past the group's end load nothing (lane 0
                    // re-reads row 0, so every DMA instruction is issued)
#pragma unroll
  for (int j = 0; j < C::JA; ++j) {
    const int r = 8 * (wid * C::JA + j) + lrow;
    aon[j] = r < rows || lane == 0;
    const int rr = r < rows ? r : 0;
    int64_t src_row;
    if (MODE == 0) {
      src_row = shared ? static_cast<int64_t>(row0 + rr) : a.sorted[row0 + rr] / a.k;
      src_row = min<int64_t>(max<int64_t>(src_row, 0), a.T - 1);
    } else {
      src_row = row0 + rr;
    }
    aoff[j] = static_cast<uint32_t>(src_row * K + lchunk * 8);
  }
  // B rows: each wave's rows are consecutive and lie in one matrix (for
  // gate/up the first half of the tile is W_gate, the second W_up).
  const uint16_t* bsrc;
  {
    const int r0 = 8 * wid * C::JB;  // first B row of this wave
    const uint16_t* mat;
    int mrow;
    if (MODE == 0) {
      const bool up = r0 >= BN / 2;
      mat = up ? (shared ? a.ws_up : a.w_up + static_cast<int64_t>(e) * a.I * H)
               : (shared ? a.ws_gate : a.w_gate + static_cast<int64_t>(e) * a.I * H);
      mrow = n0 + r0 - (up ? BN / 2 : 0);
    } else {
      mat = shared ? a.ws_down : a.w_down + static_cast<int64_t>(e) * H * a.I;
      mrow = n0 + r0;
    }
    bsrc = mat + static_cast<int64_t>(mrow + lrow) * K + lchunk * 8;
  }

  auto issue = [&](int kt) {
    uint8_t* st = smem + (kt % S) * C::STAGE_BYTES;
    const int k0 = kt * BK;
#pragma unroll
    for (int j = 0; j < C::JA; ++j)
      if (aon[j]) dma16(abase + aoff[j] + k0, st + (wid * C::JA + j) * 1024);
#pragma unroll
    for (int j = 0; j < C::JB; ++j)
      dma16(bsrc + static_cast<int64_t>(8 * j) * K + k0,
            st + BM * 128 + (wid * C::JB + j) * 1024);
  };

  // ---- fragment addressing.  Wave (wm, wn) owns rows [wm*BM/WM, +BM/WM).
  const int wm = wid / WN, wn = wid % WN;
  const int fr = lane & 31;
  const int fh = lane >> 5;
  // Byte offset of (row, logical chunk c) inside a stage: row*128 + ((c ^ (row&7)) * 16);
  // fr & 7 == row & 7 for every fragment row since blocks start at multiples of 32.
  int a_off[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) a_off[mb] = (wm * (BM / WM) + 32 * mb + fr) * 128;
  int b_off[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    int brow;
    if (MODE == 0) {
      // blocks 0..NB/2-1 are gate, NB/2.. the matching up blocks
      const int half = C::NB / 2;
      const int hcol = wn * (BN / 2 / WN) + 32 * (nb % half);
      brow = (nb < half ? 0 : BN / 2) + hcol;
    } else {
      brow = wn * (BN / WN) + 32 * nb;
    }
    b_off[nb] = BM * 128 + (brow + fr) * 128;
  }
  const int KT = K / BK;
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < KT) issue(s);

  // The ring protocol, shared by waves that multiply and waves whose rows
  // all lie past the group's end (those only keep the barriers and DMAs).
  auto ring_step = [&](int kt) {
    if (kt + S - 2 < KT)
      wait_vmcnt<(S - 2) * (C::JA + C::JB)>();
    else
      wait_vmcnt<0>();
    // Bare barrier: orders the ring without draining the prefetches (the
    // "memory" clobber keeps the compiler from moving LDS accesses across).
    asm volatile("s_barrier" ::: "memory");
    if (kt + S - 1 < KT) issue(kt + S - 1);
  };

  if (wm * (BM / WM) >= rows) {
    for (int kt = 0; kt < KT; ++kt) ring_step(kt);
    return;
  }

  f32x16 acc[C::MB][C::NB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) acc[mb][nb] = f32x16{};

  for (int kt = 0; kt < KT; ++kt) {
    ring_step(kt);
    // Fragments of k-substep ks+1 are read while the MFMAs of ks run; the
    // scheduling barriers keep at most two fragment sets live.
    const uint8_t* st = smem + (kt % S) * C::STAGE_BYTES;
    bf16x8 af[2][C::MB], bf[2][C::NB];
    auto load_frags = [&](int ks, int set) {
      const int sw = ((2 * ks + fh) ^ (fr & 7)) * 16;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
        bf[set][nb] = *reinterpret_cast<const bf16x8*>(st + b_off[nb] + sw);
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
        af[set][mb] = *reinterpret_cast<const bf16x8*>(st + a_off[mb] + sw);
    };
    load_frags(0, 0);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if (ks + 1 < BK / 16) load_frags(ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
          acc[mb][nb] = mfma32(af[ks & 1][mb], bf[ks & 1][nb], acc[mb][nb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- epilogue
  if (MODE == 0) {
    uint16_t* out = shared ? a.h_shared : a.h_routed;
    const float lim = shared ? a.limit_shared : a.limit;
    const int half = C::NB / 2;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
#pragma unroll
      for (int nb = 0; nb < half; ++nb) {
        const int col = n0 + wn * (BN / 2 / WN) + 32 * nb + fr;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * (BM / WM) + 32 * mb + mfma32_row(r, lane);
          if (row < rows) {
            const float hv = swiglu_f32(acc[mb][nb][r], acc[mb][nb + half][r], lim);
            out[static_cast<int64_t>(row0 + row) * N + col] =
                static_cast<uint16_t>(f32_to_bf16_bits(hv));
          }
        }
      }
    }
  } else {
    uint16_t* out = shared ? a.o_shared : a.o_routed;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * (BM / WM) + 32 * mb + mfma32_row(r, lane);
        if (row < rows) {
          const float wt = shared ? 1.0f : a.topk_w[a.sorted[row0 + row]];
          uint16_t* orow = out + static_cast<int64_t>(row0 + row) * H + n0 + wn * (BN / WN) + fr;
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb)
            orow[32 * nb] = static_cast<uint16_t>(f32_to_bf16_bits(acc[mb][nb][r] * wt));
        }
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

// Tile shapes.
using BigTile = Cfg<256, 256, 2, 2, 2>;
using SmallTile = Cfg<64, 128, 2, 2, 3>;

template <int MODE, int BM, int BN, int WM, int WN, int S>
hipError_t launch_one(const ExpertArgs& a, int tile_capacity, int NT, hipStream_t stream) {
  using C = Cfg<BM, BN, WM, WN, S>;
  const int64_t units = static_cast<int64_t>(tile_capacity) * NT;
  const int64_t grid = (units + kNumXcd - 1) / kNumXcd * kNumXcd;
  if (grid <= 0) return hipSuccess;
  ExpertArgs b = a;
  b.NT = NT;
  expert_gemm<MODE, BM, BN, WM, WN, S><<<static_cast<unsigned>(grid), C::THREADS, 0, stream>>>(b);
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

hipError_t launch_gateup(const ExpertArgs& a, int shape, int tile_capacity, hipStream_t stream) {
  const int maxn = std::max(a.I, a.Is);
  if (shape == kTileBig) {
    return launch_one<0, 256, 256, 2, 2, 2>(a, tile_capacity, (maxn + 127) / 128, stream);
  }
  return launch_one<0, 64, 128, 2, 2, 3>(a, tile_capacity, (maxn + 63) / 64, stream);
}

hipError_t launch_down(const ExpertArgs& a, int shape, int tile_capacity, hipStream_t stream) {
  if (shape == kTileBig) {
    return launch_one<1, 256, 256, 2, 2, 2>(a, tile_capacity, a.H / 256, stream);
  }
  return launch_one<1, 64, 128, 2, 2, 3>(a, tile_capacity, a.H / 128, stream);
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
