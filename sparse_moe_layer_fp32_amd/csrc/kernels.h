// Host-side launchers of the MoE kernels (internal to libmoe.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace moe {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kPermuteChunk = 2048;  // pairs per rank/histogram chunk

struct GateUpArgs {
  const uint16_t* x;
  const int32_t* sorted;
  int k;
  int64_t T;
  int H;
  const uint16_t* w_gate;
  const uint16_t* w_up;
  int I;
  float limit;
  const uint16_t* ws_gate;
  const uint16_t* ws_up;
  int Is;
  float limit_shared;
  const int2* tiles;
  const int32_t* ntiles;
  const int32_t* offsets;
  int E;
  uint16_t* h_routed;  // [P][I]
  uint16_t* h_shared;  // [T][Is]
  int NT;              // 64-column tiles of max(I, Is)
};

struct DownArgs {
  const uint16_t* h_routed;
  const uint16_t* h_shared;
  const uint16_t* w_down;
  const uint16_t* ws_down;
  int H, I, Is;
  const int2* tiles;
  const int32_t* ntiles;
  const int32_t* offsets;
  int E;
  int64_t T;
  const int32_t* sorted;
  const float* topk_w;
  uint16_t* o_routed;  // [P][H]
  uint16_t* o_shared;  // [T][H]
  int NT;              // 128-column tiles of H
};

// router.hip
int router_split(int T, int H, int E);
hipError_t launch_router_gemm(const uint16_t* x, const float* wg, float* zpart, int T, int H,
                              int E, int S, hipStream_t stream);
hipError_t launch_topk(const float* zpart, int S, const float* bias, int T, int E, int k,
                       float scaling, int renorm, int32_t* ids, float* w, hipStream_t stream);

// permute.hip; ev (optional) receives three events, one before each kernel.
hipError_t launch_permute(const int32_t* ids, int P, int E, int64_t T, int bm, int with_shared,
                          int32_t* rank, int32_t* hist, int32_t* base, int32_t* offsets,
                          int32_t* sorted, int32_t* pos, int2* tiles, int32_t* ntiles,
                          hipStream_t stream, hipEvent_t* ev);

hipError_t launch_fill_zero(int32_t* p, int n, hipStream_t stream);

// experts.hip
int experts_tile_rows();
int experts_tile_capacity(int64_t T, int P, int E, int with_shared);
hipError_t launch_gateup(const GateUpArgs& a, int tile_capacity, hipStream_t stream);
hipError_t launch_down(const DownArgs& a, int tile_capacity, hipStream_t stream);
hipError_t launch_combine(const uint16_t* o_routed, const uint16_t* o_shared,
                          const int32_t* pair_pos, int k, int64_t T, int H, uint16_t* y,
                          hipStream_t stream);

}  // namespace moe
