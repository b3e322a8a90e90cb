// Host-side launchers of the MoE kernels (internal to libmoe.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace moe {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kTopkBlockTokens = 2048;  // below: one top-k block per token
// Queue counters of the persistent big-tile GEMMs: one per XCD for gate/up,
// then one per XCD for down; the tile-list writer zeroes them.
constexpr int kQueueWords = 16;

// Where the router's partial logits live: partial s of logit (t, e) is
// zpart[t ld + e es + s ps], summed over s = 0 .. S-1 in order.
struct PartialLayout {
  int S;
  int64_t ld, es, ps;
};

// Arguments of the grouped expert GEMMs (gate/up and down share them).
struct ExpertArgs {
  const uint16_t* x;        // [T][H]
  const int32_t* sorted;    // [P] pair ids in expert order
  const float* w_sorted;    // [P] gating weights in expert order (w_sorted[i] = w[sorted[i]])
  int k;
  int64_t T;
  int H, I, Is, E;
  const uint16_t* w_gate;   // [E][I][H]
  const uint16_t* w_up;     // [E][I][H]
  const uint16_t* w_down;   // [E][H][I]
  const uint16_t* ws_gate;  // [Is][H]
  const uint16_t* ws_up;    // [Is][H]
  const uint16_t* ws_down;  // [H][Is]
  float limit, limit_shared;
  const int2* tiles;        // (group, first row) per row tile; group E = shared
  const int32_t* ntiles;    // number of valid tiles
  const int32_t* offsets;   // [E+1]
  uint16_t* h_routed;       // [P][I]
  uint16_t* h_shared;       // [T][Is]
  uint16_t* o_routed;       // [P][H]
  uint16_t* o_shared;       // [T][H]
  int NT;                   // column tiles (set by the launcher)
  uint32_t* queue;          // kQueueWords work-queue counters (persistent big tiles)
  // FP8 routed experts (when the launch says so): e4m3 codes in the layouts of
  // w_gate/w_up/w_down and one fp32 scale per output row.
  const uint8_t* w8_gate;   // [E][I][H]
  const uint8_t* w8_up;     // [E][I][H]
  const uint8_t* w8_down;   // [E][H][I]
  const float* s_gate;      // [E][I]
  const float* s_up;        // [E][I]
  const float* s_down;      // [E][H]
  // Router logits as a GEMM (mode 2): zout[t][n] = x[t] . wsplit[n], n < Np.
  const uint16_t* wsplit;   // [Np][H] bf16 planes of the router weight, row 3e+p
  float* zout;              // [T][Np]
  int Np;                   // rows of wsplit (a multiple of the column tile)
};

// Single-launch forward for small batches (fused.hip).  Control words live
// in the workspace: words [0, kCtlReset) are zero before a launch and the
// last block to finish sets them back to zero; kCtlStatus collects the
// flags of waits that ran out (sticky).
constexpr int kFusedMaxTokens = 256;
constexpr int kFusedMaxPairs = 2048;
constexpr int kFusedMaxRoutedTiles = kFusedMaxPairs / 64 + kMaxExperts;
constexpr int kFusedMaxSharedTiles = kFusedMaxTokens / 64;
enum FusedCtl : int {
  kCtlTicket = 0,        // one ticket counter per phase (8)
  kCtlRouterDone = 8,    // router tiles finished
  kCtlTopkDone = 9,      // top-k units finished
  kCtlPermDone = 10,     // permutation published (0 / 1)
  kCtlDownDone = 11,     // down tiles finished (shared and routed)
  kCtlExit = 12,         // blocks finished
  kCtlNtiles = 13,       // routed row tiles (valid once kCtlPermDone is set)
  kCtlSharedGu = 16,     // per shared row tile: gate/up tiles finished
  kCtlTileGu = kCtlSharedGu + kFusedMaxSharedTiles,  // per routed row tile: the same
  kCtlReset = kCtlTileGu + kFusedMaxRoutedTiles,
  kCtlStatus = kCtlReset,
  kCtlWords = (kCtlReset + 1 + 63) / 64 * 64,
};
// kCtlStatus bits: which wait gave up.
enum FusedStatus : uint32_t {
  kStRouter = 1, kStTopk = 2, kStPerm = 4, kStSharedGu = 8, kStGu = 16, kStDown = 32,
};

constexpr int kTileBig = 0;    // 256 x 256 tiles
constexpr int kTileSmall = 1;  // 64-row tiles

// Arguments of the single-launch forward: the expert GEMMs' arguments plus
// the router's, the buffers the permutation writes and the control words.
struct FusedArgs {
  ExpertArgs g;
  const float* wg;      // [E][H]
  const float* bias;    // [E] or null
  float* zpart;         // [T][E][S] router partial logits
  int S;                // router k splits
  PartialLayout pl;     // where the partials live
  float scaling;
  int renorm;
  int32_t* ids;         // [T][k]
  float* w;             // [T][k]
  int32_t* offsets;     // [E+1]     (g.offsets, writable)
  int32_t* sorted;      // [P]       (g.sorted)
  float* w_sorted;      // [P]       (g.w_sorted)
  int32_t* pos;         // [P]
  int2* tiles;          // routed row tiles of 64 rows
  int tile_cap;         // capacity of tiles
  uint16_t* y;          // [T][H]
  uint32_t* ctl;        // kCtlWords control words
};
hipError_t launch_fused(const FusedArgs& f, hipStream_t stream);

// router.hip
int router_split(int T, int H, int E);
// Router logits as one bf16 GEMM over the weight's three bf16 planes (from
// this many tokens on): zpart[t][3e + p] with row stride Np.
constexpr int kRouterGemmTokens = 1024;
constexpr int kRouterGemmTileN = 128;  // column tile of that GEMM
hipError_t launch_router_split(const float* wg, int E, int H, int Np, uint16_t* wsplit,
                               hipStream_t stream);
hipError_t launch_router_logits(const ExpertArgs& a, hipStream_t stream);
hipError_t launch_router_gemm(const uint16_t* x, const float* wg, float* zpart, int T, int H,
                              int E, int S, hipStream_t stream);
hipError_t launch_topk(const float* zpart, PartialLayout pl, const float* bias, int T, int E,
                       int k, float scaling, int renorm, int32_t* ids, float* w,
                       hipStream_t stream);

// permute.hip; ev (optional) receives three events, one before each kernel.
// queue (may be null): kQueueWords counters zeroed with the tile list.
hipError_t launch_permute(const int32_t* ids, int P, int E, int64_t T, int bm, int with_shared,
                          int32_t* rank, int32_t* hist, int32_t* base, int32_t* offsets,
                          int32_t* sorted, int32_t* pos, int2* tiles, int32_t* ntiles,
                          uint32_t* queue, const float* topk_w, float* w_sorted,
                          hipStream_t stream, hipEvent_t* ev);

hipError_t launch_fill_zero(int32_t* p, int n, hipStream_t stream);
hipError_t launch_dense_tiles(int2* tiles, int32_t* ntiles, uint32_t* queue, int64_t T, int bm,
                              int group, hipStream_t stream);
int permute_chunk(int P);        // pairs per rank/histogram chunk (at most 64 chunks)
int permute_hist_stride(int P);  // histogram row stride: chunk count rounded up to 4

// experts.hip
int experts_pick_shape(int64_t T, int P, int E, int H, int I, int Is);
int experts_tile_rows(int shape);
int experts_tile_capacity(int64_t T, int P, int E, int with_shared, int shape);
hipError_t launch_gateup(const ExpertArgs& a, int shape, int tile_capacity, hipStream_t stream,
                         int fp8 = 0);
hipError_t launch_down(const ExpertArgs& a, int shape, int tile_capacity, hipStream_t stream,
                       int fp8 = 0);
hipError_t launch_combine(const uint16_t* o_routed, const uint16_t* o_shared,
                          const int32_t* pair_pos, int k, int64_t T, int H, uint16_t* y,
                          hipStream_t stream);

}  // namespace moe
