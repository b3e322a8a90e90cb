// CPU oracle of the Step-3.5-Flash sparse-MoE FFN layer forward.
//
// TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
// baseline leg of the benchmark may load this library.  The GPU product path
// never calls it, links it or shares code with it.
//
// What it computes, per token, in double precision (inputs are widened
// exactly from bf16 / fp32), following the pages:
//
//  * sglang-jax issue "[Feature] Support Step 3.5 Flash (StepFun) Model",
//    section "Model configuration", MoE bullet: 288 routed experts plus one
//    shared expert of intermediate 1280, top-8, a sigmoid router evaluated
//    in fp32, a router bias, top-k weights normalised and scaled by 3.0; and
//    the clamped-SwiGLU bullet (a limit of zero disables the clamp).
//  * same issue, "Key difficulties", item 1: the sigmoid scores are taken in
//    fp32; the router bias only decides which experts are selected; the
//    gating weights come from the scores without the bias, then are
//    normalised over the selected experts and multiplied by the routed
//    scaling factor 3.0.
//  * same issue, "Reuse map": experts are SwiGLU MLPs (SiLU of the gate
//    times the up projection), with the clamp as an elementwise option of
//    that activation.
//  * llm-atlas Step-3.5-Flash model card, "Raw config fields": hidden_size,
//    moe_num_experts, moe_top_k, moe_intermediate_size, share_expert_dim,
//    norm_expert_weight, moe_router_activation (sigmoid),
//    moe_router_scaling_factor (3), use_moe_router_bias, need_fp32_gate,
//    swiglu_limits, swiglu_limits_shared.
//
// Readings taken where the pages leave a step open (each is pinned by a test
// or marked unpinned there):
//  R1 the bias is added to the sigmoid score: key = sigmoid(z) + b.
//  R2 plain top-k over all experts (no expert groups among the raw fields).
//  R3 equal keys: the lower expert index ranks first.
//  R5 no epsilon in the renormalisation.
//  R6 the shared expert enters with weight 1.0 and no gate.
//  R7 clamp: gate = min(gate, L), up = clamp(up, -L, L), then SiLU(gate)*up.
//
// Weight layouts (out x in, row-major): gate/up [E][I][H], down [E][H][I],
// shared gate/up [Is][H], shared down [H][Is], router [E][H].

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

namespace {

struct Cfg {
  int64_t T;
  int32_t H, E, k, I, Is;
  double routed_scaling;
  int32_t renormalize;
  double limit;         // routed clamp, <= 0: none
  double limit_shared;  // shared clamp, <= 0: none
};

double bf16_to_double(uint16_t b) {
  uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return static_cast<double>(f);
}

double sigmoid(double v) { return 1.0 / (1.0 + std::exp(-v)); }

// SwiGLU activation of one intermediate unit, with the optional clamp (R7).
double swiglu(double g, double u, double limit) {
  if (limit > 0.0) {
    g = std::min(g, limit);
    u = std::min(std::max(u, -limit), limit);
  }
  return g * sigmoid(g) * u;  // SiLU(g) * u
}

// OCP FP8 E4M3 ("e4m3fn") code -> value, from the format's definition:
// bit 7 sign, bits 6..3 exponent with bias 7, bits 2..0 mantissa; exponent 0
// holds the subnormals (mantissa/8) * 2^-6; all-ones exponent and mantissa
// is NaN (no infinities).  The sglang-jax issue's "Model configuration" lists
// FP8 among the official weight formats and says nothing more about it; the
// OCP E4M3 codes with one fp32 scale per output row are this oracle's
// reading of that format (not a fact the pages state).
double e4m3_to_double(uint8_t c) {
  const int sign = c >> 7, ex = (c >> 3) & 15, man = c & 7;
  double v;
  if (ex == 15 && man == 7)
    v = std::numeric_limits<double>::quiet_NaN();
  else if (ex == 0)
    v = std::ldexp(man / 8.0, -6);
  else
    v = std::ldexp(1.0 + man / 8.0, ex - 7);
  return sign ? -v : v;
}

// Weight matrices [rows][cols] as the oracle reads them: bf16, or e4m3 codes
// times a per-row scale.
struct Bf16W {
  const uint16_t* p;
  int64_t cols;
  double operator()(int64_t r, int64_t c) const { return bf16_to_double(p[r * cols + c]); }
};
// The 256 values of the e4m3 codes, each from e4m3_to_double (filled once;
// a weight read looks its code up instead of decoding it again).
struct E4m3Values {
  double v[256];
  E4m3Values() {
    for (int c = 0; c < 256; ++c) v[c] = e4m3_to_double(static_cast<uint8_t>(c));
  }
};
const E4m3Values& e4m3_values() {
  static const E4m3Values table;
  return table;
}

struct Fp8W {
  const uint8_t* p;
  const float* scale;
  int64_t cols;
  const double* value = e4m3_values().v;
  double operator()(int64_t r, int64_t c) const {
    return value[p[r * cols + c]] * static_cast<double>(scale[r]);
  }
};

// One SwiGLU expert on one activation row: out[d] = sum_i down[d][i] * a[i],
// a[i] = swiglu(gate[i] . x, up[i] . x).  Optionally returns a (the
// intermediate) in h.
template <class W>
void expert_row_w(const double* x, int H, int I, const W& gate, const W& up, const W& down,
                  double limit, double* out, double* h) {
  std::vector<double> a(I);
  for (int i = 0; i < I; ++i) {
    double g = 0.0, u = 0.0;
    for (int c = 0; c < H; ++c) {
      g += x[c] * gate(i, c);
      u += x[c] * up(i, c);
    }
    a[i] = swiglu(g, u, limit);
    if (h) h[i] = a[i];
  }
  for (int d = 0; d < H; ++d) {
    double o = 0.0;
    for (int i = 0; i < I; ++i) o += down(d, i) * a[i];
    out[d] = o;
  }
}

void expert_row(const double* x, int H, int I, const uint16_t* gate, const uint16_t* up,
                const uint16_t* down, double limit, double* out, double* h) {
  expert_row_w(x, H, I, Bf16W{gate, H}, Bf16W{up, H}, Bf16W{down, I}, limit, out, h);
}

void router_row(const Cfg& c, const double* x, const float* wg, const float* bias, double* s,
                double* key) {
  for (int e = 0; e < c.E; ++e) {
    const float* wr = wg + static_cast<int64_t>(e) * c.H;
    double z = 0.0;
    for (int h = 0; h < c.H; ++h) z += x[h] * static_cast<double>(wr[h]);
    s[e] = sigmoid(z);
    key[e] = s[e] + (bias ? static_cast<double>(bias[e]) : 0.0);
  }
}

// Top-k by (key descending, expert index ascending); returns the k ids in
// that order and the gap between the k-th and (k+1)-th keys.
double select_topk(const Cfg& c, const double* key, int32_t* ids) {
  std::vector<int32_t> order(c.E);
  for (int e = 0; e < c.E; ++e) order[e] = e;
  std::sort(order.begin(), order.end(), [key](int32_t a, int32_t b) {
    if (key[a] != key[b]) return key[a] > key[b];
    return a < b;
  });
  for (int j = 0; j < c.k; ++j) ids[j] = order[j];
  if (c.k >= c.E) return std::numeric_limits<double>::infinity();
  return key[order[c.k - 1]] - key[order[c.k]];
}

// Gating weights from the bias-free scores of the selected experts.
void gating_weights(const Cfg& c, const double* s, const int32_t* ids, double* w) {
  double sum = 0.0;
  for (int j = 0; j < c.k; ++j) {
    w[j] = s[ids[j]];
    sum += w[j];
  }
  for (int j = 0; j < c.k; ++j) {
    if (c.renormalize) w[j] /= sum;
    w[j] *= c.routed_scaling;
  }
}

template <class F>
void parallel_for(int64_t n, int threads, F f) {
  if (threads < 1) threads = 1;
  if (n < threads) threads = static_cast<int>(std::max<int64_t>(n, 1));
  if (threads == 1) {
    for (int64_t i = 0; i < n; ++i) f(i);
    return;
  }
  std::vector<std::thread> pool;
  int64_t chunk = (n + threads - 1) / threads;
  for (int t = 0; t < threads; ++t) {
    int64_t b = t * chunk, e = std::min<int64_t>(n, b + chunk);
    if (b >= e) break;
    pool.emplace_back([=] {
      for (int64_t i = b; i < e; ++i) f(i);
    });
  }
  for (auto& th : pool) th.join();
}

bool cfg_ok(const Cfg* c) {
  return c && c->T >= 0 && c->H > 0 && c->E > 0 && c->k >= 1 && c->k <= c->E && c->I > 0 &&
         c->Is >= 0;
}

}  // namespace

extern "C" {

// Routing of every token: ids [T][k] (key descending, ties to the lower
// index), gating weights w [T][k], gap [T] = key(k-th) - key((k+1)-th)
// (+inf when k == E), and optionally all keys [T][E] and scores [T][E].
int oracle_route(const Cfg* c, const uint16_t* x, const float* wg, const float* bias,
                 int32_t* ids, double* w, double* gap, double* keys, double* scores,
                 int threads) {
  if (!cfg_ok(c) || !x || !wg || !ids || !w || !gap) return 1;
  parallel_for(c->T, threads, [&](int64_t t) {
    std::vector<double> xr(c->H), s(c->E), key(c->E);
    for (int h = 0; h < c->H; ++h) xr[h] = bf16_to_double(x[t * c->H + h]);
    router_row(*c, xr.data(), wg, bias, s.data(), key.data());
    gap[t] = select_topk(*c, key.data(), ids + t * c->k);
    gating_weights(*c, s.data(), ids + t * c->k, w + t * c->k);
    if (keys) std::copy(key.begin(), key.end(), keys + t * c->E);
    if (scores) std::copy(s.begin(), s.end(), scores + t * c->E);
  });
  return 0;
}

// Layer output for `ntok` tokens (token ids in `tokens`, or 0..ntok-1 when
// tokens is null).  When forced_ids [ntok][k] is given the router's choice is
// replaced by it and the gating weights are recomputed from the bias-free
// scores over that set.  y [ntok][H]; ids_out/w_out [ntok][k] optional.
int oracle_forward(const Cfg* c, const uint16_t* x, const float* wg, const float* bias,
                   const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                   const uint16_t* ws_gate, const uint16_t* ws_up, const uint16_t* ws_down,
                   const int64_t* tokens, int64_t ntok, const int32_t* forced_ids, double* y,
                   int32_t* ids_out, double* w_out, int threads) {
  if (!cfg_ok(c) || !x || !wg || !w_gate || !w_up || !w_down || !y || ntok < 0) return 1;
  if (c->Is > 0 && (!ws_gate || !ws_up || !ws_down)) return 1;
  const int64_t HI = static_cast<int64_t>(c->H) * c->I;
  parallel_for(ntok, threads, [&](int64_t n) {
    const int64_t t = tokens ? tokens[n] : n;
    std::vector<double> xr(c->H), s(c->E), key(c->E), o(c->H), acc(c->H, 0.0), w(c->k);
    std::vector<int32_t> ids(c->k);
    for (int h = 0; h < c->H; ++h) xr[h] = bf16_to_double(x[t * c->H + h]);
    router_row(*c, xr.data(), wg, bias, s.data(), key.data());
    if (forced_ids)
      std::copy(forced_ids + n * c->k, forced_ids + (n + 1) * c->k, ids.begin());
    else
      select_topk(*c, key.data(), ids.data());
    gating_weights(*c, s.data(), ids.data(), w.data());
    for (int j = 0; j < c->k; ++j) {
      const int64_t e = ids[j];
      expert_row(xr.data(), c->H, c->I, w_gate + e * HI, w_up + e * HI, w_down + e * HI,
                 c->limit, o.data(), nullptr);
      for (int d = 0; d < c->H; ++d) acc[d] += w[j] * o[d];
    }
    if (c->Is > 0) {
      expert_row(xr.data(), c->H, c->Is, ws_gate, ws_up, ws_down, c->limit_shared, o.data(),
                 nullptr);
      for (int d = 0; d < c->H; ++d) acc[d] += o[d];
    }
    std::copy(acc.begin(), acc.end(), y + n * c->H);
    if (ids_out) std::copy(ids.begin(), ids.end(), ids_out + n * c->k);
    if (w_out) std::copy(w.begin(), w.end(), w_out + n * c->k);
  });
  return 0;
}

// oracle_forward with the routed experts' weights in FP8 (forced_ids as
// there): e4m3 codes
// w8_gate/w8_up [E][I][H], w8_down [E][H][I] and fp32 scales per output row
// s_gate/s_up [E][I], s_down [E][H]; weight = e4m3_to_double(code) * scale.
// The shared expert stays bf16.
int oracle_forward_fp8(const Cfg* c, const uint16_t* x, const float* wg, const float* bias,
                       const uint8_t* w8_gate, const uint8_t* w8_up, const uint8_t* w8_down,
                       const float* s_gate, const float* s_up, const float* s_down,
                       const uint16_t* ws_gate, const uint16_t* ws_up, const uint16_t* ws_down,
                       const int64_t* tokens, int64_t ntok, const int32_t* forced_ids, double* y,
                       int32_t* ids_out, double* w_out, int threads) {
  if (!cfg_ok(c) || !x || !wg || !w8_gate || !w8_up || !w8_down || !s_gate || !s_up || !s_down ||
      !y || ntok < 0)
    return 1;
  if (c->Is > 0 && (!ws_gate || !ws_up || !ws_down)) return 1;
  const int64_t HI = static_cast<int64_t>(c->H) * c->I;
  parallel_for(ntok, threads, [&](int64_t n) {
    const int64_t t = tokens ? tokens[n] : n;
    std::vector<double> xr(c->H), s(c->E), key(c->E), o(c->H), acc(c->H, 0.0), w(c->k);
    std::vector<int32_t> ids(c->k);
    for (int h = 0; h < c->H; ++h) xr[h] = bf16_to_double(x[t * c->H + h]);
    router_row(*c, xr.data(), wg, bias, s.data(), key.data());
    if (forced_ids)
      std::copy(forced_ids + n * c->k, forced_ids + (n + 1) * c->k, ids.begin());
    else
      select_topk(*c, key.data(), ids.data());
    gating_weights(*c, s.data(), ids.data(), w.data());
    for (int j = 0; j < c->k; ++j) {
      const int64_t e = ids[j];
      expert_row_w(xr.data(), c->H, c->I, Fp8W{w8_gate + e * HI, s_gate + e * c->I, c->H},
                   Fp8W{w8_up + e * HI, s_up + e * c->I, c->H},
                   Fp8W{w8_down + e * HI, s_down + e * c->H, c->I}, c->limit, o.data(), nullptr);
      for (int d = 0; d < c->H; ++d) acc[d] += w[j] * o[d];
    }
    if (c->Is > 0) {
      expert_row(xr.data(), c->H, c->Is, ws_gate, ws_up, ws_down, c->limit_shared, o.data(),
                 nullptr);
      for (int d = 0; d < c->H; ++d) acc[d] += o[d];
    }
    std::copy(acc.begin(), acc.end(), y + n * c->H);
    if (ids_out) std::copy(ids.begin(), ids.end(), ids_out + n * c->k);
    if (w_out) std::copy(w.begin(), w.end(), w_out + n * c->k);
  });
  return 0;
}

// e4m3 codes -> values (for the format's pins).
int oracle_e4m3_decode(const uint8_t* codes, int64_t n, double* out) {
  if (n < 0 || (n > 0 && (!codes || !out))) return 1;
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_to_double(codes[i]);
  return 0;
}

// One SwiGLU expert applied row by row (the per-expert loop):
// rows [n][H] bf16 -> h [n][I] (the activation SiLU(g)*u) and o [n][H].
int oracle_expert(int32_t H, int32_t I, double limit, const uint16_t* rows, int64_t n,
                  const uint16_t* gate, const uint16_t* up, const uint16_t* down, double* h,
                  double* o, int threads) {
  if (H <= 0 || I <= 0 || n < 0 || !rows || !gate || !up || !down || !o) return 1;
  parallel_for(n, threads, [&](int64_t r) {
    std::vector<double> xr(H);
    for (int c = 0; c < H; ++c) xr[c] = bf16_to_double(rows[r * H + c]);
    expert_row(xr.data(), H, I, gate, up, down, limit, o + r * H, h ? h + r * I : nullptr);
  });
  return 0;
}

// Expert-sorted order of the (token, slot) pairs p = t*k + j, by a stable
// counting sort on the expert id: offsets [E+1] (exclusive prefix of the
// per-expert counts), sorted [T*k] (pair ids grouped by expert, ascending p
// within an expert), pos [T*k] (inverse: pos[sorted[i]] = i).
int oracle_permute(int64_t T, int32_t k, int32_t E, const int32_t* ids, int32_t* offsets,
                   int32_t* sorted, int32_t* pos) {
  if (T < 0 || k < 1 || E < 1 || !offsets || (T > 0 && (!ids || !sorted || !pos))) return 1;
  const int64_t P = T * k;
  std::vector<int64_t> count(E, 0);
  for (int64_t p = 0; p < P; ++p) {
    if (ids[p] < 0 || ids[p] >= E) return 2;
    ++count[ids[p]];
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = static_cast<int32_t>(offsets[e] + count[e]);
  std::vector<int64_t> next(offsets, offsets + E);
  for (int64_t p = 0; p < P; ++p) {
    const int64_t i = next[ids[p]]++;
    sorted[i] = static_cast<int32_t>(p);
    pos[p] = static_cast<int32_t>(i);
  }
  return 0;
}

int oracle_hardware_threads(void) {
  unsigned n = std::thread::hardware_concurrency();
  return n ? static_cast<int>(n) : 1;
}

}  // extern "C"
