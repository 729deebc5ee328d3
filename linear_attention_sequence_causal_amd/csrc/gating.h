// gating.h -- the gating step of the hyper-parallel page's CP wrappers
// (LinearAttentionP2PCPWrapper.forward and its siblings), per token t and
// value head h:
//   beta = sigmoid(b),   g = -exp(A_log[h]) * softplus(a + dt_bias[h])
// in float32, with softplus(x) = max(x, 0) + log1p(exp(-|x|)) (no overflow).
// Shared by the standalone gating kernels and the chunk prep, so both form
// bit-identical gates.
#pragma once

#include <hip/hip_runtime.h>

#include "gdn_common.h"

namespace gdn_gate {

GDN_DEV float sigmoid(float x) { return 1.f / (1.f + __expf(-x)); }
GDN_DEV float softplus(float x) { return fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x))); }
GDN_DEV float beta_of(float b) { return sigmoid(b); }
GDN_DEV float g_of(float a, float A_log, float dt_bias) {
  return -__expf(A_log) * softplus(a + dt_bias);
}

// Where a prep or state pass finds the gates of (token, value head): either
// given (g, beta [T, Hv] float32) or formed from the projections a, b (token
// stride ld_ab, activation type E) and the per-head A_log, dt_bias.  With
// g_out / beta_out set, formed gates are also stored there ([T, Hv]).
struct Gates {
  const float* g;
  const float* beta;
  const void* a;
  const void* b;
  int64_t ld_ab;
  const float* A_log;
  const float* dt_bias;
  float* g_out;
  float* beta_out;
};

template <typename E>
GDN_DEV void load_gates(const Gates& G, int64_t t, int h, int Hv, float& g, float& beta) {
  if (G.a) {
    const E* ap = (const E*)G.a + t * G.ld_ab + h;
    const E* bp = (const E*)G.b + t * G.ld_ab + h;
    g = g_of(to_f(*ap), G.A_log[h], G.dt_bias[h]);
    beta = beta_of(to_f(*bp));
    if (G.g_out) G.g_out[t * Hv + h] = g;
    if (G.beta_out) G.beta_out[t * Hv + h] = beta;
  } else {
    g = G.g[t * Hv + h];
    beta = G.beta[t * Hv + h];
  }
}

}  // namespace gdn_gate
