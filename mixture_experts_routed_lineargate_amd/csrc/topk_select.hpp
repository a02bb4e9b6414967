// Top-k selection tail shared by the router's top-k pass and the small-batch
// routing kernel: one wavefront picks k experts by (logit desc, index asc) and
// writes their ids in ascending order with the renormalised softmax weights
// (evidence page, "Layer-qualified experts": LinearGate selection; Model card:
// top-8 of 128).
#pragma once

#include <float.h>

#include "internal.hpp"

namespace moe {

// Pick k winners by (value desc, index asc) with wave arg-max rounds, then
// w_j = exp(l_j - l_max) / sum_selected exp(l - l_max), written in ascending id
// order.  v[i] is the logit of expert i * WAVE + lane (ignored past E).  The
// ids also go to sorted_ids[0..k) (LDS) when given.
template <int PL>
__device__ inline void select_and_write(const float (&v)[PL], int E, int k, int64_t t, int wave,
                                        int lane, float (*sel_l)[MAX_K], int (*sel_e)[MAX_K],
                                        int32_t* __restrict__ ids, float* __restrict__ w,
                                        int* sorted_ids = nullptr) {
  // A NaN logit ranks with -inf.  Every untaken expert is a candidate, so a
  // round always finds one, even when fewer than k logits are finite (an
  // expert masked with a -inf bias): ties among -inf go to the lower index.
  constexpr int NONE = 0x7fffffff;
  uint32_t taken = 0;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int be = NONE;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = i * WAVE + lane;
      const bool ok = e < E && !((taken >> i) & 1u);
      const float vi = __builtin_isnan(v[i]) ? -INFINITY : v[i];
      if (ok && (be == NONE || vi > bv || (vi == bv && e < be))) {
        bv = vi;
        be = e;
      }
    }
    // wave argmax: largest value, then the lowest index among equals (lanes
    // without a candidate hold -inf and NONE and never win)
    const float m = wave_max(bv);
    be = wave_min(bv == m ? be : NONE);
    be = min(be, E - 1);                 // E > k >= 1 untaken experts remain, so be < E
    bv = m;
    if ((be & (WAVE - 1)) == lane) taken |= 1u << (be / WAVE);
    if (lane == 0) {
      sel_l[wave][r] = bv;
      sel_e[wave][r] = be;
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  if (lane < k) {
    const float lmax = sel_l[wave][0];
    float den = 0.f;
    for (int r = 0; r < k; ++r) den += expf(sel_l[wave][r] - lmax);
    const int me = sel_e[wave][lane];
    int rank = 0;
    for (int r = 0; r < k; ++r) rank += sel_e[wave][r] < me;
    ids[t * k + rank] = me;
    if (sorted_ids) sorted_ids[rank] = me;
    w[t * k + rank] = expf(sel_l[wave][lane] - lmax) / den;
  }
}

}  // namespace moe
