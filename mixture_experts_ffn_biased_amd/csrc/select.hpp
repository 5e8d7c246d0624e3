// Top-k selection of one token by one wave, shared by the router kernels and
// the fused small-layer kernel.
//
// "Mixture of Experts and Hybrid Architectures", "The router in code";
// "Sparse MoE FFN" (DeepSeek-V3), "How it works", Routing: s = l (softmax
// mode) or sigmoid(l); sb = s + bias; with groups, group score = sum of the
// two largest sb, keep the topk_groups best groups; top-k of sb over the
// eligible experts, larger first, ties to the lower index, NaN last.  Gates
// come from the raw scores: softmax over the chosen logits, or s / sum(s)
// over the chosen, times route_scale.
#pragma once

#include "common.hpp"
#include "plan.hpp"

namespace moe {
namespace {

struct SelArgs {
  int E, k, score_fn, G, M;
  float route_scale;
  const float *bias;
};

// Selection for one token by one wave; lg = the token's E logits (LDS).
__device__ inline void select_token(const float *lg, const SelArgs &a, int32_t *idx_out,
                                    float *gate_out) {
  const int lane = threadIdx.x & 63;
  constexpr int P = kMaxExperts / 64;
  float gs[P];       // raw score used by the gates (l or sigmoid(l))
  uint64_t key[P];   // ranking key of s + bias; 0 = not a candidate
  int grp[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int e = lane + 64 * p;
    gs[p] = 0.f;
    key[p] = 0;
    grp[p] = 0;
    if (e < a.E) {
      const float l = lg[e];
      const float s = a.score_fn == MOE_SCORE_SIGMOID ? 1.0f / (1.0f + expf(-l)) : l;
      const float sb = s + (a.bias ? a.bias[e] : 0.0f);
      gs[p] = s;
      key[p] = rank_key(sb, e);
      grp[p] = e / (a.E / a.G);
    }
  }

  if (a.G > 1) {
    // Group score: the two largest biased scores of each group.
    float my_gscore = 0.f;
    if (a.E == 32 * a.G && (a.E & 63) == 0) {
      // Groups of 32: slot p of lane l is expert l + 64p, in group 2p + l/32,
      // so each half of the wave holds one whole group per slot, and one
      // half-wave maximum gives two groups' largest key at once.
#pragma unroll
      for (int p = 0; p < P; ++p) {
        if (2 * p >= a.G) break;
        const uint64_t k1 = half_max_u64(key[p]);
        const uint64_t k2 = half_max_u64(key[p] != k1 ? key[p] : 0);
        const int sc = __float_as_int(key_value(k1) + key_value(k2));
        const float s0 = __int_as_float(__builtin_amdgcn_readlane(sc, 0));   // group 2p
        const float s1 = __int_as_float(__builtin_amdgcn_readlane(sc, 32));  // group 2p + 1
        if (lane == 2 * p) my_gscore = s0;
        if (lane == 2 * p + 1) my_gscore = s1;
      }
    } else {
      for (int g = 0; g < a.G; ++g) {
        uint64_t k1 = 0;
#pragma unroll
        for (int p = 0; p < P; ++p)
          if (grp[p] == g && key[p] > k1) k1 = key[p];
        k1 = wave_max_u64(k1);
        uint64_t k2 = 0;
#pragma unroll
        for (int p = 0; p < P; ++p)
          if (grp[p] == g && key[p] != k1 && key[p] > k2) k2 = key[p];
        k2 = wave_max_u64(k2);
        const float sc = key_value(k1) + key_value(k2);
        if (lane == g) my_gscore = sc;
      }
    }
    uint64_t gkey = lane < a.G ? rank_key(my_gscore, lane) : 0;
    uint64_t kept = 0;
    for (int r = 0; r < a.M; ++r) {
      const uint64_t best = wave_max_u64(gkey);
      const int g = key_index(best);
      kept |= 1ull << g;
      if (lane == g) gkey = 0;
    }
#pragma unroll
    for (int p = 0; p < P; ++p)
      if (!((kept >> grp[p]) & 1ull)) key[p] = 0;
  }

  int my_idx = 0;
  float my_gs = 0.f;
  for (int j = 0; j < a.k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int p = 0; p < P; ++p) best = key[p] > best ? key[p] : best;
    best = wave_max_u64(best);
    const int e = key_index(best);
    const int owner = e & 63, pe = e >> 6;
    float v = 0.f;
#pragma unroll
    for (int p = 0; p < P; ++p)
      if (p == pe) v = gs[p];
    v = __shfl(v, owner, 64);
    if (lane == owner) {
#pragma unroll
      for (int p = 0; p < P; ++p)
        if (p == pe) key[p] = 0;
    }
    if (lane == j) {
      my_idx = e;
      my_gs = v;
    }
  }

  const bool mine = lane < a.k;
  float gate;
  if (a.score_fn == MOE_SCORE_SIGMOID) {
    const float sum = wave_sum_f32(mine ? my_gs : 0.f);
    gate = a.route_scale * my_gs / sum;
  } else {
    float m = mine ? my_gs : -INFINITY;
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
    const float ex = mine ? expf(my_gs - m) : 0.f;
    const float sum = wave_sum_f32(ex);
    gate = a.route_scale * ex / sum;
  }
  if (mine) {
    idx_out[lane] = my_idx;
    gate_out[lane] = gate;
  }
}

}  // namespace
}  // namespace moe
