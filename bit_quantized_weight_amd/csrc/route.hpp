// Top-k softmax router for the MoE path (Decapybara page, CUDA kernel list:
// a top-8 softmax router in front of the experts).
//
// For one token's E router logits it selects the top_k experts, largest
// logit first, equal logits in increasing expert order, and weights them by
// a softmax over the selected logits only:
//     p_j = exp(l_j - l_0) / sum_{i < top_k} exp(l_i - l_0)
// (l_0 is the largest selected logit), which equals the full softmax
// renormalised over the selection. Ordering: -0 and +0 are equal; a NaN
// logit ranks below every number (and NaNs among themselves by index), so
// the selection is defined for any input; the weights are only meaningful
// for finite logits.
//
// One wave routes one token. The selection is a sequence of top_k wave-wide
// maxima of a 64-bit key (order-preserving logit bits, then the complement
// of the index), each restricted to keys below the previous maximum, so no
// per-element "taken" state is needed and any E works; the selected logit is
// recovered from its key. All arithmetic is exact except the softmax (fp32,
// fixed summation order j = 0, 1, ...).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

// Order-preserving 32-bit image of a logit: larger number -> larger key;
// -0 maps like +0; every NaN maps to 0, below -inf (which maps to 0x007FFFFF).
__device__ __forceinline__ uint32_t logit_order(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  if (v != v) return 0u;
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t route_key(float v, int e) {
  return ((uint64_t)logit_order(v) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

// Inverse of logit_order (NaN for key 0; -0 comes back as +0, which gives the
// same softmax term).
__device__ __forceinline__ float logit_from_order(uint32_t k) {
  if (k == 0u) return __builtin_nanf("");
  return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Max of an unsigned word over the wave, in every lane: quad butterflies and
// the half-row and row mirrors (DPP, each fused into the max) give each row
// of 16 its maximum; the gfx950 lane swaps of rows (permlane16) and halves
// (permlane32) finish the wave.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
  const uint32_t o = __builtin_amdgcn_update_dpp(0u, v, CTRL, 0xf, 0xf, false);
  return o > v ? o : v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_u32<0xB1>(v);    // quad_perm [1,0,3,2]
  v = dpp_max_u32<0x4E>(v);    // quad_perm [2,3,0,1]
  v = dpp_max_u32<0x141>(v);   // row_half_mirror
  v = dpp_max_u32<0x140>(v);   // row_mirror
  {
    const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = p[0] > p[1] ? p[0] : p[1];
  }
  {
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    v = p[0] > p[1] ? p[0] : p[1];
  }
  return v;
}

// Max of a 64-bit key over the wave, in every lane: the largest high word,
// then the largest low word among the lanes that hold it (two 32-bit wave
// maxima instead of one 64-bit one: each step is a single fused max).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  const uint32_t hi = wave_max_u32((uint32_t)(v >> 32));
  const uint32_t lo = wave_max_u32((uint32_t)(v >> 32) == hi ? (uint32_t)v : 0u);
  return ((uint64_t)hi << 32) | lo;
}

// The lane's logits of one token for the register-cached keys: experts lane,
// lane + 64, ... from its E logits at lg (any memory the wave can read); every
// load is issued, clamped in range, before any is used.
template <int RK>
__device__ __forceinline__ void route_logits(const float* lg, int E, float (&v)[RK]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < RK; ++i) {
    const int e = lane + 64 * i;
    v[i] = lg[e < E ? e : E - 1];
  }
}

// Their keys (0 past E).
template <int RK>
__device__ __forceinline__ void route_keys(const float (&v)[RK], int E, uint64_t (&key)[RK]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < RK; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? route_key(v[i], e) : 0ull;
  }
}

// Routes one token with the whole wave. On return lane j < top_k holds the
// j-th selected expert in *id and its weight in *gate; other lanes hold -1 /
// 0. Every real key exceeds 0 (its low word is at least 2^32 - E), so 0
// marks "nothing left", which cannot happen while top_k <= E. RK > 0: the
// lane's keys come from route_keys (E <= 64 * RK; lg unused); RK = 0: any E,
// keys recomputed from the logits at lg on every pass.
template <int RK>
__device__ __forceinline__ void route_select(const uint64_t* key, const float* lg, int E, int top_k, int* id,
                                             float* gate) {
  const int lane = threadIdx.x & 63;
  uint64_t prev = ~0ull;
  int my_id = -1;
  float my_v = 0.0f;
  for (int j = 0; j < top_k; ++j) {
    uint64_t best = 0ull;
    if constexpr (RK > 0) {
#pragma unroll
      for (int i = 0; i < RK; ++i)
        if (key[i] < prev && key[i] > best) best = key[i];
    } else {
      for (int e = lane; e < E; e += 64) {
        const uint64_t k = route_key(lg[e], e);
        if (k < prev && k > best) best = k;
      }
    }
    best = wave_max_u64(best);
    prev = best;
    if (lane == j && best != 0ull) {
      my_id = (int)(0xFFFFFFFFu - (uint32_t)best);
      my_v = logit_from_order((uint32_t)(best >> 32));
    }
  }
  // softmax over the selection, shifted by the largest selected logit
  const float v0 = __shfl(my_v, 0);
  const float ex = lane < top_k ? expf(my_v - v0) : 0.0f;
  float sum = 0.0f;
  for (int j = 0; j < top_k; ++j) sum += __shfl(ex, j);
  *id = my_id;
  *gate = lane < top_k ? ex / sum : 0.0f;
}

template <int RK>
__device__ __forceinline__ void route_token(const float* lg, int E, int top_k, int* id, float* gate) {
  if constexpr (RK > 0) {
    float v[RK];
    uint64_t key[RK];
    route_logits<RK>(lg, E, v);
    route_keys<RK>(v, E, key);
    route_select<RK>(key, lg, E, top_k, id, gate);
  } else {
    route_select<0>(nullptr, lg, E, top_k, id, gate);
  }
}

// route_token with the register-cached keys when E allows.
__device__ __forceinline__ void route_token_any(const float* lg, int E, int top_k, int* id, float* gate) {
  if (E <= 128) route_token<2>(lg, E, top_k, id, gate);
  else if (E <= 256) route_token<4>(lg, E, top_k, id, gate);
  else route_token<0>(lg, E, top_k, id, gate);
}

}  // namespace qg
