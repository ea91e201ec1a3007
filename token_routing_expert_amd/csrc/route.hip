// route.hip -- top-k selection and renormalised softmax weights per token.
//
// "Expert parallelism" (Hugging Face Transformers docs), section "Adding an
// implementation": the expert path takes each token's selected expert ids
// (top_k_index) and routing weights (top_k_weights).  Selection: the k
// largest logits, equal logits ordered by the lower expert index; weights:
// softmax over the E logits renormalised over the k picks, which equals
// exp(l_j - l_0) / sum_i exp(l_i - l_0) over the picks.
//
// Design: a group of G lanes (a whole wave64 when E > 32) owns one token and
// holds its logits in registers, S = ceil(E / G) per lane.  Each logit is
// turned into a 64-bit key that orders as the selection rule does (logit in
// the high word, mapped to an unsigned order; the complement of the expert
// index in the low word), so k rounds of a group max-reduction over lane
// shuffles pick the experts in slot order with exact integer comparisons.
#include "common.hpp"

namespace tre {
namespace {

// Unsigned order of a float32: larger float -> larger integer; -0.0 is
// mapped to +0.0 first so that the two compare equal.
__device__ __forceinline__ uint32_t float_order(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_to_float(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __builtin_bit_cast(float, u);
}

// Key of expert e: nonzero for every real expert, so 0 marks "none".
__device__ __forceinline__ uint64_t make_key(float logit, int e) {
  return ((uint64_t)float_order(logit) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

template <int G>
__device__ __forceinline__ uint64_t group_max(uint64_t v) {
#pragma unroll
  for (int off = G / 2; off > 0; off >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, off, G);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, G);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = G / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, G);
  return v;
}

template <int G, int S>
__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits, int T, int E, int k,
                                                    int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_w) {
  const int lane = threadIdx.x % G;
  const int64_t t = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / G;
  const bool active = t < T;  // a group is either wholly active or wholly idle

  uint64_t key[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int e = s * G + lane;
    key[s] = (active && e < E) ? make_key(logits[t * E + e], e) : 0ull;
  }

  uint64_t sel[S];  // pick j is held by lane j % G in slot j / G
#pragma unroll
  for (int s = 0; s < S; ++s) sel[s] = 0ull;
  uint64_t first = 0ull;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0ull;
#pragma unroll
    for (int s = 0; s < S; ++s) best = key[s] > best ? key[s] : best;
    best = group_max<G>(best);
    if (j == 0) first = best;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (key[s] == best) key[s] = 0ull;
      if (s == j / G && lane == j % G) sel[s] = best;
    }
  }
  if (!active) return;

  const float m = order_to_float((uint32_t)(first >> 32));
  float p[S];
  float local = 0.f;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const bool mine = s * G + lane < k;
    p[s] = mine ? expf(order_to_float((uint32_t)(sel[s] >> 32)) - m) : 0.f;
    local += p[s];
  }
  const float z = group_sum<G>(local);
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int j = s * G + lane;
    if (j < k) {
      topk_idx[t * k + j] = (int32_t)(0xFFFFFFFFu - (uint32_t)sel[s]);
      topk_w[t * k + j] = p[s] / z;
    }
  }
}

template <int G, int S>
hipError_t launch(const float* logits, int T, int E, int k, int32_t* idx, float* w, hipStream_t s) {
  const int per_block = 256 / G;
  const int blocks = (int)ceil_div(T, per_block);
  k_route_topk<G, S><<<blocks, 256, 0, s>>>(logits, T, E, k, idx, w);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* topk_idx,
                             float* topk_w, hipStream_t s) {
  if (E <= 8) return launch<8, 1>(logits, T, E, k, topk_idx, topk_w, s);
  if (E <= 16) return launch<16, 1>(logits, T, E, k, topk_idx, topk_w, s);
  if (E <= 32) return launch<32, 1>(logits, T, E, k, topk_idx, topk_w, s);
  if (E <= 64) return launch<64, 1>(logits, T, E, k, topk_idx, topk_w, s);
  if (E <= 128) return launch<64, 2>(logits, T, E, k, topk_idx, topk_w, s);
  return launch<64, 4>(logits, T, E, k, topk_idx, topk_w, s);
}

}  // namespace tre
