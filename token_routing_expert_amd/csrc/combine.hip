// combine.hip -- routing-weighted sum of the expert outputs, back in token order.
//
// "Expert parallelism" (Hugging Face Transformers docs), sections "Token
// dispatch" and "Adding an implementation": the expert outputs of a token
// are combined with its routing weights into the token's weighted expert
// output:
//   out[t] = sum over j < k (pair_row[t*k+j] valid) of pair_w[t*k+j] * y_perm[pair_row[t*k+j]]
// float32 accumulation in ascending j, one rounding to the output type.
//
// One wave per token; lanes walk the row in 16-byte vectors, so each of the
// k gathered rows is read with full 16-byte coalescing and the output row is
// written once.  Bandwidth-bound: reads P rows, writes T rows.
#include "common.hpp"

namespace tre {
namespace {

constexpr int kThreads = 256;

template <typename Elem>
struct Vec;  // one 16-byte vector of Elem and its float32 expansion
template <>
struct Vec<bf16_t> {
  static constexpr int n = 8;
  static __device__ __forceinline__ void load(const u32x4& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __builtin_bit_cast(float, v[i] << 16);
      f[2 * i + 1] = __builtin_bit_cast(float, v[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ u32x4 store(const float* f) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return v;
  }
};
template <>
struct Vec<float> {
  static constexpr int n = 4;
  static __device__ __forceinline__ void load(const u32x4& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // copy the element out first: clang's bit_cast of a vector-element
      // lvalue reads element 0 whatever the index
      const uint32_t u = v[i];
      f[i] = __builtin_bit_cast(float, u);
    }
  }
  static __device__ __forceinline__ u32x4 store(const float* f) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __builtin_bit_cast(uint32_t, f[i]);
    return v;
  }
};

// Up to KS slots: each lane first loads its vector of every slot's row (a
// row index clamped into range, a dropped slot's value discarded by a
// select), for two vectors at a time, so 2 KS gathers are in flight together.
// Every expert row is read once: non-temporal loads (measured: the cold
// combine of the 128-expert layer 47.5 -> 45.3 us).
template <typename Elem, int KS>
__device__ __forceinline__ void combine_token(const u32x4* __restrict__ y, int64_t max_rows,
                                              const int32_t* __restrict__ pair_row, const float* __restrict__ pair_w,
                                              int64_t t, int k, int64_t vec_per_row, u32x4* __restrict__ out) {
  constexpr int n = Vec<Elem>::n;
  const int lane = threadIdx.x % kWave;
  int64_t row[KS];
  float wt[KS];
  bool live[KS];
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    const int64_t r = j < k ? pair_row[t * k + j] : -1;
    MOE_DCHECK(r >= -1 && r < max_rows);   // a grouped row, or -1 for a dropped pair
    live[j] = r >= 0 && r < max_rows;
    row[j] = live[j] ? r : 0;
    wt[j] = (j < k && pair_w) ? pair_w[t * k + j] : 1.f;
  }
  for (int64_t v0 = lane; v0 < vec_per_row; v0 += 2 * kWave) {
    u32x4 g[2][KS];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t v = v0 + h * kWave;
#pragma unroll
      for (int j = 0; j < KS; ++j)
        if (j < k && max_rows > 0 && v < vec_per_row) g[h][j] = __builtin_nontemporal_load(&y[row[j] * vec_per_row + v]);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t v = v0 + h * kWave;
      if (v >= vec_per_row) continue;
      float acc[n];
#pragma unroll
      for (int i = 0; i < n; ++i) acc[i] = 0.f;
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        if (j >= k || !live[j]) continue;
        float f[n];
        Vec<Elem>::load(g[h][j], f);
#pragma unroll
        for (int i = 0; i < n; ++i) acc[i] = fmaf(wt[j], f[i], acc[i]);
      }
      out[t * vec_per_row + v] = Vec<Elem>::store(acc);
    }
  }
}

// KS > 0: at most KS slots (combine_token); KS == 0: any k, one slot at a time
template <typename Elem, int KS>
__global__ __launch_bounds__(kThreads) void k_combine(const u32x4* __restrict__ y, int64_t max_rows,
                                                      const int32_t* __restrict__ pair_row,
                                                      const float* __restrict__ pair_w, int64_t n_tok, int k,
                                                      int64_t vec_per_row, u32x4* __restrict__ out) {
  constexpr int n = Vec<Elem>::n;
  const int64_t t = (int64_t)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  if (t >= n_tok) return;
  if constexpr (KS > 0) {
    combine_token<Elem, KS>(y, max_rows, pair_row, pair_w, t, k, vec_per_row, out);
    return;
  }
  const int lane = threadIdx.x % kWave;
  for (int64_t v = lane; v < vec_per_row; v += kWave) {
    float acc[n];
#pragma unroll
    for (int i = 0; i < n; ++i) acc[i] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int64_t r = pair_row[t * k + j];
      MOE_DCHECK(r >= -1 && r < max_rows);
      if (r < 0 || r >= max_rows) continue;
      const float w = pair_w ? pair_w[t * k + j] : 1.f;
      float f[n];
      Vec<Elem>::load(y[r * vec_per_row + v], f);
#pragma unroll
      for (int i = 0; i < n; ++i) acc[i] = fmaf(w, f[i], acc[i]);
    }
    out[t * vec_per_row + v] = Vec<Elem>::store(acc);
  }
}

// Backward of the combine.  With dy_p = w_p dout_t for pair p = (t, j):
//   dy[pair_row[p]] = w_p * dout[t]          (the gradient reaching the expert)
//   dw[p]           = <dout[t], y[pair_row[p]]>  (the routing weight's gradient)
// and, when the weights are the softmax of the selected logits,
//   dlogits[t, topk_idx[p]] = w_p (dw_p - sum_i w_i dw_i), zero elsewhere.
// One wave per token, slots in ascending order; each dot product is summed
// in float32 over the lanes' 16-byte vectors and then across the wave.
template <typename Elem>
__global__ __launch_bounds__(kThreads) void k_combine_bwd(
    const u32x4* __restrict__ dout, const u32x4* __restrict__ y, int64_t max_rows, const int32_t* __restrict__ pair_row,
    const float* __restrict__ pair_w, const int32_t* __restrict__ topk_idx, int64_t n_tok, int k, int E,
    int64_t vec_per_row, u32x4* __restrict__ dy, float* __restrict__ dw, float* __restrict__ dlogits) {
  // every lane of a wave writes the same value to its token's slot j and
  // later reads back only what it wrote itself
  __shared__ float s_dw[kThreads / kWave][kMaxExperts];
  const int64_t t = (int64_t)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  if (t >= n_tok) return;
  const int lane = threadIdx.x % kWave;
  float* my_dw = s_dw[threadIdx.x / kWave];
  float inner = 0.f;
  for (int j = 0; j < k; ++j) {
    const int64_t r = pair_row[t * k + j];
    const bool live = r >= 0 && r < max_rows;
    const float w = pair_w[t * k + j];
    float dot = 0.f;
    if (live) {
      for (int64_t v = lane; v < vec_per_row; v += kWave) {
        constexpr int NV = Vec<Elem>::n;
        float g[NV], f[NV];
        Vec<Elem>::load(dout[t * vec_per_row + v], g);
        Vec<Elem>::load(y[r * vec_per_row + v], f);
#pragma unroll
        for (int i = 0; i < NV; ++i) dot = fmaf(g[i], f[i], dot);
#pragma unroll
        for (int i = 0; i < NV; ++i) g[i] *= w;
        dy[r * vec_per_row + v] = Vec<Elem>::store(g);
      }
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) dot += __shfl_xor(dot, off, kWave);
    }
    if (lane == 0) dw[t * k + j] = dot;
    my_dw[j] = dot;
    inner = fmaf(w, dot, inner);
  }
  if (!dlogits) return;
  for (int e = lane; e < E; e += kWave) {
    float v = 0.f;
    for (int j = 0; j < k; ++j)
      if (topk_idx[t * k + j] == e) v = pair_w[t * k + j] * (my_dw[j] - inner);
    dlogits[t * E + e] = v;
  }
}

// One pair per token, with the down projection writing the output rows
// itself: the rows of tokens whose pair has no grouped row (a dropped id)
// are zero, as the combine would leave them.  One thread checks each token;
// the wave then clears its flagged rows one after another, 16 bytes a lane.
__global__ __launch_bounds__(kThreads) void k_zero_unrouted(const int32_t* __restrict__ pair_row, int64_t max_rows,
                                                            int64_t T, int64_t vec_per_row,
                                                            u32x4* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int lane = threadIdx.x % kWave;
  bool dropped = false;
  if (t < T) {
    const int64_t r = pair_row[t];
    dropped = r < 0 || r >= max_rows;
  }
  uint64_t todo = __ballot(dropped);
  const int64_t t0 = t - lane;
  while (todo) {
    const int l = __builtin_ctzll(todo);
    todo &= todo - 1;
    for (int64_t v = lane; v < vec_per_row; v += kWave) out[(t0 + l) * vec_per_row + v] = u32x4{0u, 0u, 0u, 0u};
  }
}

template <typename Elem>
hipError_t launch(const Elem* y, int64_t max_rows, const int32_t* pair_row, const float* pair_w, int64_t n_tok,
                  int k, int d, Elem* out, hipStream_t s) {
  const int64_t vec_per_row = (int64_t)d * sizeof(Elem) / 16;
  const int64_t blocks = ceil_div(n_tok, kThreads / kWave);
  if (k <= 4)
    k_combine<Elem, 4><<<(unsigned)blocks, kThreads, 0, s>>>((const u32x4*)y, max_rows, pair_row, pair_w, n_tok, k,
                                                            vec_per_row, (u32x4*)out);
  else if (k <= 8)
    k_combine<Elem, 8><<<(unsigned)blocks, kThreads, 0, s>>>((const u32x4*)y, max_rows, pair_row, pair_w, n_tok, k,
                                                            vec_per_row, (u32x4*)out);
  else
    k_combine<Elem, 0><<<(unsigned)blocks, kThreads, 0, s>>>((const u32x4*)y, max_rows, pair_row, pair_w, n_tok, k,
                                                            vec_per_row, (u32x4*)out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine_bf16(const bf16_t* y_perm, int64_t max_rows, const int32_t* pair_row,
                               const float* pair_w, int64_t T, int k, int d, bf16_t* out, hipStream_t s) {
  return launch<bf16_t>(y_perm, max_rows, pair_row, pair_w, T, k, d, out, s);
}

namespace {

template <typename Elem>
hipError_t launch_bwd(const Elem* dout, const Elem* y_perm, int64_t max_rows, const int32_t* pair_row,
                      const float* pair_w, const int32_t* topk_idx, int64_t T, int k, int d, int E, Elem* dy_perm,
                      float* dw, float* dlogits, hipStream_t s) {
  const int64_t vec_per_row = (int64_t)d * sizeof(Elem) / 16;
  const int64_t blocks = ceil_div(T, kThreads / kWave);
  k_combine_bwd<Elem><<<(unsigned)blocks, kThreads, 0, s>>>((const u32x4*)dout, (const u32x4*)y_perm, max_rows,
                                                           pair_row, pair_w, topk_idx, T, k, E, vec_per_row,
                                                           (u32x4*)dy_perm, dw, dlogits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine_bwd_bf16(const bf16_t* dout, const bf16_t* y_perm, int64_t max_rows,
                                  const int32_t* pair_row, const float* pair_w, const int32_t* topk_idx, int64_t T,
                                  int k, int d, int E, bf16_t* dy_perm, float* dw, float* dlogits, hipStream_t s) {
  return launch_bwd<bf16_t>(dout, y_perm, max_rows, pair_row, pair_w, topk_idx, T, k, d, E, dy_perm, dw, dlogits, s);
}

hipError_t launch_combine_bwd_f32(const float* dout, const float* y_perm, int64_t max_rows,
                                  const int32_t* pair_row, const float* pair_w, const int32_t* topk_idx, int64_t T,
                                  int k, int d, int E, float* dy_perm, float* dw, float* dlogits, hipStream_t s) {
  return launch_bwd<float>(dout, y_perm, max_rows, pair_row, pair_w, topk_idx, T, k, d, E, dy_perm, dw, dlogits, s);
}

hipError_t launch_zero_unrouted_bf16(const int32_t* pair_row, int64_t max_rows, int64_t T, int d, bf16_t* out,
                                     hipStream_t s) {
  k_zero_unrouted<<<(unsigned)ceil_div(T, kThreads), kThreads, 0, s>>>(pair_row, max_rows, T, (int64_t)d * 2 / 16,
                                                                      (u32x4*)out);
  return hipGetLastError();
}

hipError_t launch_combine_f32(const float* y_perm, int64_t max_rows, const int32_t* pair_row,
                              const float* pair_w, int64_t T, int k, int d, float* out, hipStream_t s) {
  return launch<float>(y_perm, max_rows, pair_row, pair_w, T, k, d, out, s);
}

}  // namespace tre
