// route.hip -- top-k selection and renormalised softmax weights per token.
//
// "Expert parallelism" (Hugging Face Transformers docs), section "Adding an
// implementation": the expert path takes each token's selected expert ids
// (top_k_index) and routing weights (top_k_weights).  Selection: the k
// largest logits, equal logits ordered by the lower expert index; weights:
// softmax over the E logits renormalised over the k picks, which equals
// exp(l_j - l_0) / sum_i exp(l_i - l_0) over the picks.
//
// Design: a group of G lanes (16 for 65-128 experts, a whole wave64 for 33-64
// and for more than 128) owns one token and
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

// Route token t from this lane's logits lg[s] = logit of expert s * G + lane
// (a group of G lanes per token; the group is wholly active or wholly idle).
template <int G, int S>
__device__ __forceinline__ void route_token(const float (&lg)[S], int64_t t, bool active, int E, int k,
                                            int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  const int lane = threadIdx.x % G;
  uint64_t key[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int e = s * G + lane;
    key[s] = (active && e < E) ? make_key(lg[s], e) : 0ull;
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
__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits, int T, int E, int k,
                                                    int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_w) {
  const int lane = threadIdx.x % G;
  const int64_t t = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / G;
  const bool active = t < T;
  float lg[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int e = s * G + lane;
    lg[s] = (active && e < E) ? logits[t * E + e] : 0.f;
    MOE_DCHECK(__builtin_isfinite(lg[s]));   // logits are finite
  }
  route_token<G, S>(lg, t, active, E, k, topk_idx, topk_w);
}

template <int G, int S>
hipError_t launch(const float* logits, int T, int E, int k, int32_t* idx, float* w, hipStream_t s) {
  const int per_block = 256 / G;
  const int blocks = (int)ceil_div(T, per_block);
  k_route_topk<G, S><<<blocks, 256, 0, s>>>(logits, T, E, k, idx, w);
  return hipGetLastError();
}

// ---- router projection fused with routing --------------------------------
// "Expert parallelism" (introduction: a router sends each token to its
// experts; the router module is the model's gate linear layer, mlp.gate or
// mlp.router, "Token dispatch"): logits[t, e] = sum_c x[t, c] * Wr[e, c]
// with the layer's weight Wr [E, d], float32 accumulation; each token is then
// routed exactly as k_route_topk routes it.  Narrow routers (bf16 with at
// most 32 experts, and every float32 router): a workgroup of four waves
// takes 16 tokens, wave w sums the columns of quarter w of d straight from
// global memory, and the four partial sums are added in wave order through
// LDS.  Wider bf16 routers use the staged kernel further down.
constexpr int kProjTokens = 16;
constexpr int kProjWaves = 4;

// bf16: v_mfma_f32_16x16x32_bf16 with 16 router rows (experts) as the first
// operand and the 16 token rows as the second; both fragments are 16
// contiguous bytes of a row (lane l: row l % 16, columns 8 (l / 16) .. +7 of
// the 32-column step).  Lane l receives experts 4 (l / 16) .. +3 of token
// l % 16.  NEB = 16-expert blocks, one accumulator each.
template <int NEB, int NW>
__device__ __forceinline__ void project_bf16(const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, int64_t t0,
                                             int T, int d, int E, float (*s_part)[16 * NEB]) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int tl = lane % 16, q = lane / 16;
  const bool t_ok = t0 + tl < T;
  const int steps = d / 32, s0 = wave * steps / NW, s1 = (wave + 1) * steps / NW;
  const bf16_t* xr = x + (t_ok ? t0 + tl : 0) * (int64_t)d + q * 8;
  const bf16_t* wr[NEB];
  bool e_ok[NEB];
#pragma unroll
  for (int b = 0; b < NEB; ++b) {
    e_ok[b] = 16 * b + tl < E;
    wr[b] = w + (int64_t)(e_ok[b] ? 16 * b + tl : 0) * d + q * 8;
  }
  bf16x8 zero;
#pragma unroll
  for (int i = 0; i < 8; ++i) zero[i] = (__bf16)0.f;
  f32x4 acc[NEB];
#pragma unroll
  for (int b = 0; b < NEB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  static_assert(NEB <= 2, "wider bf16 routers use the staged kernel");
  constexpr int U = 4;  // steps whose loads are issued together
  int st = s0;
  for (; st + U <= s1; st += U) {
    bf16x8 xb[U], wb[U][NEB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      xb[u] = t_ok ? *(const bf16x8*)(xr + (st + u) * 32) : zero;
#pragma unroll
      for (int b = 0; b < NEB; ++b) wb[u][b] = e_ok[b] ? *(const bf16x8*)(wr[b] + (st + u) * 32) : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int b = 0; b < NEB; ++b) acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[u][b], xb[u], acc[b], 0, 0, 0);
  }
  for (; st < s1; ++st) {
    const bf16x8 xb = t_ok ? *(const bf16x8*)(xr + st * 32) : zero;
#pragma unroll
    for (int b = 0; b < NEB; ++b)
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e_ok[b] ? *(const bf16x8*)(wr[b] + st * 32) : zero, xb,
                                                       acc[b], 0, 0, 0);
  }
#pragma unroll
  for (int b = 0; b < NEB; ++b)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (16 * b + 4 * q + v < E) s_part[wave * kProjTokens + tl][16 * b + 4 * q + v] = acc[b][v];
}

// float32: per-lane dot products in ascending column order over the wave's
// part of d (lane l: token l % 16, experts l / 16, l / 16 + 4, ...).
template <int NEB, int NW>
__device__ __forceinline__ void project_f32(const float* __restrict__ x, const float* __restrict__ w, int64_t t0,
                                            int T, int d, int E, float (*s_part)[16 * NEB]) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int tl = lane % 16, q = lane / 16;
  if (t0 + tl >= T) return;
  const int c0 = wave * d / NW, c1 = (wave + 1) * d / NW;
  const float* xr = x + (t0 + tl) * (int64_t)d;
  for (int e = q; e < E; e += 4) {
    const float* wrow = w + (int64_t)e * d;
    float acc = 0.f;
    for (int c = c0; c < c1; ++c) acc = fmaf(xr[c], wrow[c], acc);
    s_part[wave * kProjTokens + tl][e] = acc;
  }
}

template <typename Elem, int G, int S, int NEB, int NW>
__global__ __launch_bounds__(NW * kWave) void k_route_project(
    const Elem* __restrict__ x, const Elem* __restrict__ w, int T, int d, int E, int k, float* __restrict__ logits,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  __shared__ float s_part[NW * kProjTokens][16 * NEB];  // E <= 16 NEB
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * kProjTokens;
  if constexpr (sizeof(Elem) == 2)
    project_bf16<NEB, NW>(x, w, t0, T, d, E, s_part);
  else
    project_f32<NEB, NW>(x, w, t0, T, d, E, s_part);
  __syncthreads();
  // the NW parts of d, added in order, into the first wave's rows
  for (int i = tid; i < kProjTokens * E; i += NW * kWave) {
    const int tl = i / E, e = i % E;
    if (t0 + tl >= T) continue;
    float v = s_part[tl][e];
#pragma unroll
    for (int wq = 1; wq < NW; ++wq) v += s_part[wq * kProjTokens + tl][e];
    s_part[tl][e] = v;
    if (logits) logits[(t0 + tl) * E + e] = v;
  }
  __syncthreads();
  // G lanes per token, 64 NW / G tokens at a time
  constexpr int per_pass = NW * kWave / G;
#pragma unroll
  for (int pass = 0; pass < (kProjTokens + per_pass - 1) / per_pass; ++pass) {
    const int tl = pass * per_pass + tid / G;
    const int64_t t = t0 + tl;
    const bool active = tl < kProjTokens && t < T;
    float lg[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int e = s * G + tid % G;
      lg[s] = (active && e < E) ? s_part[tl][e] : 0.f;
    }
    route_token<G, S>(lg, t, active, E, k, topk_idx, topk_w);
  }
}

template <typename Elem, int G, int S, int NEB>
hipError_t launch_project(const Elem* x, const Elem* w, int T, int d, int E, int k, float* logits, int32_t* idx,
                          float* wt, hipStream_t s) {
  k_route_project<Elem, G, S, NEB, kProjWaves><<<(unsigned)ceil_div(T, kProjTokens), kProjWaves * kWave, 0, s>>>(
      x, w, T, d, E, k, logits, idx, wt);
  return hipGetLastError();
}

// ---- wide routers (bf16, more than 32 experts) -----------------------------
// With many experts every workgroup streams the whole router weight (E rows
// of d) past its tokens, so the weight dominates the traffic and the loop is
// bound by how fast one CU can pull scattered rows from L2.  The operands go
// through a ring of NS LDS stages of 64 columns filled by loads that write LDS
// directly (both x rows and router rows, 128 bytes each per stage, 16-byte
// chunk c of row r stored at slot c ^ (r & 7) so that 16 consecutive rows of
// one chunk touch every bank once).  Wave w owns expert blocks w, w + NW, ...
// for all 16 TG tokens of the workgroup and accumulates over the whole of d,
// so the logits need no reduction across waves.
template <int NEB, int TG, int NS, int NW>
__global__ __launch_bounds__(NW * kWave) void k_route_project_staged(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, int T, int d, int E, int k,
    float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  constexpr int XR = 16 * TG, WR = 16 * NEB;  // x rows and router rows of a stage
  constexpr int NI = (XR + WR) / 8;           // 1 KB loads per stage (8 rows of 128 B each)
  constexpr int PER_HI = (NI + NW - 1) / NW, NBW = NEB / NW;
  static_assert(NEB % NW == 0, "whole expert blocks per wave");
  __shared__ __attribute__((aligned(1024))) bf16_t s_st[NS][(XR + WR) * 64];
  __shared__ float s_lg[XR][WR];
  const int lane = threadIdx.x % kWave, wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  // waves below NI % NW issue one load more per stage than the others
  const bool hi = NI % NW == 0 || wave < NI % NW;
  const int64_t t0 = (int64_t)blockIdx.x * XR;
  const int rows = (int)(T - t0 < XR ? T - t0 : XR);
  // rows past the tokens or the experts are past num_records and read zeros
  // (d < 2^22, checked on the host, keeps every byte count below 2^31)
  const __amdgpu_buffer_rsrc_t x_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(x + t0 * d), (short)0, rows * d * 2, kBufferConfig);
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)w, (short)0, E * d * 2, kBufferConfig);
  // load p of this wave fills stacked rows 8 i .. 8 i + 7 (x rows first), i = wave + NW p
  uint32_t voff[PER_HI];
  bool from_x[PER_HI];
#pragma unroll
  for (int p = 0; p < PER_HI; ++p) {
    const int r = 8 * (wave + NW * p) + lane / 8, c = (lane & 7) ^ (r & 7);
    from_x[p] = r < XR;
    const int src_row = r < XR ? r : (r - XR < WR ? r - XR : 0);
    voff[p] = (uint32_t)(src_row * d * 2 + c * 16);
  }
  const int n_stages = d / 64;
  auto issue = [&](int st) {
    const uint32_t base = lds_address(&s_st[st % NS][0]);
#pragma unroll
    for (int p = 0; p < PER_HI; ++p)
      if (p < PER_HI - 1 || hi) dma16(from_x[p] ? x_rsrc : w_rsrc, base + (wave + NW * p) * 1024, voff[p] + st * 128);
  };
  f32x4 acc[TG][NBW];
#pragma unroll
  for (int g = 0; g < TG; ++g)
#pragma unroll
    for (int b = 0; b < NBW; ++b) acc[g][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int st = 0; st < NS - 1 && st < n_stages; ++st) issue(st);
  const int rr = lane % 16, q = lane / 16;
  for (int st = 0; st < n_stages; ++st) {
    // this wave's loads of stage st have landed once at most the younger
    // stages' loads are outstanding; near the end fewer are, so wait for all
    if (st + NS - 2 < n_stages) {
      if (hi) wait_vmcnt<(NS - 2) * PER_HI>(); else wait_vmcnt<(NS - 2) * (PER_HI - 1)>();
    } else {
      wait_vmcnt<0>();
    }
    stage_barrier();  // stage st visible to all; every wave is done with stage st - 1
    if (st + NS - 1 < n_stages) issue(st + NS - 1);
    const bf16_t* buf = &s_st[st % NS][0];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = 4 * h + q;  // chunk of 8 columns this lane supplies to step h
      bf16x8 xf[TG], wf[NBW];
#pragma unroll
      for (int g = 0; g < TG; ++g) {
        const int r = 16 * g + rr;
        xf[g] = *(const bf16x8*)(buf + r * 64 + (c ^ (r & 7)) * 8);
      }
#pragma unroll
      for (int b = 0; b < NBW; ++b) {
        const int r = XR + 16 * (wave + NW * b) + rr;
        wf[b] = *(const bf16x8*)(buf + r * 64 + (c ^ (r & 7)) * 8);
      }
#pragma unroll
      for (int g = 0; g < TG; ++g)
#pragma unroll
        for (int b = 0; b < NBW; ++b)
          acc[g][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[b], xf[g], acc[g][b], 0, 0, 0);
    }
  }
  // lane l holds experts 16 (wave + NW b) + 4 (l / 16) .. +3 of token 16 g + l % 16
#pragma unroll
  for (int g = 0; g < TG; ++g)
#pragma unroll
    for (int b = 0; b < NBW; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) s_lg[16 * g + rr][16 * (wave + NW * b) + 4 * q + v] = acc[g][b][v];
  __syncthreads();
  if (logits)
    for (int i = threadIdx.x; i < rows * E; i += NW * kWave) logits[t0 * E + i] = s_lg[i / E][i % E];
  // all XR tokens at once, G lanes each: the shuffle chains of the k picks
  // are short and run for every token of the workgroup together
  constexpr int G = NW * kWave / XR, S = WR / G;
  static_assert(G >= 8 && G * S == WR, "routing lanes");
  const int tl = (int)threadIdx.x / G;
  float lg[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int e = s * G + (int)threadIdx.x % G;
    lg[s] = (tl < rows && e < E) ? s_lg[tl][e] : 0.f;
  }
  route_token<G, S>(lg, t0 + tl, tl < rows, E, k, topk_idx, topk_w);
}

template <int NEB, int TG, int NS, int NW>
hipError_t launch_staged(const bf16_t* x, const bf16_t* w, int T, int d, int E, int k, float* logits, int32_t* idx,
                         float* wt, hipStream_t s) {
  k_route_project_staged<NEB, TG, NS, NW><<<(unsigned)ceil_div(T, 16 * TG), NW * kWave, 0, s>>>(
      x, w, T, d, E, k, logits, idx, wt);
  return hipGetLastError();
}

template <typename Elem>
hipError_t dispatch_project(const Elem* x, const Elem* w, int T, int d, int E, int k, float* logits, int32_t* idx,
                            float* wt, hipStream_t s) {
  if (E <= 8) return launch_project<Elem, 8, 1, 1>(x, w, T, d, E, k, logits, idx, wt, s);
  if (E <= 16) return launch_project<Elem, 16, 1, 1>(x, w, T, d, E, k, logits, idx, wt, s);
  if (E <= 32) return launch_project<Elem, 32, 1, 2>(x, w, T, d, E, k, logits, idx, wt, s);
  if constexpr (sizeof(Elem) == 2) {
    // stage shapes measured best on MI355X: 32 tokens per workgroup once
    // there are enough of them to fill the CUs, else 16 with 8 waves
    if (E <= 64) return launch_staged<4, 1, 4, 4>(x, w, T, d, E, k, logits, idx, wt, s);
    if (E <= 128) {
      if (T >= 4096) return launch_staged<8, 2, 4, 4>(x, w, T, d, E, k, logits, idx, wt, s);
      return launch_staged<8, 1, 4, 8>(x, w, T, d, E, k, logits, idx, wt, s);
    }
    return launch_staged<16, 1, 4, 8>(x, w, T, d, E, k, logits, idx, wt, s);
  } else {
    if (E <= 64) return launch_project<Elem, 64, 1, 4>(x, w, T, d, E, k, logits, idx, wt, s);
    if (E <= 128) return launch_project<Elem, 64, 2, 8>(x, w, T, d, E, k, logits, idx, wt, s);
    return launch_project<Elem, 64, 4, 16>(x, w, T, d, E, k, logits, idx, wt, s);
  }
}

}  // namespace

hipError_t launch_route_project_bf16(const bf16_t* x, const bf16_t* w_router, int T, int d, int E, int k,
                                    float* logits, int32_t* topk_idx, float* topk_w, hipStream_t s) {
  return dispatch_project<bf16_t>(x, w_router, T, d, E, k, logits, topk_idx, topk_w, s);
}

hipError_t launch_route_project_f32(const float* x, const float* w_router, int T, int d, int E, int k,
                                   float* logits, int32_t* topk_idx, float* topk_w, hipStream_t s) {
  return dispatch_project<float>(x, w_router, T, d, E, k, logits, topk_idx, topk_w, s);
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* topk_idx,
                             float* topk_w, hipStream_t s) {
  if (E <= 8) return launch<8, 1>(logits, T, E, k, topk_idx, topk_w, s);
  if (E <= 16) return launch<16, 1>(logits, T, E, k, topk_idx, topk_w, s);
  if (E <= 32) return launch<32, 1>(logits, T, E, k, topk_idx, topk_w, s);
  if (E <= 64) return launch<64, 1>(logits, T, E, k, topk_idx, topk_w, s);
  // 65-128 experts: groups of 16 lanes holding 8 logits each (four tokens a
  // wave): each pick is a local maximum over a lane's keys and four shuffle
  // steps, instead of six over a whole wave per token
  if (E <= 128) return launch<16, 8>(logits, T, E, k, topk_idx, topk_w, s);
  return launch<64, 4>(logits, T, E, k, topk_idx, topk_w, s);
}

}  // namespace tre
