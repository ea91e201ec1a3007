// common.hpp -- shared device helpers and internal launcher declarations of
// the gfx950 MoE library.  Not part of the public ABI (include/moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tre {

constexpr int kWave = 64;      // CDNA wavefront width
constexpr int kMaxExperts = 256;

typedef uint16_t bf16_t;  // bfloat16 bit pattern in memory
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

// Two floats rounded to nearest even and packed, lo in bits [15:0]: one
// v_cvt_pk_bf16_f32 (a scalar conversion per value followed by a shift and an
// OR costs three more instructions).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Device-side contract checks.  The release library clamps every value it
// reads on the device (expert ids, offsets, row indices) to the buffers it
// indexes, so bad input gives bad output but never an out-of-range access.
// Built with MOE_DEVICE_CHECKS (libmoe_debug.so), the kernels also stop at
// the first value outside its contract, with a trap (no message: a printf
// call inside the grouped GEMM's loop would cost it its scalar registers).
// Only valid input may be given to that build.
#ifdef MOE_DEVICE_CHECKS
#define MOE_DCHECK(cond) \
  do {                   \
    if (!(cond)) __builtin_trap(); \
  } while (0)
#else
#define MOE_DCHECK(cond) ((void)0)
#endif

template <typename T>
__device__ __forceinline__ T clampi(T v, T lo, T hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ constexpr int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// ---- loads that write LDS directly (the GEMM and the router projection) ----

// Buffer descriptor word 3 for raw (untyped) buffer loads on CDNA.  A load at
// a byte offset past num_records returns zeros.
constexpr int kBufferConfig = 0x00020000;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  // vmcnt in bits [3:0] and [15:14]; expcnt (7) and lgkmcnt (15) not waited on
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// A wave-uniform pointer, marked as such (both halves through readfirstlane).
__device__ __forceinline__ void* uniform_ptr(const void* p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  return (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// LDS (address space 3) byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One wave-wide 16-byte-per-lane buffer load written straight to LDS at
// lds_base + 16 * lane.  Issued as inline assembly so that the compiler does
// not wait on it conservatively before unrelated LDS reads; completion is
// tracked explicitly with wait_vmcnt, visibility with a workgroup barrier.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_base, uint32_t voffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voffset), "s"(rsrc)
               : "memory");
}

// The same load with a scalar byte offset added to the lane offset: a loop
// that walks k-stages advances one scalar register instead of recomputing
// every lane's offset.  voffset + soffset must stay inside the buffer for
// the lanes that load (lanes parked past num_records by voffset alone still
// read zeros).
__device__ __forceinline__ void dma16s(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_base, uint32_t voffset,
                                       uint32_t soffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_base), "v"(voffset), "s"(rsrc), "s"(soffset)
               : "memory");
}

// The same load marked non-temporal (the nt cache policy): for a stream
// read once, so that it does not push data that will be read again out of
// L2.
__device__ __forceinline__ void dma16s_nt(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_base, uint32_t voffset,
                                          uint32_t soffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
               :
               : "s"(lds_base), "v"(voffset), "s"(rsrc), "s"(soffset)
               : "memory");
}

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// MFMA operand (32 rows x 16 k, lane l: row l % 32, k 8 (l / 32) .. +7) from
// an LDS tile stored k-row by k-row (rows of the operand contiguous): two
// transposing 64-bit reads, at k-rows kr and kr + 4 of the lane's column.
__device__ __forceinline__ bf16x8 lds_read_b_operand(const bf16_t* p0, const bf16_t* p1) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1);
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Workgroup barrier that neither the scheduler nor the compiler's memory
// model moves work across, and that does not drain outstanding LDS-writing
// loads the way __syncthreads() does.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  compiler_fence();
  __builtin_amdgcn_s_barrier();
  compiler_fence();
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier after this wave's LDS accesses have completed, without
// waiting for its global stores (which __syncthreads() also drains): for
// loops that share only LDS between their steps and stream results out.
__device__ __forceinline__ void lds_barrier() {
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

// ---- launchers (each returns hipGetLastError() of its launches) ----------

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* topk_idx,
                             float* topk_w, hipStream_t s);
// router projection logits = x @ w_router^T (w_router [E, d]) fused with the
// routing above; logits (float32 [T, E]) written only when non-null
hipError_t launch_route_project_bf16(const bf16_t* x, const bf16_t* w_router, int T, int d, int E, int k,
                                    float* logits, int32_t* topk_idx, float* topk_w, hipStream_t s);
hipError_t launch_route_project_f32(const float* x, const float* w_router, int T, int d, int E, int k,
                                   float* logits, int32_t* topk_idx, float* topk_w, hipStream_t s);

// Stable grouping of pairs by expert: per-chunk expert counts (chunks of
// kPermuteChunk pairs), then the scatter, which also scans the counts when
// there are few enough of them (else a one-workgroup scan runs between).
constexpr int kPermuteChunk = 512;
size_t permute_index_workspace(int64_t P, int E);
// sched (optional): kSchedWords words that the grouping also sets to zero,
// the tile counters of the grouped products that follow it.
// row_w (optional): row_w[pair_row[p]] = pair_w[p], each grouped row's
// routing weight.
hipError_t launch_permute_index(const int32_t* pair_expert, int64_t P, int k, int E,
                                int32_t* row_token, int32_t* pair_row, int32_t* expert_offsets,
                                void* ws, hipStream_t s, int32_t* sched = nullptr,
                                const float* pair_w = nullptr, float* row_w = nullptr);
// x_perm[pair_row[t*k+j]] = x[t] for every pair with a row (token-major:
// each row of x is read once); row_bytes % 16 == 0.
hipError_t launch_move_rows(const void* x, int64_t T, int k, int64_t row_bytes, const int32_t* pair_row,
                            int64_t max_rows, void* x_perm, hipStream_t s);
// The grouping (as launch_permute_index, without row weights) and the row move
// (as launch_move_rows into P = T * k rows) together: for more than a
// decode-sized batch, the scatter and the move are one kernel.
hipError_t launch_permute_rows(const int32_t* pair_expert, int64_t T, int k, int E, int32_t* row_token,
                               int32_t* pair_row, int32_t* expert_offsets, void* ws, hipStream_t s, int32_t* sched,
                               const void* x, int64_t row_bytes, void* x_perm);

// Tile counters of the grouped products (zero before each product that uses
// one): the gate/up product's at sched[0], the down product's at
// sched[kSchedDown] (64 bytes apart).  With a counter, the ping-pong kernel
// hands out its last round and a half of tiles in order to whichever
// workgroup is free; without, every tile is dealt round-robin.
constexpr int kSchedDown = 16;
constexpr int kSchedWords = 32;
hipError_t launch_sched_reset(int32_t* sched, hipStream_t s);

// Grouped SwiGLU feed-forward, as two launches (gate/up + SwiGLU, then down).
// h: [max_rows, I] of the activation type.
// With row_token, activation row r is row row_token[r] of x ([x_rows, d]):
// the permutation's row move happens inside the load.  Without, x is x_perm.
// wtiled: the weights are in the column-tiled layout of launch_tile_weights_bf16.
hipError_t launch_gate_up_bf16(const bf16_t* x, const int32_t* expert_offsets, int64_t max_rows, int E, int d,
                               int I, const bf16_t* w_gate_up, bf16_t* h, hipStream_t s,
                               const int32_t* row_token = nullptr, int64_t x_rows = 0, int32_t* sched = nullptr,
                               bool wtiled = false);
// split_ws (optional, split_workspace(max_rows, E, d, I) bytes, float32):
// with few rows the down projection's k-stages are split over more
// workgroups and summed there in a fixed order (deterministic); with many,
// the tiles of a last, partial round of 256-row tiles are (the split tail).
size_t split_workspace(int64_t max_rows, int E, int d, int I);
// One pair per token (k = 1): the down projection can write the layer output
// itself, out[row_token[r]] = row_w[r] * bf16(y[r]) rounded to bf16 (what
// the combine computes for a single pair), from its 256-row tiles or its
// k-split sum; down_scatters says whether the shape takes one of those
// paths.  Rows of tokens without a pair are not written.
struct DownScatter {
  bf16_t* out;               // [T, d]
  const int32_t* row_token;  // grouped row -> token
  const float* row_w;        // grouped row -> routing weight
  int64_t T;
};
bool down_scatters(int64_t max_rows, int E, int d, int I, bool have_split_ws);
// scatter_tiles: grouped rows y, but in the tiles the scatter path (sc) would
// use (no tall tiles), so that a split tail cuts the same tiles and the rows
// equal, bit for bit, what the scatter path computes.
hipError_t launch_down_bf16(const bf16_t* h, const int32_t* expert_offsets, int64_t max_rows, int E, int d,
                            int I, const bf16_t* w_down, bf16_t* y_perm, hipStream_t s, float* split_ws = nullptr,
                            int32_t* sched = nullptr, const DownScatter* sc = nullptr, bool scatter_tiles = false,
                            bool wtiled = false);
hipError_t launch_gate_up_f32(const float* x_perm, const int32_t* expert_offsets, int64_t max_rows, int E,
                              int d, int I, const float* w_gate_up, float* h, hipStream_t s);
hipError_t launch_down_f32(const float* h, const int32_t* expert_offsets, int64_t max_rows, int E, int d,
                           int I, const float* w_down, float* y_perm, hipStream_t s);
hipError_t launch_grouped_ffn_bf16(const bf16_t* x_perm, const int32_t* expert_offsets,
                                   int64_t max_rows, int E, int d, int I, const bf16_t* w_gate_up,
                                   const bf16_t* w_down, bf16_t* h, bf16_t* y_perm, hipStream_t s,
                                   float* split_ws = nullptr, int32_t* sched = nullptr, bool wtiled = false);
// Both expert weights in the column-tiled layout the forward products can
// read instead (same sizes; a permutation of the elements): each expert's
// weight stored as one [K][width] block per 256-column tile of the product,
// for gate/up 128 gate columns followed by the same 128 up columns.
hipError_t launch_tile_weights_bf16(const bf16_t* w_gate_up, const bf16_t* w_down, int E, int d, int I,
                                    bf16_t* wgu_tiled, bf16_t* wd_tiled, hipStream_t s);
hipError_t launch_grouped_ffn_f32(const float* x_perm, const int32_t* expert_offsets,
                                  int64_t max_rows, int E, int d, int I, const float* w_gate_up,
                                  const float* w_down, float* h, float* y_perm, hipStream_t s);

hipError_t launch_combine_bf16(const bf16_t* y_perm, int64_t max_rows, const int32_t* pair_row,
                               const float* pair_w, int64_t T, int k, int d, bf16_t* out,
                               hipStream_t s);
hipError_t launch_combine_f32(const float* y_perm, int64_t max_rows, const int32_t* pair_row,
                              const float* pair_w, int64_t T, int k, int d, float* out,
                              hipStream_t s);
// (pair_w == nullptr: every weight is 1 -- the backward's sum of a token's row gradients)
// k = 1: out[t] = 0 for every token whose pair has no grouped row (pair_row
// outside [0, max_rows)); the other rows are left alone
hipError_t launch_zero_unrouted_bf16(const int32_t* pair_row, int64_t max_rows, int64_t T, int d, bf16_t* out,
                                     hipStream_t s);

// ---- backward (bf16) ----
// forward gate/up that also keeps the pre-activations: gu [max_rows, 2I] = [x Wg | x Wu]
hipError_t launch_gate_up_save_bf16(const bf16_t* x, const int32_t* expert_offsets, int64_t max_rows, int E, int d,
                                    int I, const bf16_t* w_gate_up, bf16_t* h, bf16_t* gu, hipStream_t s,
                                    const int32_t* row_token = nullptr, int64_t x_rows = 0,
                                    int32_t* sched = nullptr);
// dy[pair_row[p]] = w_p dout[t]; dw[p] = <dout[t], y_perm[pair_row[p]]>; dlogits (when non-null) through
// the renormalised softmax of the selected logits
hipError_t launch_combine_bwd_bf16(const bf16_t* dout, const bf16_t* y_perm, int64_t max_rows,
                                  const int32_t* pair_row, const float* pair_w, const int32_t* topk_idx, int64_t T,
                                  int k, int d, int E, bf16_t* dy_perm, float* dw, float* dlogits, hipStream_t s);
// dgu = [dg | du] from dh = dy Wd^T and the saved gu
hipError_t launch_down_dgrad_swiglu_bf16(const bf16_t* dy, const int32_t* expert_offsets, int64_t max_rows, int E,
                                         int d, int I, const bf16_t* w_down, const bf16_t* gu, bf16_t* dgu,
                                         hipStream_t s);
// dx_perm = dgu Wgu^T
hipError_t launch_gate_up_dgrad_bf16(const bf16_t* dgu, const int32_t* expert_offsets, int64_t max_rows, int E,
                                     int d, int I, const bf16_t* w_gate_up, bf16_t* dx_perm, hipStream_t s);
// p[0, n) = 0 by a plain kernel (no memset node when captured in a graph); n % 8 == 0
hipError_t launch_zero_bf16(bf16_t* p, int64_t n, hipStream_t s);
// dW[e] [M, N] = sum over the rows r of expert e of a[r][:M]^T b[r][:N]
hipError_t launch_wgrad_bf16(const bf16_t* a, int lda, int M, const bf16_t* b, int ldb, int N,
                             const int32_t* expert_offsets, int64_t max_rows, int E, bf16_t* dw, hipStream_t s);

// ---- backward (float32): the same steps on float32 rows and weights ----
hipError_t launch_gate_up_save_f32(const float* x_perm, const int32_t* expert_offsets, int64_t max_rows, int E,
                                   int d, int I, const float* w_gate_up, float* h, float* gu, hipStream_t s);
hipError_t launch_combine_bwd_f32(const float* dout, const float* y_perm, int64_t max_rows,
                                  const int32_t* pair_row, const float* pair_w, const int32_t* topk_idx, int64_t T,
                                  int k, int d, int E, float* dy_perm, float* dw, float* dlogits, hipStream_t s);
hipError_t launch_down_dgrad_swiglu_f32(const float* dy, const int32_t* expert_offsets, int64_t max_rows, int E,
                                        int d, int I, const float* w_down, const float* gu, float* dgu,
                                        hipStream_t s);
hipError_t launch_gate_up_dgrad_f32(const float* dgu, const int32_t* expert_offsets, int64_t max_rows, int E,
                                    int d, int I, const float* w_gate_up, float* dx_perm, hipStream_t s);
hipError_t launch_wgrad_f32(const float* a, int lda, int M, const float* b, int ldb, int N,
                            const int32_t* expert_offsets, int64_t max_rows, int E, float* dw, hipStream_t s);

}  // namespace tre
