// grouped_ffn.hip -- each expert's SwiGLU feed-forward over its own rows.
//
// "Tensor parallelism for inference" (Hugging Face Transformers docs),
// section "Packed strategies": the gate and up projections are one packed
// [E, d, 2I] weight applied as x @ W and split in two along the last
// dimension, gate half first.  The down projection (down_proj, "Expert
// parallelism", section "Overriding plans") is [E, I, d] in the same
// orientation.  Rows of expert e are [offsets[e], offsets[e+1]) of x_perm:
//   H[r] = silu(x_perm[r] @ Wgu[e][:, :I]) * (x_perm[r] @ Wgu[e][:, I:])
//   Y[r] = H[r] @ Wd[e]
//
// bf16 path (MFMA, gfx950):
//   * One kernel template, two instances: gate/up with the SwiGLU epilogue
//     (output H, bf16) and down (output Y, bf16); float32 accumulation in
//     v_mfma_f32_32x32x16_bf16.
//   * Workgroup tile 128 rows x 256 weight columns x 64 k, 4 waves in 2 x 2,
//     each wave 64 x 128 (2 x 4 MFMA tiles).  For gate/up the 256 columns
//     are 128 gate columns and the matching 128 up columns, and every wave
//     holds gate column j and up column j in the same lane, so the SwiGLU
//     epilogue is elementwise in registers.
//   * Activation tile [128][64] and weight tile [64][256] staged in LDS with
//     padded rows; the next k-stage is prefetched into registers while the
//     current one is multiplied.  Activation rows are k-contiguous and read
//     with ds_read_b128; weight rows are n-contiguous and read with the
//     gfx950 transposing ds_read_b64_tr_b16, two per operand.
//   * Persistent grid: each workgroup derives the tile list from the device
//     offsets (no host synchronisation), walks it round-robin, and tiles are
//     ordered expert, then column tile, then row tile so that the row tiles
//     sharing a weight slice run at the same time on one XCD's L2.
// float32 path: plain per-element dot products (small, exact-ish, for the
// float32 workloads).
#include "common.hpp"

namespace tre {
namespace {

constexpr int BM = 128;          // rows per tile
constexpr int BK = 64;           // k per stage
constexpr int BNB = 256;         // weight columns per tile
constexpr int NTHR = 256;        // 4 waves
constexpr int A_LD = BK + 8;     // 144-byte rows: ds_read_b128 of 16 rows hits distinct banks
constexpr int B_LD = BNB + 32;   // 576-byte rows: 4 consecutive k-rows fall on distinct banks
constexpr int kXcd = 8;          // XCDs per MI355X; workgroups are dealt round-robin over them

typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ bf16x8 lds_read_b_operand(const bf16_t* p0, const bf16_t* p1) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1);
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) s_wave[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NTHR / kWave; ++w) {
    before += (w < wave) ? s_wave[w] : 0;
    all += s_wave[w];
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// A: [max_rows, K] activations; W: [E, K, ldw] weights; Out: [max_rows, N].
// SWIGLU: N = I, ldw = 2I, a tile covers output columns [n0, n0 + 128).
// plain:  N = d, ldw = d,  a tile covers output columns [n0, n0 + 256).
template <bool SWIGLU>
__global__ __launch_bounds__(NTHR, 1) void k_grouped_gemm_bf16(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ offsets, int64_t max_rows, int E, int K,
    int N, int ldw, const bf16_t* __restrict__ W, bf16_t* __restrict__ Out, int n_tiles) {
  __shared__ __attribute__((aligned(16))) bf16_t As[BM * A_LD];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[BK * B_LD];
  __shared__ int s_start[kMaxExperts];
  __shared__ int s_mt[kMaxExperts];
  __shared__ int64_t s_lo[kMaxExperts];
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_wave[NTHR / kWave];

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave / 2, wn = wave % 2;

  // ---- tile list from the device offsets ----
  int mt = 0;
  if (tid < E) {
    const int64_t lo = clampi<int64_t>(offsets[tid], 0, max_rows);
    const int64_t hi = clampi<int64_t>(offsets[tid + 1], lo, max_rows);
    s_lo[tid] = lo;
    s_cnt[tid] = (int)(hi - lo);
    mt = (int)ceil_div(hi - lo, BM);
    s_mt[tid] = mt;
  }
  int total_mt = 0;
  const int start = block_exclusive_scan(mt, s_wave, &total_mt);
  if (tid < E) s_start[tid] = start;
  __syncthreads();
  const int64_t total_tiles = (int64_t)total_mt * n_tiles;

  // XCD-aware order: workgroups b, b+8, b+16 ... share an XCD; give them
  // consecutive tiles.
  const int G = gridDim.x;
  const int vb = (blockIdx.x % kXcd) * (G / kXcd) + blockIdx.x / kXcd;

  // per-thread constant parts of the global->LDS copies
  const int a_chunk = tid % 8, a_row0 = tid / 8;     // 8 x 16 B per 64-k row, 32 rows per pass
  const int b_chunk = tid % 32, b_row0 = tid / 32;   // 32 x 16 B per 256-col row, 8 rows per pass
  const int b_tcol = b_chunk * 8;                     // tile column of this thread's chunk

  for (int64_t v = vb; v < total_tiles; v += G) {
    // expert: the last one whose first tile is <= v (empty experts own no tiles)
    int lo_e = 0, hi_e = E - 1;
    while (lo_e < hi_e) {
      const int mid = (lo_e + hi_e + 1) / 2;
      if ((int64_t)s_start[mid] * n_tiles <= v) lo_e = mid; else hi_e = mid - 1;
    }
    const int e = lo_e;
    const int64_t local = v - (int64_t)s_start[e] * n_tiles;
    const int e_mt = s_mt[e];
    const int nt = (int)(local / e_mt);
    const int mtile = (int)(local % e_mt);
    const int64_t row0 = s_lo[e] + (int64_t)mtile * BM;
    const int rows = min(BM, s_cnt[e] - mtile * BM);
    const int n0 = nt * (SWIGLU ? BNB / 2 : BNB);
    const bf16_t* Wb = W + (int64_t)e * K * ldw;

    // this thread's weight column (global) and whether it exists
    int b_gcol;
    bool b_ok;
    if (SWIGLU) {
      const int hc = n0 + (b_tcol % (BNB / 2));
      b_ok = hc < N;
      b_gcol = (b_tcol < BNB / 2) ? hc : N + hc;
    } else {
      b_gcol = n0 + b_tcol;
      b_ok = b_gcol < N;
    }

    u32x4 ra[4], rb[8];
    auto gload = [&](int kt) {
      const int kb = kt * BK;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int r = a_row0 + 32 * p;
        ra[p] = (r < rows) ? *(const u32x4*)(A + (row0 + r) * K + kb + a_chunk * 8) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int kr = b_row0 + 8 * p;
        rb[p] = b_ok ? *(const u32x4*)(Wb + (int64_t)(kb + kr) * ldw + b_gcol) : u32x4{0, 0, 0, 0};
      }
    };
    auto lstore = [&]() {
#pragma unroll
      for (int p = 0; p < 4; ++p) *(u32x4*)&As[(a_row0 + 32 * p) * A_LD + a_chunk * 8] = ra[p];
#pragma unroll
      for (int p = 0; p < 8; ++p) *(u32x4*)&Bs[(b_row0 + 8 * p) * B_LD + b_tcol] = rb[p];
    };

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    // tile column base of this wave's MFMA column tile j
    auto col_base = [&](int j) {
      if (SWIGLU) return (j < 2) ? 64 * wn + 32 * j : BNB / 2 + 64 * wn + 32 * (j - 2);
      return 128 * wn + 32 * j;
    };

    const int g = lane / 16, L = lane % 16;
    const int nk = K / BK;
    gload(0);
    lstore();
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        bf16x8 a[2], b[4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          a[i] = *(const bf16x8*)&As[(64 * wm + 32 * i + lane % 32) * A_LD + ks * 16 + (lane / 32) * 8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int krow = ks * 16 + (g / 2) * 8 + L / 4;
          const int col = col_base(j) + (g % 2) * 16 + 4 * (L % 4);
          b[j] = lds_read_b_operand(&Bs[krow * B_LD + col], &Bs[(krow + 4) * B_LD + col]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
      __syncthreads();
      if (kt + 1 < nk) {
        lstore();
        __syncthreads();
      }
    }

    // ---- epilogue: lane holds column (lane % 32) of each 32x32 tile, rows
    // (q / 4) * 8 + (lane / 32) * 4 + q % 4 ----
    const int lc = lane % 32;
    if (SWIGLU) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int c = n0 + 64 * wn + 32 * j + lc;
          if (c >= N) continue;
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int r = 64 * wm + 32 * i + (q / 4) * 8 + (lane / 32) * 4 + q % 4;
            if (r < rows) {
              const float gt = acc[i][j][q], up = acc[i][j + 2][q];
              const float h = gt / (1.f + __expf(-gt)) * up;
              Out[(row0 + r) * N + c] = f32_to_bf16(h);
            }
          }
        }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = n0 + 128 * wn + 32 * j + lc;
          if (c >= N) continue;
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int r = 64 * wm + 32 * i + (q / 4) * 8 + (lane / 32) * 4 + q % 4;
            if (r < rows) Out[(row0 + r) * N + c] = f32_to_bf16(acc[i][j][q]);
          }
        }
    }
  }
}

int g_num_cus = 0;

int num_cus() {
  if (g_num_cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      g_num_cus = n;
    else
      g_num_cus = 256;
  }
  return g_num_cus;
}

// Workgroups for a persistent launch: no more than the tiles that can exist,
// no more than one per CU, a multiple of the XCD count.
int persistent_grid(int64_t max_rows, int E, int n_tiles) {
  const int64_t max_mt = max_rows / BM + (int64_t)(E < max_rows ? E : max_rows);
  const int64_t want = max_mt * n_tiles;
  const int64_t cap = (int64_t)num_cus();
  const int64_t g = want < cap ? want : cap;
  return (int)round_up(g < 1 ? 1 : g, kXcd);
}

// ---- float32 path -----------------------------------------------------------

__device__ __forceinline__ int expert_of_row(const int32_t* offsets, int E, int64_t r) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (offsets[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void k_ffn_gate_up_f32(const float* __restrict__ x, const int32_t* __restrict__ offsets,
                                                         int64_t max_rows, int E, int d, int I,
                                                         const float* __restrict__ wgu, float* __restrict__ h) {
  const int64_t r = blockIdx.x;
  const int c = blockIdx.y * blockDim.x + threadIdx.x;
  const int64_t n_rows = clampi<int64_t>(offsets[E], 0, max_rows);
  if (r >= n_rows || c >= I) return;
  const int e = expert_of_row(offsets, E, r);
  const float* xr = x + r * d;
  const float* we = wgu + (int64_t)e * d * 2 * I;
  float g = 0.f, u = 0.f;
  for (int q = 0; q < d; ++q) {
    const float xv = xr[q];
    g = fmaf(xv, we[(int64_t)q * 2 * I + c], g);
    u = fmaf(xv, we[(int64_t)q * 2 * I + I + c], u);
  }
  h[r * I + c] = g / (1.f + expf(-g)) * u;
}

__global__ __launch_bounds__(256) void k_ffn_down_f32(const float* __restrict__ h, const int32_t* __restrict__ offsets,
                                                      int64_t max_rows, int E, int d, int I,
                                                      const float* __restrict__ wd, float* __restrict__ y) {
  const int64_t r = blockIdx.x;
  const int c = blockIdx.y * blockDim.x + threadIdx.x;
  const int64_t n_rows = clampi<int64_t>(offsets[E], 0, max_rows);
  if (r >= n_rows || c >= d) return;
  const int e = expert_of_row(offsets, E, r);
  const float* hr = h + r * I;
  const float* we = wd + (int64_t)e * I * d;
  float acc = 0.f;
  for (int q = 0; q < I; ++q) acc = fmaf(hr[q], we[(int64_t)q * d + c], acc);
  y[r * d + c] = acc;
}

}  // namespace

hipError_t launch_grouped_ffn_bf16(const bf16_t* x_perm, const int32_t* expert_offsets, int64_t max_rows,
                                   int E, int d, int I, const bf16_t* w_gate_up, const bf16_t* w_down,
                                   bf16_t* h, bf16_t* y_perm, hipStream_t s) {
  const int nt1 = (int)ceil_div(I, BNB / 2);
  k_grouped_gemm_bf16<true><<<persistent_grid(max_rows, E, nt1), NTHR, 0, s>>>(
      x_perm, expert_offsets, max_rows, E, d, I, 2 * I, w_gate_up, h, nt1);
  const int nt2 = (int)ceil_div(d, BNB);
  k_grouped_gemm_bf16<false><<<persistent_grid(max_rows, E, nt2), NTHR, 0, s>>>(
      h, expert_offsets, max_rows, E, I, d, d, w_down, y_perm, nt2);
  return hipGetLastError();
}

hipError_t launch_grouped_ffn_f32(const float* x_perm, const int32_t* expert_offsets, int64_t max_rows, int E,
                                  int d, int I, const float* w_gate_up, const float* w_down, float* h,
                                  float* y_perm, hipStream_t s) {
  dim3 g1((unsigned)max_rows, (unsigned)ceil_div(I, 256));
  k_ffn_gate_up_f32<<<g1, 256, 0, s>>>(x_perm, expert_offsets, max_rows, E, d, I, w_gate_up, h);
  dim3 g2((unsigned)max_rows, (unsigned)ceil_div(d, 256));
  k_ffn_down_f32<<<g2, 256, 0, s>>>(h, expert_offsets, max_rows, E, d, I, w_down, y_perm);
  return hipGetLastError();
}

}  // namespace tre
