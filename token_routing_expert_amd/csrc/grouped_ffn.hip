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
// bf16 path (MFMA, gfx950), one kernel template with two instances: gate/up
// with the SwiGLU epilogue (output H) and down (output Y), both bf16 with
// float32 accumulation in v_mfma_f32_32x32x16_bf16:
//   * workgroup tile 128 rows x 256 weight columns, 4 waves in 2 x 2, each
//     wave 64 x 128 (2 x 4 MFMA tiles); for gate/up the 256 columns are 128
//     gate columns and the matching 128 up columns, and each wave holds gate
//     column j and up column j in the same lane, so SwiGLU is elementwise in
//     registers;
//   * k-stages of 32 stream through a ring of three LDS buffers filled by
//     buffer loads that write LDS directly; two workgroups per CU, so one
//     workgroup's waits overlap the other's multiplications;
//   * weight rows are n-contiguous and reach the MFMA through the gfx950
//     transposing LDS read ds_read_b64_tr_b16;
//   * persistent grid: each workgroup derives the tile list from the device
//     offsets (no host synchronisation) and walks it round-robin; tiles are
//     ordered expert, then column tile, then row tile, and consecutive tiles
//     go to workgroups of one XCD, so the row tiles that share a weight slice
//     run together on one L2.
// float32 path: plain per-element dot products (small, for the float32
// workloads).
#include "common.hpp"

namespace tre {
namespace {

constexpr int NTHR = 256;        // 4 waves per workgroup
constexpr int kXcd = 8;          // XCDs per MI355X; workgroups are dealt round-robin over them
// Buffer descriptor word 3 for raw (untyped) buffer loads on CDNA, and byte
// offsets that are always past num_records (a load there returns zeros).
constexpr int kBufferConfig = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ bf16x8 lds_read_b_operand(const bf16_t* p0, const bf16_t* p1) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1);
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

template <int NWAVES>
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
  for (int w = 0; w < NWAVES; ++w) {
    before += (w < wave) ? s_wave[w] : 0;
    all += s_wave[w];
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// ---------------------------------------------------------------------------
// The bf16 grouped GEMM.  Tiles stream through a ring of three LDS stages
// filled by buffer loads that write LDS directly (no staging registers):
// while stage s is multiplied, stages s+1 and s+2 are in flight.  One
// barrier per stage; each wave waits for its own loads of the stage (vmcnt)
// before the barrier, so after the barrier the whole stage is resident.
// LDS layouts are dense (a DMA instruction fills 1 KB contiguously) and
// XOR-swizzled instead of padded, so that the activation reads
// (ds_read_b128 of 16 consecutive rows) and the transposing weight reads (4
// consecutive k-rows x 32 bytes per 16-lane group) touch every bank once.
namespace dma {


template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  // vmcnt in bits [3:0] and [15:14]; expcnt (7) and lgkmcnt (15) not waited on
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS (address space 3) byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One wave-wide 16-byte-per-lane buffer load written straight to LDS at
// lds_base + 16 * lane.  Issued as inline assembly so that the compiler does
// not wait on it conservatively before unrelated LDS reads; completion is
// tracked explicitly with wait_vmcnt, visibility with the stage barrier.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t lds_base, uint32_t voffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voffset), "s"(rsrc)
               : "memory");
}

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Stage geometry for k-depth BK (64 or 32) and NJ MFMA column tiles per
// wave (BNB = 64 NJ weight columns per workgroup tile).  Activation rows hold
// BK elements (BK/8 chunks of 16 B); a DMA instruction fills 1 KB = RPI
// activation rows or BRPI weight rows.
template <int BK, int NJ, int WM>
struct Geo {
  static constexpr int WAVES = 2 * WM;                   // WM x 2 waves, each 64 rows x 32 NJ columns
  static constexpr int BM = 64 * WM;                     // rows per workgroup tile
  static constexpr int BNB = 64 * NJ;                    // weight columns per tile
  static constexpr int BROW = BNB * 2;                   // bytes per weight row in LDS
  static constexpr int BCPR = BROW / 16;                 // 16-byte chunks per weight row
  static constexpr int BRPI = 1024 / BROW;               // weight rows per DMA instruction
  static constexpr int CPR = BK / 8;                     // 16-byte chunks per activation row
  static constexpr int RPI = 1024 / (BK * 2);            // activation rows per DMA instruction
  static constexpr int A_BYTES = BM * BK * 2;
  static constexpr int B_BYTES = BK * BROW;
  static constexpr int A_INSTR = A_BYTES / 1024 / WAVES;  // per wave per stage
  static constexpr int B_INSTR = B_BYTES / 1024 / WAVES;
  static constexpr int PER_STAGE = A_INSTR + B_INSTR;
  // chunk c of activation row r sits in slot c ^ swz(r): 16 consecutive rows
  // read at one logical chunk land on 16 distinct bank groups
  static __device__ __forceinline__ int swz(int r) { return BK == 64 ? (r >> 1) & 7 : (r >> 2) & 3; }
  static __device__ __forceinline__ uint32_t a_byte(int r, int c) {
    return (uint32_t)(r * (BK * 2) + ((c ^ swz(r)) << 4));
  }
  // chunk c of weight k-row kr sits in slot c ^ (4 * (kr & 3)): the 4
  // consecutive k-rows x 32 bytes read by a 16-lane ds_read_b64_tr_b16 group
  // (and the neighbouring group's next 32 bytes) fall on distinct banks
  static __device__ __forceinline__ uint32_t b_byte(int kr, int c) {
    return (uint32_t)(kr * BROW + ((c ^ ((kr & 3) << 2)) << 4));
  }
};

template <bool SWIGLU, int BK, int OCC, int NJ, int WM>
__global__ __launch_bounds__(128 * WM, OCC) void k_grouped_gemm(const bf16_t* __restrict__ A, const int32_t* __restrict__ offsets,
                                                           int64_t max_rows, int E, int K, int N, int ldw,
                                                           const bf16_t* __restrict__ W, bf16_t* __restrict__ Out,
                                                           int n_tiles, const int32_t* __restrict__ row_token,
                                                           int64_t a_rows) {
  typedef Geo<BK, NJ, WM> GE;
  constexpr int BM = GE::BM, WAVES = GE::WAVES;
  constexpr int BNB = GE::BNB;
  constexpr int WCOL = 32 * NJ;       // weight columns per wave
  __shared__ __attribute__((aligned(1024))) char sA0[GE::A_BYTES];
  __shared__ __attribute__((aligned(1024))) char sA1[GE::A_BYTES];
  __shared__ __attribute__((aligned(1024))) char sA2[GE::A_BYTES];
  __shared__ __attribute__((aligned(1024))) char sB0[GE::B_BYTES];
  __shared__ __attribute__((aligned(1024))) char sB1[GE::B_BYTES];
  __shared__ __attribute__((aligned(1024))) char sB2[GE::B_BYTES];
  __shared__ int s_start[kMaxExperts];
  __shared__ int s_mt[kMaxExperts];
  __shared__ int64_t s_lo[kMaxExperts];
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_wave[WAVES];

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / 2, wn = wave % 2;
  const int g = lane / 16, L = lane % 16;

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
  const int start = block_exclusive_scan<WAVES>(mt, s_wave, &total_mt);
  if (tid < E) s_start[tid] = start;
  __syncthreads();
  const int64_t total_tiles = (int64_t)total_mt * n_tiles;
  const int G = gridDim.x;
  const int vb = (blockIdx.x % kXcd) * (G / kXcd) + blockIdx.x / kXcd;

  auto col_base = [&](int j) {
    if (SWIGLU) return (j < NJ / 2) ? (WCOL / 2) * wn + 32 * j : BNB / 2 + (WCOL / 2) * wn + 32 * (j - NJ / 2);
    return WCOL * wn + 32 * j;
  };

  for (int64_t v = vb; v < total_tiles; v += G) {
    int lo_e = 0, hi_e = E - 1;
    while (lo_e < hi_e) {
      const int mid = (lo_e + hi_e + 1) / 2;
      if ((int64_t)s_start[mid] * n_tiles <= v) lo_e = mid; else hi_e = mid - 1;
    }
    // every lane found the same tile; say so, so that its addresses and
    // buffer descriptors live in scalar registers
    const int e = __builtin_amdgcn_readfirstlane(lo_e);
    const int e_start = __builtin_amdgcn_readfirstlane(s_start[e]);
    const int e_mt = __builtin_amdgcn_readfirstlane(s_mt[e]);
    const int e_cnt = __builtin_amdgcn_readfirstlane(s_cnt[e]);
    const int64_t e_lo = s_lo[e];
    const int64_t e_row0 = ((int64_t)__builtin_amdgcn_readfirstlane((int)(e_lo >> 32)) << 32) |
                           (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)e_lo);
    const int64_t local = v - (int64_t)e_start * n_tiles;
    const int nt = (int)(local / e_mt);
    const int mtile = (int)(local % e_mt);
    const int64_t row0 = e_row0 + (int64_t)mtile * BM;
    const int rows = min(BM, e_cnt - mtile * BM);
    const int n0 = nt * (SWIGLU ? BNB / 2 : BNB);

    // Buffer descriptors bound this tile's activation rows and this expert's
    // weights: a load past num_records returns zeros without touching memory.
    // Activation rows: either rows row0.. of A (expert-ordered rows), or,
    // with row_token, the token rows row_token[row0 + r] of A read in place
    // (the permutation's row move fused into this load).
    const __amdgpu_buffer_rsrc_t a_rsrc =
        row_token ? __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, (int)(a_rows * K * 2), kBufferConfig)
                  : __builtin_amdgcn_make_buffer_rsrc((void*)(A + row0 * K), (short)0, rows * K * 2, kBufferConfig);
    const __amdgpu_buffer_rsrc_t b_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(W + (int64_t)e * K * ldw), (short)0, K * ldw * 2, kBufferConfig);

    // byte offsets at k = 0 (out of range where the row or column does not
    // exist).  Activation instruction p of this wave fills rows
    // (wave + 4p) * RPI + lane / CPR; weight instruction p fills k-rows
    // (wave + 4p) * 2 + lane / 32.
    uint32_t a_voff[GE::A_INSTR], b_voff[GE::B_INSTR];
#pragma unroll
    for (int p = 0; p < GE::A_INSTR; ++p) {
      const int r = (wave + WAVES * p) * GE::RPI + lane / GE::CPR;
      const int c = (lane % GE::CPR) ^ GE::swz(r);
      int64_t src = r;
      if (row_token) src = (r < rows) ? row_token[row0 + r] : -1;
      a_voff[p] = (r < rows && src >= 0 && src < (row_token ? a_rows : rows)) ? (uint32_t)(src * K + c * 8) * 2u
                                                                               : kOutOfRange;
    }
#pragma unroll
    for (int p = 0; p < GE::B_INSTR; ++p) {
      const int kr = (wave + WAVES * p) * GE::BRPI + lane / GE::BCPR;
      const int c = (lane % GE::BCPR) ^ ((kr & 3) << 2);
      const int tc = c * 8;
      int gcol;
      bool ok;
      if (SWIGLU) {
        const int hc = n0 + (tc % (BNB / 2));
        ok = hc < N;
        gcol = (tc < BNB / 2) ? hc : N + hc;
      } else {
        gcol = n0 + tc;
        ok = gcol < N;
      }
      b_voff[p] = ok ? (uint32_t)(kr * ldw + gcol) * 2u : kOutOfRange;
    }
    const int nk = K / BK;

    auto issue = [&](int s, char* a_buf, char* b_buf) {
      const uint32_t ka = (uint32_t)s * BK * 2u;
      const uint32_t kb = (uint32_t)s * BK * ldw * 2u;
      const uint32_t a_lds = lds_address(a_buf) + wave * 1024;
      const uint32_t b_lds = lds_address(b_buf) + wave * 1024;
#pragma unroll
      for (int p = 0; p < GE::A_INSTR; ++p) dma16(a_rsrc, a_lds + p * WAVES * 1024, a_voff[p] + ka);
#pragma unroll
      for (int p = 0; p < GE::B_INSTR; ++p) dma16(b_rsrc, b_lds + p * WAVES * 1024, b_voff[p] + kb);
    };

    f32x16 acc[NJ][2];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[j][i][q] = 0.f;

    auto compute = [&](const char* a_buf, const char* b_buf) {
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        bf16x8 a[2], b[NJ];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = 64 * wm + 32 * i + lane % 32;
          a[i] = *(const bf16x8*)(a_buf + GE::a_byte(r, ks * 2 + lane / 32));
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int kr = ks * 16 + (g / 2) * 8 + L / 4;
          const int col = col_base(j) + (g % 2) * 16 + 4 * (L % 4);
          const uint32_t off = GE::b_byte(kr, col >> 3) + ((col >> 2) & 1) * 8;
          b[j] = lds_read_b_operand((const bf16_t*)(b_buf + off), (const bf16_t*)(b_buf + off + 4 * GE::BROW));
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int i = 0; i < 2; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[j][i], 0, 0, 0);
      }
    };

    // Stage kt lives in buffer kt % 3.  At step kt each wave waits for its
    // own loads of stage kt, the barrier makes the whole stage visible and
    // guarantees every wave is done with stage kt - 1, whose buffer then
    // receives stage kt + 2.
    auto step = [&](int kt, const char* a_cur, const char* b_cur, char* a_nxt, char* b_nxt) {
      if (kt + 1 < nk) wait_vmcnt<GE::PER_STAGE>(); else wait_vmcnt<0>();
      compiler_fence();
      __builtin_amdgcn_s_barrier();
      compiler_fence();
      if (kt + 2 < nk) issue(kt + 2, a_nxt, b_nxt);
      compute(a_cur, b_cur);
    };
    issue(0, sA0, sB0);
    if (nk > 1) issue(1, sA1, sB1);
    for (int kt = 0;;) {
      step(kt, sA0, sB0, sA2, sB2);
      if (++kt >= nk) break;
      step(kt, sA1, sB1, sA0, sB0);
      if (++kt >= nk) break;
      step(kt, sA2, sB2, sA1, sB1);
      if (++kt >= nk) break;
    }

    // ---- epilogue (registers only); acc[j][i] holds output row 64*wm + 32*i + lane%32,
    // columns col_base(j) + 8*q4 + 4*(lane/32) + {0..3} ----
    const int lr = lane % 32, lc = 4 * (lane / 32);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 64 * wm + 32 * i + lr;
      if (r >= rows) continue;
      bf16_t* orow = Out + (row0 + r) * N;
      if (SWIGLU) {
#pragma unroll
        for (int j = 0; j < NJ / 2; ++j)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int c = n0 + (WCOL / 2) * wn + 32 * j + 8 * q4 + lc;
            if (c >= N) continue;
            uint32_t packed[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              float hv[2];
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const float gt = acc[j][i][4 * q4 + 2 * h2 + u], up = acc[j + NJ / 2][i][4 * q4 + 2 * h2 + u];
                hv[u] = gt / (1.f + __expf(-gt)) * up;
              }
              packed[h2] = (uint32_t)f32_to_bf16(hv[0]) | ((uint32_t)f32_to_bf16(hv[1]) << 16);
            }
            *(uint2*)(orow + c) = make_uint2(packed[0], packed[1]);
          }
      } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int c = n0 + WCOL * wn + 32 * j + 8 * q4 + lc;
            if (c >= N) continue;
            const uint32_t p0 = (uint32_t)f32_to_bf16(acc[j][i][4 * q4]) |
                                ((uint32_t)f32_to_bf16(acc[j][i][4 * q4 + 1]) << 16);
            const uint32_t p1 = (uint32_t)f32_to_bf16(acc[j][i][4 * q4 + 2]) |
                                ((uint32_t)f32_to_bf16(acc[j][i][4 * q4 + 3]) << 16);
            *(uint2*)(orow + c) = make_uint2(p0, p1);
          }
      }
    }
    // the next tile's first loads overwrite buffers 0 and 1: every wave must be
    // done reading them
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
  }
}

}  // namespace dma

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
// no more than the workgroups per CU the tile allows, a multiple of the XCD count.
int persistent_grid(int64_t max_rows, int E, int bm, int n_tiles, int occ) {
  const int64_t max_mt = max_rows / bm + (int64_t)(E < max_rows ? E : max_rows);
  const int64_t want = max_mt * n_tiles;
  const int64_t cap = (int64_t)occ * num_cus();
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

template <bool SWIGLU, int BK = 32, int OCC = 2, int NJ = 4, int WM = 2>
hipError_t launch_dma(const bf16_t* a, const int32_t* offsets, int64_t max_rows, int E, int K, int N, int ldw,
                      const bf16_t* w, bf16_t* out, hipStream_t s, const int32_t* row_token = nullptr,
                      int64_t a_rows = 0) {
  constexpr int BNO = SWIGLU ? 32 * NJ : 64 * NJ;   // output columns per tile
  const int nt = (int)ceil_div(N, BNO);
  dma::k_grouped_gemm<SWIGLU, BK, OCC, NJ, WM><<<persistent_grid(max_rows, E, 64 * WM, nt, OCC), 128 * WM, 0, s>>>(
      a, offsets, max_rows, E, K, N, ldw, w, out, nt, row_token, a_rows);
  return hipGetLastError();
}

// Tile shape from sizes the host knows: 256-row tiles (8 waves sharing each
// LDS stage, half the weight traffic per flop) once experts hold 256 rows
// or more on average, 128-row tiles (two workgroups per CU) below that.
bool wide_rows(int64_t max_rows, int E, int64_t threshold) { return max_rows >= threshold * E; }

}  // namespace

hipError_t launch_gate_up_bf16(const bf16_t* x, const int32_t* expert_offsets, int64_t max_rows, int E, int d,
                               int I, const bf16_t* w_gate_up, bf16_t* h, hipStream_t s, const int32_t* row_token,
                               int64_t x_rows) {
  if (wide_rows(max_rows, E, 256))
    return launch_dma<true, 32, 1, 4, 4>(x, expert_offsets, max_rows, E, d, I, 2 * I, w_gate_up, h, s, row_token,
                                         x_rows);
  return launch_dma<true>(x, expert_offsets, max_rows, E, d, I, 2 * I, w_gate_up, h, s, row_token, x_rows);
}

hipError_t launch_down_bf16(const bf16_t* h, const int32_t* expert_offsets, int64_t max_rows, int E, int d,
                            int I, const bf16_t* w_down, bf16_t* y_perm, hipStream_t s) {
  if (wide_rows(max_rows, E, 1024))
    return launch_dma<false, 32, 1, 4, 4>(h, expert_offsets, max_rows, E, I, d, d, w_down, y_perm, s);
  return launch_dma<false>(h, expert_offsets, max_rows, E, I, d, d, w_down, y_perm, s);
}

hipError_t launch_gate_up_f32(const float* x_perm, const int32_t* expert_offsets, int64_t max_rows, int E,
                              int d, int I, const float* w_gate_up, float* h, hipStream_t s) {
  dim3 g((unsigned)max_rows, (unsigned)ceil_div(I, 256));
  k_ffn_gate_up_f32<<<g, 256, 0, s>>>(x_perm, expert_offsets, max_rows, E, d, I, w_gate_up, h);
  return hipGetLastError();
}

hipError_t launch_down_f32(const float* h, const int32_t* expert_offsets, int64_t max_rows, int E, int d,
                           int I, const float* w_down, float* y_perm, hipStream_t s) {
  dim3 g((unsigned)max_rows, (unsigned)ceil_div(d, 256));
  k_ffn_down_f32<<<g, 256, 0, s>>>(h, expert_offsets, max_rows, E, d, I, w_down, y_perm);
  return hipGetLastError();
}

hipError_t launch_grouped_ffn_bf16(const bf16_t* x_perm, const int32_t* expert_offsets, int64_t max_rows,
                                   int E, int d, int I, const bf16_t* w_gate_up, const bf16_t* w_down,
                                   bf16_t* h, bf16_t* y_perm, hipStream_t s) {
  const hipError_t e = launch_gate_up_bf16(x_perm, expert_offsets, max_rows, E, d, I, w_gate_up, h, s, nullptr, 0);
  if (e != hipSuccess) return e;
  return launch_down_bf16(h, expert_offsets, max_rows, E, d, I, w_down, y_perm, s);
}

hipError_t launch_grouped_ffn_f32(const float* x_perm, const int32_t* expert_offsets, int64_t max_rows, int E,
                                  int d, int I, const float* w_gate_up, const float* w_down, float* h,
                                  float* y_perm, hipStream_t s) {
  const hipError_t e = launch_gate_up_f32(x_perm, expert_offsets, max_rows, E, d, I, w_gate_up, h, s);
  if (e != hipSuccess) return e;
  return launch_down_f32(h, expert_offsets, max_rows, E, d, I, w_down, y_perm, s);
}

}  // namespace tre
