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

constexpr int NTHR = 256;        // 4 waves per workgroup
constexpr int kXcd = 8;          // XCDs per MI355X; workgroups are dealt round-robin over them
// Buffer descriptor word 3 for raw (untyped) buffer loads on CDNA, and byte
// offsets that are always past num_records (a load there returns zeros).
constexpr int kBufferConfig = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr uint32_t kStagePast = 0x40000000u;
// LDS rows are padded: activation rows by 16 bytes (16 consecutive rows of a
// ds_read_b128 land on distinct banks for 64- and 32-element rows), weight
// rows by 64 bytes (the 4 consecutive k-rows of a ds_read_b64_tr_b16 group
// land on distinct banks).

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

// Tile shape.  Four waves; wave tile WTM rows x 128 weight columns (MI x 4
// MFMA 32x32 tiles, MI = WTM / 32); WM x WN waves per workgroup.
template <int WTM_, int WM_, int BK_, bool SWIGLU_, int OCC_ = 1>
struct Tile {
  static constexpr int WTM = WTM_, WM = WM_, WN = 4 / WM_, BK = BK_;
  static constexpr int OCC = OCC_;                       // workgroups per CU the launch aims for
  static constexpr bool SWIGLU = SWIGLU_;
  static constexpr int MI = WTM / 32;                    // MFMA row tiles per wave
  static constexpr int BM = WTM * WM;                    // rows per workgroup tile
  static constexpr int BNB = 128 * WN;                   // weight columns per tile
  static constexpr int BNO = SWIGLU ? BNB / 2 : BNB;     // output columns per tile
  static constexpr int A_LD = BK + 8;                    // padded LDS row (elements)
  static constexpr int B_LD = BNB + 32;
  static constexpr int A_STAGE = BM * A_LD;              // elements per LDS stage
  static constexpr int B_STAGE = BK * B_LD;
  static constexpr int A_CHUNKS = BM * BK / 8 / NTHR;    // 16-byte copies per thread per stage
  static constexpr int B_CHUNKS = BK * BNB / 8 / NTHR;
  static_assert(A_CHUNKS >= 1 && B_CHUNKS >= 1, "tile too small for 256 threads");
  static constexpr size_t LDS_BYTES = 2 * (A_STAGE + B_STAGE) * sizeof(bf16_t);
};

// A: [max_rows, K] activations; W: [E, K, ldw] weights; Out: [max_rows, N].
// SWIGLU: N = I, ldw = 2I; the weight tile holds BNB/2 gate columns and the
// matching BNB/2 up columns, output columns [n0, n0 + BNB/2).
// plain:  N = d, ldw = d; output columns [n0, n0 + BNB).
// The MFMA is issued with the weight fragment as its first operand, so the
// accumulator is the transposed tile: each lane owns one output row and
// groups of 4 consecutive output columns, stored 8 bytes at a time.
template <class C>
__global__ __launch_bounds__(NTHR, C::OCC) void k_grouped_gemm_bf16(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ offsets, int64_t max_rows, int E, int K,
    int N, int ldw, const bf16_t* __restrict__ W, bf16_t* __restrict__ Out, int n_tiles) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2 * C::A_STAGE];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2 * C::B_STAGE];
  __shared__ int s_start[kMaxExperts];
  __shared__ int s_mt[kMaxExperts];
  __shared__ int64_t s_lo[kMaxExperts];
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_wave[NTHR / kWave];

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave / C::WN, wn = wave % C::WN;

  // ---- tile list from the device offsets ----
  int mt = 0;
  if (tid < E) {
    const int64_t lo = clampi<int64_t>(offsets[tid], 0, max_rows);
    const int64_t hi = clampi<int64_t>(offsets[tid + 1], lo, max_rows);
    s_lo[tid] = lo;
    s_cnt[tid] = (int)(hi - lo);
    mt = (int)ceil_div(hi - lo, C::BM);
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

  // per-thread constant parts of the global->LDS copies (16 B each)
  constexpr int A_CPR = C::BK / 8;        // chunks per activation row
  constexpr int B_CPR = C::BNB / 8;       // chunks per weight row
  const int a_col = (tid % A_CPR) * 8, a_row0 = tid / A_CPR;
  const int b_tcol = (tid % B_CPR) * 8, b_row0 = tid / B_CPR;
  constexpr int A_RSTEP = NTHR / A_CPR, B_RSTEP = NTHR / B_CPR;

  const int g = lane / 16, L = lane % 16;

  for (int64_t v = vb; v < total_tiles; v += G) {
    // expert: the last one whose first tile is <= v (empty experts own no tiles)
    int lo_e = 0, hi_e = E - 1;
    while (lo_e < hi_e) {
      const int mid = (lo_e + hi_e + 1) / 2;
      if ((int64_t)s_start[mid] * n_tiles <= v) lo_e = mid; else hi_e = mid - 1;
    }
    // every lane computed the same tile; make that visible to the compiler so
    // the tile's addresses and buffer descriptors live in scalar registers
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
    const int64_t row0 = e_row0 + (int64_t)mtile * C::BM;
    const int rows = min(C::BM, e_cnt - mtile * C::BM);
    const int n0 = nt * C::BNO;
    const bf16_t* Wb = W + (int64_t)e * K * ldw;

    int b_gcol;
    bool b_ok;
    if (C::SWIGLU) {
      const int hc = n0 + (b_tcol % (C::BNB / 2));
      b_ok = hc < N;
      b_gcol = (b_tcol < C::BNB / 2) ? hc : N + hc;
    } else {
      b_gcol = n0 + b_tcol;
      b_ok = b_gcol < N;
    }

    // Buffer descriptors bound this tile's activation rows and this expert's
    // weights: a load past num_records returns zeros without touching memory,
    // so ragged rows, absent columns and the stages past the last need no
    // branches (and the compiler can count outstanding loads exactly).
    const __amdgpu_buffer_rsrc_t a_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(A + row0 * K), (short)0, rows * K * 2, kBufferConfig);
    const __amdgpu_buffer_rsrc_t b_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)Wb, (short)0, K * ldw * 2, kBufferConfig);
    uint32_t a_off[C::A_CHUNKS], b_off[C::B_CHUNKS];
#pragma unroll
    for (int p = 0; p < C::A_CHUNKS; ++p) {
      const int r = a_row0 + A_RSTEP * p;
      a_off[p] = (r < rows) ? (uint32_t)(r * K + a_col) * 2u : kOutOfRange;
    }
#pragma unroll
    for (int p = 0; p < C::B_CHUNKS; ++p) {
      const int kr = b_row0 + B_RSTEP * p;
      b_off[p] = b_ok ? (uint32_t)(kr * ldw + b_gcol) * 2u : kOutOfRange;
    }
    const int nk = K / C::BK;
    constexpr int NR = C::A_CHUNKS + C::B_CHUNKS;
    // stage s -> registers; stages past the last read nothing
    auto gload = [&](int s, u32x4* R) {
      const uint32_t ka = (s < nk) ? (uint32_t)s * C::BK * 2u : kStagePast;
      const uint32_t kb = (s < nk) ? (uint32_t)s * C::BK * ldw * 2u : kStagePast;
#pragma unroll
      for (int p = 0; p < C::A_CHUNKS; ++p) R[p] = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, a_off[p] + ka, 0, 0);
#pragma unroll
      for (int p = 0; p < C::B_CHUNKS; ++p)
        R[C::A_CHUNKS + p] = __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, b_off[p] + kb, 0, 0);
    };
    auto lstore = [&](int buf, const u32x4* R) {
      bf16_t* as = As + buf * C::A_STAGE;
      bf16_t* bs = Bs + buf * C::B_STAGE;
#pragma unroll
      for (int p = 0; p < C::A_CHUNKS; ++p) *(u32x4*)&as[(a_row0 + A_RSTEP * p) * C::A_LD + a_col] = R[p];
#pragma unroll
      for (int p = 0; p < C::B_CHUNKS; ++p)
        *(u32x4*)&bs[(b_row0 + B_RSTEP * p) * C::B_LD + b_tcol] = R[C::A_CHUNKS + p];
    };

    // tile column of this wave's MFMA column tile j
    auto col_base = [&](int j) {
      if (C::SWIGLU) return (j < 2) ? 64 * wn + 32 * j : C::BNB / 2 + 64 * wn + 32 * (j - 2);
      return 128 * wn + 32 * j;
    };

    f32x16 acc[4][C::MI];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < C::MI; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[j][i][q] = 0.f;

    auto compute = [&](int buf) {
      const bf16_t* as = As + buf * C::A_STAGE;
      const bf16_t* bs = Bs + buf * C::B_STAGE;
#pragma unroll
      for (int ks = 0; ks < C::BK / 16; ++ks) {
        bf16x8 a[C::MI], b[4];
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
          a[i] = *(const bf16x8*)&as[(C::WTM * wm + 32 * i + lane % 32) * C::A_LD + ks * 16 + (lane / 32) * 8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int krow = ks * 16 + (g / 2) * 8 + L / 4;
          const int col = col_base(j) + (g % 2) * 16 + 4 * (L % 4);
          b[j] = lds_read_b_operand(&bs[krow * C::B_LD + col], &bs[(krow + 4) * C::B_LD + col]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < C::MI; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[j][i], 0, 0, 0);
      }
    };

    // Two stages in registers, two in LDS: stage s is loaded in iteration
    // s - 2, written to LDS at the end of iteration s - 1 and multiplied in
    // iteration s; one barrier per stage.
    u32x4 R0[NR], R1[NR];
    gload(0, R0);
    gload(1, R1);
    lstore(0, R0);
    __syncthreads();
    // (scheduling fences keep the compiler from sinking the loads of stage
    // s + 2 below the multiplications they are meant to overlap)
    for (int kt = 0;;) {
      gload(kt + 2, R0);
      __builtin_amdgcn_sched_barrier(0);
      compute(0);
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 1 < nk) lstore(1, R1);
      __syncthreads();
      if (++kt >= nk) break;
      gload(kt + 2, R1);
      __builtin_amdgcn_sched_barrier(0);
      compute(1);
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 1 < nk) lstore(0, R0);
      __syncthreads();
      if (++kt >= nk) break;
    }

    // ---- epilogue: acc[j][i] holds output rows C::WTM*wm + 32*i + lane%32,
    // columns col_base(j) + 8*q4 + 4*(lane/32) + {0..3} in elements 4*q4.. ----
    const int lr = lane % 32, lc = 4 * (lane / 32);
#pragma unroll
    for (int i = 0; i < C::MI; ++i) {
      const int r = C::WTM * wm + 32 * i + lr;
      if (r >= rows) continue;
      bf16_t* orow = Out + (row0 + r) * N;
      if (C::SWIGLU) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int c = n0 + 64 * wn + 32 * j + 8 * q4 + lc;
            if (c >= N) continue;
            uint32_t packed[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              float hv[2];
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const float gt = acc[j][i][4 * q4 + 2 * h2 + u], up = acc[j + 2][i][4 * q4 + 2 * h2 + u];
                hv[u] = gt / (1.f + __expf(-gt)) * up;
              }
              packed[h2] = (uint32_t)f32_to_bf16(hv[0]) | ((uint32_t)f32_to_bf16(hv[1]) << 16);
            }
            *(uint2*)(orow + c) = make_uint2(packed[0], packed[1]);
          }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int c = n0 + 128 * wn + 32 * j + 8 * q4 + lc;
            if (c >= N) continue;
            const uint32_t p0 = (uint32_t)f32_to_bf16(acc[j][i][4 * q4]) |
                                ((uint32_t)f32_to_bf16(acc[j][i][4 * q4 + 1]) << 16);
            const uint32_t p1 = (uint32_t)f32_to_bf16(acc[j][i][4 * q4 + 2]) |
                                ((uint32_t)f32_to_bf16(acc[j][i][4 * q4 + 3]) << 16);
            *(uint2*)(orow + c) = make_uint2(p0, p1);
          }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// LDS-DMA pipeline (the bf16 path).  Workgroup tile 128 rows x 256 weight
// columns x 64 k; 4 waves in 2 x 2, each 64 x 128 (2 x 4 MFMA 32x32 tiles).
// Tiles stream through a ring of three LDS stages filled by buffer loads that
// write LDS directly (no staging registers): while stage s is multiplied,
// stages s+1 and s+2 are in flight.  One barrier per stage; each wave waits
// for its own loads of the stage (vmcnt) before the barrier, so after the
// barrier the whole stage is resident.
// LDS layouts are dense (a DMA instruction fills 1 KB contiguously) and
// XOR-swizzled instead of padded:
//   activation rows (64 k = 128 B = 8 chunks of 16 B): chunk c of row r sits
//     in slot c ^ ((r >> 1) & 7), so a ds_read_b128 of 16 consecutive rows
//     touches every bank once;
//   weight rows (256 columns = 512 B = 32 chunks): chunk c of k-row kr sits
//     in slot c ^ (4 * (kr & 3)), so the 4 consecutive k-rows x 32 bytes a
//     16-lane ds_read_b64_tr_b16 group reads fall on distinct banks.
namespace dma {

constexpr int BM = 128, BNB = 256, BK = 64;
constexpr int A_BYTES = BM * BK * 2;           // 16 KB
constexpr int B_BYTES = BK * BNB * 2;          // 32 KB
constexpr int A_INSTR = A_BYTES / 1024 / 4;    // DMA instructions per wave per stage
constexpr int B_INSTR = B_BYTES / 1024 / 4;
constexpr int PER_STAGE = A_INSTR + B_INSTR;

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

__device__ __forceinline__ uint32_t a_slot_byte(int r, int c) { return (uint32_t)(r * 128 + ((c ^ ((r >> 1) & 7)) << 4)); }
__device__ __forceinline__ uint32_t b_slot_byte(int kr, int c) { return (uint32_t)(kr * 512 + ((c ^ ((kr & 3) << 2)) << 4)); }

template <bool SWIGLU>
__global__ __launch_bounds__(NTHR, 1) void k_grouped_gemm(const bf16_t* __restrict__ A, const int32_t* __restrict__ offsets,
                                                         int64_t max_rows, int E, int K, int N, int ldw,
                                                         const bf16_t* __restrict__ W, bf16_t* __restrict__ Out,
                                                         int n_tiles) {
  __shared__ __attribute__((aligned(1024))) char sA0[A_BYTES];
  __shared__ __attribute__((aligned(1024))) char sA1[A_BYTES];
  __shared__ __attribute__((aligned(1024))) char sA2[A_BYTES];
  __shared__ __attribute__((aligned(1024))) char sB0[B_BYTES];
  __shared__ __attribute__((aligned(1024))) char sB1[B_BYTES];
  __shared__ __attribute__((aligned(1024))) char sB2[B_BYTES];
  __shared__ int s_start[kMaxExperts];
  __shared__ int s_mt[kMaxExperts];
  __shared__ int64_t s_lo[kMaxExperts];
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_wave[NTHR / kWave];

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
  const int start = block_exclusive_scan(mt, s_wave, &total_mt);
  if (tid < E) s_start[tid] = start;
  __syncthreads();
  const int64_t total_tiles = (int64_t)total_mt * n_tiles;
  const int G = gridDim.x;
  const int vb = (blockIdx.x % kXcd) * (G / kXcd) + blockIdx.x / kXcd;

  // this lane's DMA slots: activation instruction p covers rows (wave + 4p) * 8 + lane / 8,
  // weight instruction p covers k-rows (wave + 4p) * 2 + lane / 32
  const int a_slot = lane % 8, b_slot = lane % 32;

  auto col_base = [&](int j) {
    if (SWIGLU) return (j < 2) ? 64 * wn + 32 * j : BNB / 2 + 64 * wn + 32 * (j - 2);
    return 128 * wn + 32 * j;
  };

  for (int64_t v = vb; v < total_tiles; v += G) {
    int lo_e = 0, hi_e = E - 1;
    while (lo_e < hi_e) {
      const int mid = (lo_e + hi_e + 1) / 2;
      if ((int64_t)s_start[mid] * n_tiles <= v) lo_e = mid; else hi_e = mid - 1;
    }
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

    const __amdgpu_buffer_rsrc_t a_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(A + row0 * K), (short)0, rows * K * 2, kBufferConfig);
    const __amdgpu_buffer_rsrc_t b_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(W + (int64_t)e * K * ldw), (short)0, K * ldw * 2, kBufferConfig);

    // byte offsets at k = 0 (out of range where the row or column does not exist)
    uint32_t a_voff[A_INSTR], b_voff[B_INSTR];
#pragma unroll
    for (int p = 0; p < A_INSTR; ++p) {
      const int r = (wave + 4 * p) * 8 + lane / 8;
      const int c = a_slot ^ ((r >> 1) & 7);
      a_voff[p] = (r < rows) ? (uint32_t)(r * K + c * 8) * 2u : kOutOfRange;
    }
#pragma unroll
    for (int p = 0; p < B_INSTR; ++p) {
      const int kr = (wave + 4 * p) * 2 + lane / 32;
      const int c = b_slot ^ ((kr & 3) << 2);
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
      for (int p = 0; p < A_INSTR; ++p) dma16(a_rsrc, a_lds + p * 4096, a_voff[p] + ka);
#pragma unroll
      for (int p = 0; p < B_INSTR; ++p) dma16(b_rsrc, b_lds + p * 4096, b_voff[p] + kb);
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[j][i][q] = 0.f;

    auto compute = [&](const char* a_buf, const char* b_buf) {
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        bf16x8 a[2], b[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = 64 * wm + 32 * i + lane % 32;
          a[i] = *(const bf16x8*)(a_buf + a_slot_byte(r, ks * 2 + lane / 32));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kr = ks * 16 + (g / 2) * 8 + L / 4;
          const int col = col_base(j) + (g % 2) * 16 + 4 * (L % 4);
          const uint32_t off = b_slot_byte(kr, col >> 3) + ((col >> 2) & 1) * 8;
          b[j] = lds_read_b_operand((const bf16_t*)(b_buf + off), (const bf16_t*)(b_buf + off + 4 * 512));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 2; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[j][i], 0, 0, 0);
      }
    };

    // stage kt lives in buffer kt % 3; stage kt + 2 is issued once every wave
    // is past stage kt - 1 (the barrier), into the buffer stage kt - 1 used.
    auto step = [&](int kt, const char* a_cur, const char* b_cur, char* a_nxt, char* b_nxt) {
      if (kt + 1 < nk) wait_vmcnt<PER_STAGE>(); else wait_vmcnt<0>();
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
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int c = n0 + 64 * wn + 32 * j + 8 * q4 + lc;
            if (c >= N) continue;
            uint32_t packed[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              float hv[2];
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const float gt = acc[j][i][4 * q4 + 2 * h2 + u], up = acc[j + 2][i][4 * q4 + 2 * h2 + u];
                hv[u] = gt / (1.f + __expf(-gt)) * up;
              }
              packed[h2] = (uint32_t)f32_to_bf16(hv[0]) | ((uint32_t)f32_to_bf16(hv[1]) << 16);
            }
            *(uint2*)(orow + c) = make_uint2(packed[0], packed[1]);
          }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int c = n0 + 128 * wn + 32 * j + 8 * q4 + lc;
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

// Tile shapes: activation rows per workgroup tile (BM) against the rows an
// expert is expected to hold.  Chosen on the host from sizes alone.
typedef Tile<64, 2, 64, true> GateUpM128;     // BM 128, 128 gate + 128 up columns
typedef Tile<64, 2, 64, false> DownM128;      // BM 128, 256 output columns

template <class C>
hipError_t launch_gemm(const bf16_t* a, const int32_t* offsets, int64_t max_rows, int E, int K, int N, int ldw,
                       const bf16_t* w, bf16_t* out, hipStream_t s) {
  const int nt = (int)ceil_div(N, C::BNO);
  k_grouped_gemm_bf16<C><<<persistent_grid(max_rows, E, C::BM, nt, C::OCC), NTHR, 0, s>>>(a, offsets, max_rows, E, K, N,
                                                                                  ldw, w, out, nt);
  return hipGetLastError();
}

template <bool SWIGLU>
hipError_t launch_dma(const bf16_t* a, const int32_t* offsets, int64_t max_rows, int E, int K, int N, int ldw,
                      const bf16_t* w, bf16_t* out, hipStream_t s) {
  const int nt = (int)ceil_div(N, SWIGLU ? dma::BNB / 2 : dma::BNB);
  dma::k_grouped_gemm<SWIGLU><<<persistent_grid(max_rows, E, dma::BM, nt, 1), NTHR, 0, s>>>(a, offsets, max_rows, E, K, N,
                                                                                          ldw, w, out, nt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_bf16(const bf16_t* x_perm, const int32_t* expert_offsets, int64_t max_rows, int E,
                               int d, int I, const bf16_t* w_gate_up, bf16_t* h, hipStream_t s) {
  return launch_dma<true>(x_perm, expert_offsets, max_rows, E, d, I, 2 * I, w_gate_up, h, s);
}

hipError_t launch_down_bf16(const bf16_t* h, const int32_t* expert_offsets, int64_t max_rows, int E, int d,
                            int I, const bf16_t* w_down, bf16_t* y_perm, hipStream_t s) {
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
  const hipError_t e = launch_gate_up_bf16(x_perm, expert_offsets, max_rows, E, d, I, w_gate_up, h, s);
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
