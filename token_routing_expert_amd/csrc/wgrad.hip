// wgrad.hip -- per-expert weight gradients of the grouped feed-forward.
//
// "Expert parallelism" (Hugging Face Transformers docs), "Combining with
// FSDP2": an expert's gradient is the sum over every batch (here: every row)
// it served, and an expert that received no tokens still has one (zero).
// For the down projection y = h Wd[e] and the gate/up projection
// [g | u] = x Wgu[e] of the rows r of expert e:
//   dWd[e]  = sum_r h[r]^T  dy[r]          [I, d]
//   dWgu[e] = sum_r x[r]^T [dg | du][r]    [d, 2I]
// i.e. dW[e] = A_e^T B_e with the expert's rows as the contraction.
//
// Design: one workgroup per 128 x 256 tile of one expert's gradient (4
// waves, each 64 x 128 as 2 x 4 v_mfma_f32_32x32x16_bf16 tiles), stages of
// 32 of the expert's rows streamed through a ring of three LDS buffers by
// loads that write LDS directly.  Both operands are stored in LDS row by row
// of the contraction (as they lie in memory) and read with the transposing
// ds_read_b64_tr_b16, which yields the MFMA operand layout directly.  Rows
// past the expert's last row and columns past the matrix read zeros through
// the buffer descriptors, so ragged tiles need no branches; an expert with no
// rows writes a zero tile.  Float32 accumulation over all of the expert's
// rows, one rounding to bf16.
#include "common.hpp"

namespace tre {
namespace {

constexpr int kBM = 128, kBN = 256, kBK = 32, kNS = 3;
constexpr int kXcd = 8;
constexpr uint32_t kPast = 0x80000000u;  // a byte offset past every descriptor's num_records

// k-row kr of a stage tile holds ROWB bytes; its 16-byte chunk c sits in
// slot c ^ 4 (kr & 3), so that the transposing reads (4 consecutive k-rows x
// 32 bytes per 16-lane group) spread over the banks
template <int ROWB>
__device__ __forceinline__ uint32_t tile_byte(int kr, int c) {
  return (uint32_t)(kr * ROWB + ((c ^ ((kr & 3) << 2)) << 4));
}

__global__ __launch_bounds__(256, 2) void k_wgrad(const bf16_t* __restrict__ a, int lda, int M,
                                                  const bf16_t* __restrict__ b, int ldb, int N,
                                                  const int32_t* __restrict__ offsets, int64_t max_rows, int E,
                                                  bf16_t* __restrict__ dw, int m_tiles, int n_tiles) {
  constexpr int AROW = kBM * 2, BROW = kBN * 2;                 // bytes per k-row of a stage
  constexpr int A_BYTES = kBK * AROW, B_BYTES = kBK * BROW;     // 8 KB and 16 KB
  constexpr int A_RPI = 1024 / AROW, B_RPI = 1024 / BROW;       // k-rows per 1 KB load
  constexpr int A_CPR = AROW / 16, B_CPR = BROW / 16;           // 16-byte chunks per k-row
  constexpr int A_INSTR = A_BYTES / 1024 / 4, B_INSTR = B_BYTES / 1024 / 4;  // loads per wave per stage
  constexpr int PER = A_INSTR + B_INSTR;
  __shared__ __attribute__((aligned(1024))) char sA[kNS * A_BYTES];
  __shared__ __attribute__((aligned(1024))) char sB[kNS * B_BYTES];

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / 2, wn = wave % 2;
  const int g16 = lane / 16, L = lane % 16;

  // consecutive tiles (one expert, one row block of the gradient) go to one
  // XCD, whose L2 then holds the expert's rows for all of them
  const int G = gridDim.x;
  const int vb = (blockIdx.x % kXcd) * (G / kXcd) + blockIdx.x / kXcd;
  if (vb >= E * m_tiles * n_tiles) return;
  const int e = vb / (m_tiles * n_tiles);
  const int rem = vb - e * (m_tiles * n_tiles);
  const int m0 = (rem / n_tiles) * kBM, n0 = (rem % n_tiles) * kBN;
  const int lo = (int)clampi<int64_t>(offsets[e], 0, max_rows);
  const int cnt = (int)clampi<int64_t>(offsets[e + 1], lo, max_rows) - lo;
  const int n_stages = (cnt + kBK - 1) / kBK;

  // load p of this wave fills k-rows RPI (wave + 4 p) .. +RPI-1 of its tile
  uint32_t a_off[A_INSTR], b_off[B_INSTR];
#pragma unroll
  for (int p = 0; p < A_INSTR; ++p) {
    const int kr = A_RPI * (wave + 4 * p) + lane / A_CPR;
    const int col = m0 + 8 * ((lane % A_CPR) ^ ((kr & 3) << 2));
    a_off[p] = col < M ? (uint32_t)(kr * lda + col) * 2u : kPast;
  }
#pragma unroll
  for (int p = 0; p < B_INSTR; ++p) {
    const int kr = B_RPI * (wave + 4 * p) + lane / B_CPR;
    const int col = n0 + 8 * ((lane % B_CPR) ^ ((kr & 3) << 2));
    b_off[p] = col < N ? (uint32_t)(kr * ldb + col) * 2u : kPast;
  }
  auto issue = [&](int st) {
    const int64_t r0 = lo + (int64_t)st * kBK;
    const int rows = min(kBK, cnt - st * kBK);
    // descriptors over this stage's rows only: k-rows past them read zeros
    const __amdgpu_buffer_rsrc_t ar =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a + r0 * lda), (short)0, rows * lda * 2, kBufferConfig);
    const __amdgpu_buffer_rsrc_t br =
        __builtin_amdgcn_make_buffer_rsrc((void*)(b + r0 * ldb), (short)0, rows * ldb * 2, kBufferConfig);
    const int buf = st % kNS;
    const uint32_t a_lds = lds_address(sA + buf * A_BYTES) + wave * 1024;
    const uint32_t b_lds = lds_address(sB + buf * B_BYTES) + wave * 1024;
#pragma unroll
    for (int p = 0; p < A_INSTR; ++p) dma16(ar, a_lds + p * 4 * 1024, a_off[p]);
#pragma unroll
    for (int p = 0; p < B_INSTR; ++p) dma16(br, b_lds + p * 4 * 1024, b_off[p]);
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[j][i][q] = 0.f;

  for (int st = 0; st < kNS - 1 && st < n_stages; ++st) issue(st);
  for (int st = 0; st < n_stages; ++st) {
    // this wave's loads of stage st are done once at most the younger
    // stages' loads are outstanding (near the end: once none are)
    if (st + kNS - 2 < n_stages) wait_vmcnt<(kNS - 2) * PER>(); else wait_vmcnt<0>();
    stage_barrier();  // stage st visible to all; every wave is done with stage st - 1
    if (st + kNS - 1 < n_stages) issue(st + kNS - 1);
    const char* at = sA + (st % kNS) * A_BYTES;
    const char* bt = sB + (st % kNS) * B_BYTES;
    bf16x8 fa[2][2], fb[2][4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kr = ks * 16 + (g16 / 2) * 8 + L / 4;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int col = 64 * wm + 32 * i + (g16 % 2) * 16 + 4 * (L % 4);
        const uint32_t off = tile_byte<AROW>(kr, col >> 3) + ((col >> 2) & 1) * 8;
        fa[ks][i] = lds_read_b_operand((const bf16_t*)(at + off), (const bf16_t*)(at + off + 4 * AROW));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = 128 * wn + 32 * j + (g16 % 2) * 16 + 4 * (L % 4);
        const uint32_t off = tile_byte<BROW>(kr, col >> 3) + ((col >> 2) & 1) * 8;
        fb[ks][j] = lds_read_b_operand((const bf16_t*)(bt + off), (const bf16_t*)(bt + off + 4 * BROW));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks][j], fa[ks][i], acc[j][i], 0, 0, 0);
  }

  // acc[j][i]: gradient row m0 + 64 wm + 32 i + lane % 32, columns
  // n0 + 128 wn + 32 j + 8 q4 + 4 (lane / 32) + {0..3}
  bf16_t* out = dw + (int64_t)e * M * N;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + 64 * wm + 32 * i + lane % 32;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int n = n0 + 128 * wn + 32 * j + 8 * q4 + 4 * (lane / 32);
        if (n >= N) continue;
        float f[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) f[v] = acc[j][i][4 * q4 + v];
        *(uint2*)(out + (int64_t)m * N + n) =
            make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
      }
  }
}

__global__ __launch_bounds__(256) void k_zero(u32x4* __restrict__ p, int64_t n_vec) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_vec; i += (int64_t)gridDim.x * 256)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

}  // namespace

hipError_t launch_zero_bf16(bf16_t* p, int64_t n, hipStream_t s) {
  if (n % 8 != 0) return hipErrorInvalidValue;
  const int64_t n_vec = n / 8;
  if (n_vec == 0) return hipSuccess;
  const int64_t blocks = ceil_div(n_vec, 256) < 4096 ? ceil_div(n_vec, 256) : 4096;
  k_zero<<<(unsigned)blocks, 256, 0, s>>>((u32x4*)p, n_vec);
  return hipGetLastError();
}

hipError_t launch_wgrad_bf16(const bf16_t* a, int lda, int M, const bf16_t* b, int ldb, int N,
                             const int32_t* expert_offsets, int64_t max_rows, int E, bf16_t* dw, hipStream_t s) {
  if (M % 4 != 0 || N % 4 != 0 || lda < M || ldb < N) return hipErrorInvalidValue;
  const int m_tiles = (int)ceil_div(M, kBM), n_tiles = (int)ceil_div(N, kBN);
  const int64_t tiles = (int64_t)E * m_tiles * n_tiles;
  const int64_t grid = round_up(tiles, kXcd);
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  k_wgrad<<<(unsigned)grid, 256, 0, s>>>(a, lda, M, b, ldb, N, expert_offsets, max_rows, E, dw, m_tiles, n_tiles);
  return hipGetLastError();
}

}  // namespace tre
