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
// Design: 128 x 256 tiles of one expert's gradient (4 waves, each 64 x 128
// as 2 x 4 v_mfma_f32_32x32x16_bf16 tiles), stages of 32 of the expert's rows
// streamed through a ring of three LDS buffers by loads that write LDS
// directly.  The grid is persistent (two workgroups per CU): a workgroup's
// tiles form one stream of stages, so the next tile's first stages load
// while the current tile finishes and stores its results -- an expert's rows
// are a short contraction (a few stages), which one workgroup per tile would
// spend mostly filling and draining its ring.  The gradient is as large as
// the weights and written once, so the stores set much of the pace: they
// leave through LDS as whole 128-byte row pieces, non-temporal.  Both operands are stored in LDS row by row
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
  static_assert(kNS == 3, "the stage wait below counts at most one younger stage");
  __shared__ __attribute__((aligned(1024))) char sA[kNS * A_BYTES];
  __shared__ __attribute__((aligned(1024))) char sB[kNS * B_BYTES];

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / 2, wn = wave % 2;
  const int g16 = lane / 16, L = lane % 16;

  // Persistent.  The tile list (expert by expert; in an expert, row blocks
  // of the gradient fastest, so a run of consecutive tiles shares the
  // smaller operand, the expert's rows of a) is cut into one contiguous range
  // per XCD holding an equal share of the work (tiles x stages of 32 rows):
  // an XCD's L2 then holds one or two experts' rows at a time, and skewed
  // expert sizes still spread evenly.  The XCD's W workgroups take its tiles
  // round-robin.
  const int G = gridDim.x, W = G / kXcd;
  const int xcd = blockIdx.x % kXcd, local = blockIdx.x / kXcd;
  const int per_e = m_tiles * n_tiles;
  const int n_all = E * per_e;
  struct Tile {
    int e, m0, n0, lo, cnt, ns;
  };
  // every expert's first row and row count, held by lane e / 4 (slot e % 4):
  // a tile is then decoded from registers, without a memory round trip
  int lo4[4], cnt4[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * lane + q;
    lo4[q] = e < E ? (int)clampi<int64_t>(offsets[e], 0, max_rows) : 0;
    cnt4[q] = e < E ? (int)clampi<int64_t>(offsets[e + 1], lo4[q], max_rows) - lo4[q] : 0;
  }
  auto pick = [&](const int (&v)[4], int e) {   // v of expert e (wave-uniform)
    const int q = e & 3;
    const int x = q == 0 ? v[0] : q == 1 ? v[1] : q == 2 ? v[2] : v[3];
    return __builtin_amdgcn_readlane(x, e >> 2);
  };
  auto decode = [&](int vb) {
    Tile t;
    t.e = vb / per_e;
    const int rem = vb - t.e * per_e;
    t.m0 = (rem % m_tiles) * kBM;
    t.n0 = (rem / m_tiles) * kBN;
    t.lo = pick(lo4, t.e);
    t.cnt = pick(cnt4, t.e);
    t.ns = (t.cnt + kBK - 1) / kBK;
    return t;
  };
  // the range [v_lo, v_hi) of this XCD: lane j sums the stages of experts
  // 4j .. 4j + 3, a wave scan gives every expert's first unit of work
  int v_lo, v_hi;
  {
    int ns4[4];
    int64_t s4 = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ns4[q] = (cnt4[q] + kBK - 1) / kBK;
      s4 += ns4[q];
    }
    int64_t incl = s4;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int64_t y = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += y;
    }
    const int64_t total = __shfl(incl, kWave - 1, kWave) * per_e;
    // the first tile whose work starts at or after share x of the total
    auto start_of = [&](int x) -> int {
      if (x >= kXcd) return n_all;
      const int64_t t = total * x / kXcd;
      if (t == 0) return 0;
      int64_t c = (incl - s4) * per_e;
      int v = -1;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t hi = c + (int64_t)per_e * ns4[q];
        if (v < 0 && t > c && t <= hi) v = (4 * lane + q) * per_e + (int)((t - c + ns4[q] - 1) / ns4[q]);
        c = hi;
      }
      const uint64_t found = __ballot(v >= 0);   // exactly one lane holds t (0 < t <= total)
      return found ? __shfl(v, __builtin_ctzll(found), kWave) : n_all;
    };
    v_lo = __builtin_amdgcn_readfirstlane(start_of(xcd));
    v_hi = __builtin_amdgcn_readfirstlane(start_of(xcd + 1));
  }
  const int v_first = v_lo + local;

  // The stage stream: every stage of this workgroup's tiles in order (tiles
  // without rows have none), loaded kNS - 1 stages ahead of the one being
  // multiplied, so the next tile's first stages load during the current
  // tile's last stages and its epilogue.  Issue side: the tile being loaded,
  // its next stage, and the lane offsets of its columns.
  int iv = v_first, ist = 0, n_issued = 0;
  Tile it{};
  uint32_t a_off[A_INSTR], b_off[B_INSTR];
  auto seek = [&]() {   // from iv on, the first tile with rows (iv >= v_hi: none)
    for (; iv < v_hi; iv += W) {
      it = decode(iv);
      if (it.ns > 0) break;
    }
    if (iv >= v_hi) return;
    // load p of this wave fills k-rows RPI (wave + 4 p) .. +RPI-1 of its stage
#pragma unroll
    for (int p = 0; p < A_INSTR; ++p) {
      const int kr = A_RPI * (wave + 4 * p) + lane / A_CPR;
      const int col = it.m0 + 8 * ((lane % A_CPR) ^ ((kr & 3) << 2));
      a_off[p] = col < M ? (uint32_t)(kr * lda + col) * 2u : kPast;
    }
#pragma unroll
    for (int p = 0; p < B_INSTR; ++p) {
      const int kr = B_RPI * (wave + 4 * p) + lane / B_CPR;
      const int col = it.n0 + 8 * ((lane % B_CPR) ^ ((kr & 3) << 2));
      b_off[p] = col < N ? (uint32_t)(kr * ldb + col) * 2u : kPast;
    }
  };
  auto issue = [&]() {
    if (iv >= v_hi) return;
    const int64_t r0 = it.lo + (int64_t)ist * kBK;
    const int rows = min(kBK, it.cnt - ist * kBK);
    // descriptors over this stage's rows only: k-rows past them read zeros
    const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(a + r0 * lda), (short)0, __builtin_amdgcn_readfirstlane(rows * lda * 2), kBufferConfig);
    const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(b + r0 * ldb), (short)0, __builtin_amdgcn_readfirstlane(rows * ldb * 2), kBufferConfig);
    const int buf = n_issued % kNS;
    const uint32_t a_lds = __builtin_amdgcn_readfirstlane(lds_address(sA + buf * A_BYTES) + wave * 1024);
    const uint32_t b_lds = __builtin_amdgcn_readfirstlane(lds_address(sB + buf * B_BYTES) + wave * 1024);
#pragma unroll
    for (int p = 0; p < A_INSTR; ++p) dma16(ar, a_lds + p * 4 * 1024, a_off[p]);
#pragma unroll
    for (int p = 0; p < B_INSTR; ++p) dma16(br, b_lds + p * 4 * 1024, b_off[p]);
    ++n_issued;
    if (++ist == it.ns) {
      ist = 0;
      iv += W;
      seek();
    }
  };

  seek();
  for (int i = 0; i < kNS - 1; ++i) issue();

  int g = 0;        // stream index of the stage being multiplied
  int ready = -1;   // stages up to this one are known to have landed
  for (int vb = v_first; vb < v_hi; vb += W) {
    const Tile t = decode(vb);
    f32x16 acc[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[j][i][q] = 0.f;

    for (int st = 0; st < t.ns; ++st, ++g) {
      // this wave's loads of stage g are done once at most the next stage's
      // loads are outstanding (at the end of the stream: once none are)
      if (g > ready) {
        if (n_issued > g + 1) wait_vmcnt<PER>(); else wait_vmcnt<0>();
      }
      stage_barrier();  // stage g visible to all; every wave is done with stage g - 1
      issue();          // stage g + kNS - 1, into the buffer of stage g - 1
      const char* at = sA + (g % kNS) * A_BYTES;
      const char* bt = sB + (g % kNS) * B_BYTES;
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

    // Stores share the load counter, so a wait for stage g issued after
    // them would wait for them too: wait for stage g's loads (issued before
    // them) here, and let the stores complete during stage g.
    if (n_issued > g) {
      if (n_issued > g + 1) wait_vmcnt<PER>(); else wait_vmcnt<0>();
      ready = g;
    }
    // acc[j][i]: gradient row m0 + 64 wm + 32 i + lane % 32, columns
    // n0 + 128 wn + 32 j + 8 q4 + 4 (lane / 32) + {0..3} (zero for an expert
    // without rows).  Stored straight from there, a store instruction would
    // write 32 bytes into each of 32 rows.  The results go out through LDS
    // instead, so that each store writes whole 128-byte pieces of 8 rows:
    // a wave stages one 32 x 64 block at a time in 4 KB of its own, in the
    // ring buffer of the stage it multiplied last (free until the next
    // stage's barrier), and reads it back 16 bytes a lane, 8 lanes a row.
    // In the staged block, 16-byte chunk c of row r sits in slot c ^ (r & 7).
    stage_barrier();   // every wave is done reading that buffer's fragments
    const int slot = (g + kNS - 1) % kNS;
    char* blk = wave < 2 ? sA + slot * A_BYTES + wave * 4096 : sB + slot * B_BYTES + (wave - 2) * 4096;
    bf16_t* out = dw + (int64_t)t.e * M * N;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jp = 0; jp < 2; ++jp) {
        {
          const int r = lane % 32;
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const f32x16& v = acc[2 * jp + jj][i];
              const int c = 4 * jj + q4;
              *(uint2*)(blk + r * 128 + ((c ^ (r & 7)) << 4) + (lane / 32) * 8) =
                  make_uint2(pack_bf16x2(v[4 * q4], v[4 * q4 + 1]), pack_bf16x2(v[4 * q4 + 2], v[4 * q4 + 3]));
            }
        }
        const int m_base = t.m0 + 64 * wm + 32 * i;
        const int n = t.n0 + 128 * wn + 64 * jp + 8 * (lane % 8);
#pragma unroll
        for (int sr = 0; sr < 4; ++sr) {
          const int r = 8 * sr + lane / 8;
          const u32x4 val = *(const u32x4*)(blk + r * 128 + (((lane % 8) ^ (r & 7)) << 4));
          // non-temporal: nothing reads the gradient back here, and written
          // lines left in L2 would evict the operands the next tiles share
          if (m_base + r < M && n < N)
            __builtin_nontemporal_store(val, (u32x4*)(out + (int64_t)(m_base + r) * N + n));
        }
      }
  }
}

// CUs of the current device (256 if the query fails)
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
    return n;
  return 256;
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
  if (M % 4 != 0 || N % 8 != 0 || lda < M || ldb < N) return hipErrorInvalidValue;
  const int m_tiles = (int)ceil_div(M, kBM), n_tiles = (int)ceil_div(N, kBN);
  const int64_t tiles = (int64_t)E * m_tiles * n_tiles;
  if (tiles > 0x7FFFFFFF - 0x10000000) return hipErrorInvalidValue;   // tile indices stay in int
  // persistent: two workgroups per CU at most, a multiple of the XCD count
  const int64_t slots = 2 * (int64_t)device_cus();
  const int64_t grid = round_up(tiles < slots ? tiles : slots, kXcd);
  k_wgrad<<<(unsigned)grid, 256, 0, s>>>(a, lda, M, b, ldb, N, expert_offsets, max_rows, E, dw, m_tiles, n_tiles);
  return hipGetLastError();
}

}  // namespace tre
