// grouped_ffn.hip -- each expert's SwiGLU feed-forward over its own rows.
//
// "Tensor parallelism for inference" (Hugging Face Transformers docs),
// section "Packed strategies": the gate and up projections are one packed
// [E, d, 2I] weight applied as x @ W and split in two along the last
// dimension, gate half first.  The down projection (down_proj, "Expert
// parallelism", section "Overriding plans") is [E, I, d] in the same
// orientation.  Grouped rows of expert e are [offsets[e], offsets[e+1]);
// grouped row r holds token row_token[r] (or row r of an already grouped
// copy x_perm):
//   H[r] = silu(x[row_token[r]] @ Wgu[e][:, :I]) * (x[row_token[r]] @ Wgu[e][:, I:])
//   Y[r] = H[r] @ Wd[e]
//
// bf16 path (MFMA, gfx950), one kernel template with two instances: gate/up
// with the SwiGLU epilogue (output H) and down (output Y), both bf16 with
// float32 accumulation in v_mfma_f32_32x32x16_bf16:
//   * each wave computes 64 rows x 128 weight columns (2 x 4 MFMA tiles);
//     workgroup tiles are 256 x 256 (8 waves in ping-pong, one workgroup per
//     CU) for large experts, 64 x 256 (2 waves, two workgroups per CU) for
//     decode-sized batches and 128 x 256 (4 waves, two workgroups per CU)
//     in between; for gate/up the 256 columns are 128 gate columns and the
//     matching 128 up columns, and each wave holds gate column j and up
//     column j in the same lane, so SwiGLU is elementwise in registers;
//   * k-stages of 32 stream through a ring of LDS buffers filled by buffer
//     loads that write LDS directly; the stages of all tiles of a workgroup
//     form one stream, so the next tile's first stages load while the
//     current tile finishes.  The stage loop is unrolled over the ring, so
//     ring slots and LDS addresses are constants and a stage costs four
//     loads, the LDS reads and the MFMAs plus a handful of scalar
//     instructions;
//   * in the 256-row (ping-pong) products the activation rows of two
//     consecutive k-stages load together, whole 128-byte lines per row;
//   * the gate/up activation loads gather token rows through row_token (the
//     index of each tile is itself fetched into LDS by DMA a tile ahead);
//   * weight rows are n-contiguous and reach the MFMA through the gfx950
//     transposing LDS read ds_read_b64_tr_b16;
//   * persistent grid: each workgroup derives the tile list from the device
//     offsets (no host synchronisation) and walks it round-robin; tiles are
//     ordered expert, then column tile, then row tile, and consecutive tiles
//     go to workgroups of one XCD, so the row tiles that share a weight slice
//     run together on one L2; with four or more rounds of 256-row tiles the
//     last round and a half is handed out by an atomic ticket counter;
//   * with one pair per token the down projection can write the layer
//     output rows itself (routing weight applied, as the combine would).
// float32 path (v_mfma_f32_32x32x2_f32): 64 x 128 tiles of four waves,
// double-buffered k-stages staged through registers into LDS.
#include "common.hpp"

#include <algorithm>
#include <type_traits>

namespace tre {
namespace {

constexpr int kXcd = 8;          // XCDs per MI355X; workgroups are dealt round-robin over them
// column-tiled weights: the columns a gate/up tile takes from each half, and
// a down tile's columns (the forward products' 256-column tiles)
constexpr int kTileGateCols = 128, kTileDownCols = 256;
// byte offset that is always past num_records (a buffer load there returns zeros)
constexpr uint32_t kOutOfRange = 0x80000000u;

// epilogues of the grouped GEMM
constexpr int kEpiPlain = 0;       // Out = A W
constexpr int kEpiSwiglu = 1;      // Out = silu(A Wg) * (A Wu) (gate/up tiles)
constexpr int kEpiSwigluSave = 2;  // as kEpiSwiglu, and Out2 = [A Wg | A Wu] (row stride 2N)
constexpr int kEpiSwigluBwd = 3;   // Out = [dg | du] from dh = A W and Aux = [g | u] (row strides 2N)
constexpr int kEpiPartial = 4;     // Part[split] = A W over the split's k-stages (float32, row stride N)
constexpr int kEpiScatter = 5;     // Out[row_token[r]] = row_w[r] * bf16(A W)[r] (one pair per token)
constexpr int kBwdBlocks = 1;      // column blocks whose g, u the backward epilogue loads together

__device__ __forceinline__ uint2 pack4(const float* f) {
  return make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
}

__device__ __forceinline__ void unpack4(uint2 v, float* f) {
  f[0] = __builtin_bit_cast(float, v.x << 16);
  f[1] = __builtin_bit_cast(float, v.x & 0xFFFF0000u);
  f[2] = __builtin_bit_cast(float, v.y << 16);
  f[3] = __builtin_bit_cast(float, v.y & 0xFFFF0000u);
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

// Split-tail workspace of the ping-pong down projection (float32 words):
// a header (split tiles, pieces per tile), one 4-word record per split tile
// (expert, first row, rows, first column) and kTailPieces partial tiles of
// up to 288 rows (256 + the 32 extra rows of a tall tile) x 256 columns.
constexpr int kTailMaxSplit = 4;   // pieces per split tile, at most
constexpr int kTailPieces = 256;   // pieces in flight, at most
constexpr int kTailHdrWords = 64;
constexpr int kTailPartOff = kTailHdrWords + 4 * kTailPieces;
constexpr int kTailPieceFloats = 288 * 256;
constexpr size_t kTailBytes = ((size_t)kTailPartOff + (size_t)kTailPieces * kTailPieceFloats) * 4;

namespace dma {


// wait for this wave's LDS reads (lgkmcnt 0), not for vector memory
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

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

// Where one tile of the work list sits: its expert, its first grouped row,
// the rows present (at most BM) and its first output column.
struct Tile {
  int e;
  int rows;
  int64_t row0;
  int n0;
};

// The tiles of one workgroup form a single stream of k-stages: stage g of
// the stream lives in ring buffer g % NS, and while stage g is multiplied,
// stages g+1 .. g+NS-1 are in flight, whichever tiles they belong to -- so
// the next tile's first stages load during the current tile's last ones
// and its epilogue.  With row_token, the grouped-row -> token map of the
// next tile is fetched into LDS by DMA one tile ahead, so that entering a
// tile never waits on a plain global load (which would drain the ring).
// (launch bounds: workgroup size and waves per SIMD -- OCC workgroups of
// 2 WM waves per CU need OCC WM / 2 of them, at least one)
template <int EPI, bool BT, int BK, int OCC, int NJ, int WM, int NS, bool PP, bool TL>
__global__ __launch_bounds__(128 * WM, (OCC * WM + 1) / 2) void k_grouped_gemm(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ offsets, int64_t max_rows, int E, int K, int N, int ldw,
    const bf16_t* __restrict__ W, bf16_t* __restrict__ Out, int n_tiles, const int32_t* __restrict__ row_token,
    int64_t a_rows, bf16_t* __restrict__ Out2, const bf16_t* __restrict__ Aux, int n_split_arg,
    float* __restrict__ Part, int32_t* __restrict__ sched, const float* __restrict__ row_w, int wtiled) {
  // (k-split ranges are only used with the lockstep tiles: the ping-pong
  // instances see one range per tile, a constant)
  const int n_split = PP ? 1 : n_split_arg;
  // gate/up tiles: 128 gate columns and the matching 128 up columns
  constexpr bool SWIGLU = EPI == kEpiSwiglu || EPI == kEpiSwigluSave;
  static_assert(!(SWIGLU && BT), "the gate/up weight is only read as [K][2N]");
  typedef Geo<BK, NJ, WM> GE;
  constexpr int BM = GE::BM, WAVES = GE::WAVES;
  constexpr int BNB = GE::BNB;
  constexpr int BNO = SWIGLU ? BNB / 2 : BNB;  // output columns per tile
  constexpr int WCOL = 32 * NJ;                 // weight columns per wave
  static_assert(NS >= 3 && NS <= 5, "a ring of 3 to 5 stages");
  static_assert(BT || (SWIGLU ? BNB == 2 * kTileGateCols : BNB == kTileDownCols),
                "column-tiled weights are blocked for the products' tile width");
  static_assert(BM <= 256, "one index DMA covers 256 rows");
  static_assert(!PP || WAVES == 8, "ping-pong pairs two groups of four waves, one wave of each per SIMD");
  // With kEpiScatter the tile's row -> token map (and row weights) serve
  // the epilogue, not the activation loads: the activations are the
  // grouped rows themselves, and the maps are kept for four tiles (the
  // issue side fetches tile n + 1's while the compute side may still be
  // finishing tile n - 2).
  constexpr bool SCATTER = EPI == kEpiScatter;
  static_assert(!SCATTER || WAVES >= 2, "the row weights are fetched by wave 1");
  constexpr int NSLOT = SCATTER ? 4 : 2;
  // Tall tiles (TL: the ping-pong plain and gate/up products): an expert's
  // last tile also takes up to XR = 32 rows past BM, so that they do not make
  // a tile of their own -- one that would stream the expert's whole weight
  // slice again, and run its whole stage loop, for a few rows.  Waves 0 and 1
  // load the extra 32-row block with one more load each per stage (with
  // row_token, its token indices arrive with the tile's by a second index
  // load).  Each wave multiplies the block with 32 weight columns: its wm-th
  // column block in the plain product; in the gate/up product, 16 of its gate
  // columns and the 16 matching up columns, read as one fragment, so that
  // SwiGLU pairs stay in one lane.  The block costs one MFMA per wave and
  // k-step.
  constexpr bool TALL = TL;
  static_assert(!TL || (PP && (EPI == kEpiPlain || EPI == kEpiSwiglu) && !BT),
                "tall tiles: ping-pong plain or gate/up products only");
  constexpr int XR = TALL ? 32 : 0;
  constexpr int A_STAGE = GE::A_BYTES + XR * BK * 2;  // LDS bytes of an activation stage
  typedef Geo<2 * BK, NJ, WM> GD;  // the activation geometry of a double-stage
  // Activation double-stages (every ping-pong product; the backward's
  // weights read as [N][K] rows keep single stages):
  // the activation rows of two consecutive k-stages arrive together, 128
  // bytes of a row per load lane group (8 rows per DMA instruction), in a
  // ring of two double-stages beside the four-stage weight ring.  A load
  // then asks L2 for whole 128-byte lines instead of half lines: half the
  // requests for the same bytes, and the number of requests a CU can have
  // in flight is what paces these loads.  The activation loads of stages
  // g, g + 1 (g even) are issued with the weight loads of stage g + 1.
  constexpr bool AD = PP;
  static_assert(!AD || (BK == 32 && NS == 4 && WAVES == 8), "double-stages: 32-wide stages, a ring of four");
  constexpr int AD_ROW = 4 * BK;                    // bytes of a row in a double-stage
  constexpr int A_DSTAGE = (BM + XR) * AD_ROW;      // LDS bytes of a double-stage
  constexpr int A_INSTR_D = BM * AD_ROW / 1024 / WAVES;  // activation loads per wave and double-stage
  constexpr int XR_WAVES = XR * AD_ROW / 1024;      // waves with one load of the extra rows
  static_assert(!AD || 2 * A_DSTAGE <= NS * A_STAGE, "the double-stage ring fits the stage ring's LDS");
  __shared__ __attribute__((aligned(1024))) char sA[NS * A_STAGE];
  __shared__ __attribute__((aligned(1024))) char sB[NS * GE::B_BYTES];
  // (tall tiles: the index of rows BM .. BM + XR - 1 arrives by a second
  // 1 KB load, so a slot spans 512 entries)
  __shared__ __attribute__((aligned(1024))) int32_t s_rt[NSLOT][TALL ? 512 : 256];
  __shared__ __attribute__((aligned(1024))) float s_rw[SCATTER ? NSLOT : 1][256];
  __shared__ int s_start[kMaxExperts];
  __shared__ int s_mt[kMaxExperts];
  __shared__ int s_lo[kMaxExperts];
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_wave[WAVES];
  __shared__ int s_ticket[4];  // claimed tail tickets of tiles n = 0, 1, ... in slot n % 4

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / 2, wn = wave % 2;
  const int g16 = lane / 16, L = lane % 16;

  // ---- tile list from the device offsets ----
  int mt = 0;
  if (tid < E) {
    // offsets are int32, so the clamped values fit an int
    MOE_DCHECK(0 <= offsets[tid] && offsets[tid] <= offsets[tid + 1] && offsets[tid + 1] <= max_rows);
    const int lo = (int)clampi<int64_t>(offsets[tid], 0, max_rows);
    const int hi = (int)clampi<int64_t>(offsets[tid + 1], lo, max_rows);
    s_lo[tid] = lo;
    s_cnt[tid] = hi - lo;
    mt = (int)ceil_div(hi - lo, BM);
    if (TALL && mt > 1 && (hi - lo) - (mt - 1) * BM <= XR) mt -= 1;  // the last tile takes the rest
    s_mt[tid] = mt;
  }
  int total_mt = 0;
  const int start = block_exclusive_scan<WAVES>(mt, s_wave, &total_mt);
  if (tid < E) s_start[tid] = start;
  __syncthreads();
#ifdef MOE_DEVICE_CHECKS
  // (device-checked build) every grouped row's token, spread over the grid
  if (row_token) {
    const int64_t n_rows = clampi<int64_t>(offsets[E], 0, max_rows);
    for (int64_t r = (int64_t)blockIdx.x * blockDim.x + tid; r < n_rows; r += (int64_t)gridDim.x * blockDim.x)
      MOE_DCHECK(row_token[r] >= 0 && row_token[r] < a_rows);
  }
#endif
  const int64_t total_tiles = (int64_t)total_mt * n_tiles;
  const int G = gridDim.x;
  const int vb = (blockIdx.x % kXcd) * (G / kXcd) + blockIdx.x / kXcd;
  const int nk = K / BK;
  // Split tail (the ping-pong down projection, with Part pointing to a tail
  // workspace, whole tiles otherwise): when the tiles fill whole rounds of
  // the grid but for t_exc <= G / 2 of them, those last tiles would make a
  // round of their own, with most workgroups idle.  Each is cut instead into
  // tS ranges of k-stages (pieces); a piece writes its float32 partial tile
  // to the workspace, and k_tail_sum adds the pieces of every such tile in
  // order (deterministic) and applies the epilogue.
  constexpr bool TAIL = PP && !BT && (EPI == kEpiPlain || EPI == kEpiScatter);
  int tS = 1;
  int64_t t_full = total_tiles, t_exc = 0;
  if (TAIL && Part != nullptr && n_split == 1 && total_tiles > G && total_tiles % G != 0) {
    const int64_t exc = total_tiles % G;
    const int64_t sp = min<int64_t>(min<int64_t>(kTailMaxSplit, G / exc),
                                    min<int64_t>(kTailPieces / exc, nk / (2 * NS)));
    if (sp >= 2) {
      tS = (int)sp;
      t_exc = exc;
      t_full = total_tiles - exc;
    }
  }
  if (TAIL && Part != nullptr && blockIdx.x == 0 && tid == 0) {
    int32_t* hdr = (int32_t*)Part;
    hdr[0] = (int)t_exc;
    hdr[1] = tS;
  }
  // Work units: each tile's k-stages cut into n_split ranges (1: whole
  // tiles), unit u = tile u / n_split, range u % n_split; or whole tiles
  // followed by the pieces of the split tail.  Consecutive units (one
  // tile's ranges) go to workgroups of one XCD.
  const int64_t total_units = tS > 1 ? t_full + t_exc * tS : total_tiles * n_split;
  if (vb >= total_units) return;  // the whole workgroup: no barrier follows
  const int my_tiles = (int)((total_units - vb + G - 1) / G);  // units of this workgroup
  auto k_begin = [&](int split) { return split * nk / n_split; };
  // unit u: its tile, its range of k-stages [k0, k1), and its piece of a
  // split tail tile (-1: a whole tile or an n_split range)
  auto unit_tile = [&](int64_t u) -> int64_t {
    if (TAIL && tS > 1 && u >= t_full) return t_full + (int)(u - t_full) / tS;
    return u / n_split;
  };
  auto unit_range = [&](int64_t u, int& k0, int& k1) {
    if (TAIL && tS > 1 && u >= t_full) {
      // (whole double-stages: every piece starts at an even stage)
      const int pc = (int)(u - t_full) % tS;
      k0 = AD ? 2 * (pc * (nk / 2) / tS) : pc * nk / tS;
      k1 = AD ? 2 * ((pc + 1) * (nk / 2) / tS) : (pc + 1) * nk / tS;
      return pc;
    }
    const int sp = (int)(u % n_split);
    k0 = k_begin(sp);
    k1 = k_begin(sp + 1);
    return -1;
  };
  // Claimed tail (ping-pong tiles, whole tiles, sched != nullptr, at least
  // four rounds of tiles): the first rs = rounds - 1 tiles of every
  // workgroup are dealt round-robin as above; the rest, units rs G ..
  // total_units - 1, are handed out in order by an atomic ticket counter
  // (*sched, zero at launch), so that workgroups that drew light tiles (an
  // expert's last rows) take more of the tail.  Each tile is still computed
  // by exactly one workgroup, so results do not depend on who takes which.
  // (With fewer rounds the tail is a large share of the tiles, and what its
  // balance gains is lost to weight slices no longer shared in one XCD's L2.)
  const bool dyn = PP && sched != nullptr && n_split == 1 && total_units >= 4 * (int64_t)G && nk >= 2 * NS;
  const int rs = dyn ? (int)(total_units / G) - 1 : 0;
  const int64_t tail0 = (int64_t)rs * G;
  const int64_t n_tail = total_units - tail0;
  int total_stages = 0;
  if (!dyn) {
    for (int i = 0; i < my_tiles; ++i) {
      int k0, k1;
      unit_range(vb + (int64_t)i * G, k0, k1);
      total_stages += k1 - k0;
    }
  } else {
    // tile 0 (dealt); later tiles count in as they become known.  rs >= 3, so
    // the first claim (of tile rs, when tile rs - 2 is entered) is made by
    // the stage loop.
    total_stages = nk;
  }
  // unit of this workgroup's tile n, -1 past its last one
  auto unit_of = [&](int n) -> int64_t {
    if (!dyn) return n < my_tiles ? vb + (int64_t)n * G : -1;
    if (n < rs) return vb + (int64_t)n * G;
    const int t = __builtin_amdgcn_readfirstlane(s_ticket[n & 3]);
    return (t >= 0 && t < n_tail) ? tail0 + t : -1;
  };

  // tile v of the list; `cursor` is the expert of an earlier tile of this
  // workgroup (tiles are visited in increasing order).  Everything is
  // wave-uniform and kept in scalar registers.
  auto decode = [&](int64_t v, int& cursor) {
    while (cursor + 1 < E && (int64_t)__builtin_amdgcn_readfirstlane(s_start[cursor + 1]) * n_tiles <= v) ++cursor;
    const int e = __builtin_amdgcn_readfirstlane(cursor);
    const int e_start = __builtin_amdgcn_readfirstlane(s_start[e]);
    const int e_mt = __builtin_amdgcn_readfirstlane(s_mt[e]);
    const int e_cnt = __builtin_amdgcn_readfirstlane(s_cnt[e]);
    const int e_lo = __builtin_amdgcn_readfirstlane(s_lo[e]);
    const int64_t local = v - (int64_t)e_start * n_tiles;
    const int64_t nt = local / e_mt;
    const int mtile = (int)(local - nt * e_mt);
    Tile t;
    t.e = e;
    t.row0 = (int64_t)e_lo + (int64_t)mtile * BM;
    t.rows = (TALL && mtile == e_mt - 1) ? e_cnt - mtile * BM : min(BM, e_cnt - mtile * BM);
    t.n0 = (int)nt * BNO;
    return t;
  };

  auto col_base = [&](int j) {
    if (SWIGLU) return (j < NJ / 2) ? (WCOL / 2) * wn + 32 * j : BNB / 2 + (WCOL / 2) * wn + 32 * (j - NJ / 2);
    return WCOL * wn + 32 * j;
  };

  // ---- issue side: the tile whose stages are being loaded ----
  // Loop counters are 32-bit: a workgroup's stage count stays far below 2^31
  // (rows * K < 2^31 is checked on the host).
  int i_tile = 0, i_k = 0, i_len = 0;
  int i_cursor = 0;
  Tile inext = decode(unit_tile(vb), i_cursor);  // the tile the issue side enters next
  int64_t inext_u = vb;                           // and its unit
  int total = total_stages;  // stages of the tiles known so far
  // Claiming a ticket (one lane of wave 0): an atomic fetch-add the compiler
  // sees, so that it keeps the returned value's register reserved and waits
  // for the return before the value is used.  It does not count the
  // inline-assembly stage loads, so that wait is vmcnt(0); the compiler
  // places it right after the claim (it moves the ticket to a scalar
  // register), at the start of a read phase, where wave 0's loads in flight
  // are the next stage's (needed by the end of the phase anyway) and the one
  // after.  A few claims per workgroup and launch: measured +0.2-1% on the
  // layer against an inline-assembly claim whose return was covered by the
  // stage waits, which depended on the compiler never touching the ticket's
  // register in between.  The post, NS - 1 stages later, copies the ticket
  // to LDS for every wave.
  int ticket = 0;  // written only by the claim, read only by the post that follows it
  int post_cnt = 0, post_slot = 0;
  auto claim = [&](int n) {
    if (wave == 0 && lane == 0) ticket = __hip_atomic_fetch_add(sched, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    post_cnt = NS - 1;
    post_slot = n & 3;
  };
  auto post = [&]() {
    if (wave == 0 && lane == 0) s_ticket[post_slot] = ticket;
  };
  __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, 0, kBufferConfig);
  __amdgpu_buffer_rsrc_t b_rsrc = a_rsrc;
  uint32_t a_voff[AD ? A_INSTR_D : GE::A_INSTR], b_voff[GE::B_INSTR];
  // tall tiles: this lane's chunk of the extra rows (waves 0, 1; with
  // double-stages waves 0 .. 3)
  uint32_t ax_voff = kOutOfRange;
  // byte offsets of the next stage's k-columns in the activation and weight
  // buffers: scalar, added to every lane's offset by the load itself
  uint32_t ka = 0, kb = 0;
  constexpr uint32_t kAStep = BK * 2;
  // (per tile with column-tiled weights: the tile's block is [K][width])
  uint32_t kb_step = BT ? (uint32_t)BK * 2u : (uint32_t)BK * (uint32_t)ldw * 2u;
  const uint32_t a_lds0 = lds_address(sA) + wave * 1024;
  const uint32_t b_lds0 = lds_address(sB) + wave * 1024;

  // wave 0 copies the token index of grouped rows t.row0 .. t.row0+rows-1
  // into s_rt[slot] (rows past the tile read as 0 and are never used), and
  // with SCATTER wave 1 their weights into s_rw[slot]
  const bool gather = !SCATTER && row_token != nullptr;  // activation row r is token row_token[r]
  auto index_dma = [&](const Tile& t, int slot) {
    // (bases and sizes through readfirstlane, as in enter: scalar operands)
    const int bytes = __builtin_amdgcn_readfirstlane(t.rows * 4);
    if (wave == 0) {
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(row_token + t.row0), (short)0, bytes, kBufferConfig);
      dma16(rs, __builtin_amdgcn_readfirstlane(lds_address(&s_rt[slot][0])), (uint32_t)lane * 16u);
      if constexpr (TALL) {
        // rows 256 .. of a tall tile (none: every lane reads past the buffer)
        const int xbytes = __builtin_amdgcn_readfirstlane(max(t.rows - 256, 0) * 4);
        const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
            uniform_ptr(row_token + t.row0 + min(t.rows, 256)), (short)0, xbytes, kBufferConfig);
        dma16(rx, __builtin_amdgcn_readfirstlane(lds_address(&s_rt[slot][256])), (uint32_t)lane * 16u);
      }
    }
    if constexpr (SCATTER) {
      if (wave == 1) {
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(row_w + t.row0), (short)0, bytes, kBufferConfig);
        dma16(rs, __builtin_amdgcn_readfirstlane(lds_address(&s_rw[slot][0])), (uint32_t)lane * 16u);
      }
    }
  };

  // Buffer descriptors bound the activation rows (this tile's rows, or with
  // row_token the whole token matrix) and this expert's weights: a load past
  // num_records returns zeros.  Activation instruction p of this wave fills
  // rows (wave + WAVES p) RPI + lane / CPR; weight instruction p fills k-rows
  // (wave + WAVES p) BRPI + lane / BCPR.  The lane offsets address k-stage 0;
  // every lane that loads stays inside its buffer up to the last stage.
  auto enter = [&]() {
    const Tile t = inext;
    const int slot = i_tile % NSLOT;
    // (bases and sizes pass through readfirstlane: they are wave-uniform,
    // and saying so keeps the descriptors in scalar registers)
    a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(gather ? (const void*)A : (const void*)(A + t.row0 * K)), (short)0,
        __builtin_amdgcn_readfirstlane(gather ? (int)(a_rows * K * 2) : t.rows * K * 2), kBufferConfig);
    // one expert's weights: [K][ldw] (read transposed by the LDS reads), or
    // with BT [N][K] (rows of k, read like the activations).  Column-tiled
    // weights (wtiled, [K][N] products only): the expert's ldw columns are
    // stored as one block per column tile, block c holding the tile's
    // columns as [K][width] -- for gate/up its gate columns, then the
    // matching up columns -- so a k-stage of a tile is one contiguous run.
    // The descriptor then spans the tile's block only.
    const int64_t w_elems = BT ? (int64_t)N * K : (int64_t)K * ldw;
    const int t_width = SWIGLU ? 2 * min(BNB / 2, N - t.n0) : min(BNB, N - t.n0);  // the tile's weight columns
    const bool tiled = !BT && wtiled;
    const int64_t w_base = (int64_t)t.e * w_elems + (tiled ? (int64_t)K * (SWIGLU ? 2 * t.n0 : t.n0) : 0);
    b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(W + w_base), (short)0,
        __builtin_amdgcn_readfirstlane(tiled ? K * t_width * 2 : (int)(w_elems * 2)), kBufferConfig);
    if (tiled) kb_step = __builtin_amdgcn_readfirstlane((uint32_t)BK * (uint32_t)t_width * 2u);
    // (double-stages: instruction p of this wave fills rows (wave + WAVES p)
    // 8 + lane / 8 with 64 k-values each, chunk lane % 8 of the LDS row)
    constexpr int ARPI = AD ? GD::RPI : GE::RPI, ACPR = AD ? GD::CPR : GE::CPR;
    auto aswz = [](int r) { return AD ? GD::swz(r) : GE::swz(r); };
#pragma unroll
    for (int p = 0; p < (AD ? A_INSTR_D : GE::A_INSTR); ++p) {
      const int r = (wave + WAVES * p) * ARPI + lane / ACPR;
      const int c = (lane % ACPR) ^ aswz(r);
      int64_t src = r;
      if (gather) src = (r < t.rows) ? s_rt[slot][r] : -1;
      a_voff[p] = (r < t.rows && src >= 0 && src < (gather ? a_rows : (int64_t)t.rows))
                      ? (uint32_t)(src * K + c * 8) * 2u
                      : kOutOfRange;
    }
    if constexpr (TALL) {
      // rows BM + ARPI wave .. of the tile (waves 0 .. XW - 1), the A buffer
      // spans t.rows rows
      constexpr int XW = AD ? XR_WAVES : 2;
      const int r = BM + ARPI * wave + lane / ACPR;
      const int c = (lane % ACPR) ^ aswz(r);
      int64_t src = r;
      if (gather) src = (wave < XW && r < t.rows) ? s_rt[slot][r] : -1;
      ax_voff = (wave < XW && r < t.rows && src >= 0 && src < (gather ? a_rows : (int64_t)t.rows))
                    ? (uint32_t)(src * K + c * 8) * 2u
                    : kOutOfRange;
    }
#pragma unroll
    for (int p = 0; p < GE::B_INSTR; ++p) {
      if constexpr (BT) {
        // weight row n of the tile holds its BK k-values like an activation row
        const int nr = (wave + WAVES * p) * GE::RPI + lane / GE::CPR;
        const int c = (lane % GE::CPR) ^ GE::swz(nr);
        const int gn = t.n0 + nr;
        b_voff[p] = gn < N ? (uint32_t)((int64_t)gn * K + c * 8) * 2u : kOutOfRange;
        continue;
      }
      const int kr = (wave + WAVES * p) * GE::BRPI + lane / GE::BCPR;
      const int c = (lane % GE::BCPR) ^ ((kr & 3) << 2);
      const int tc = c * 8;
      int gcol;
      bool ok;
      if (SWIGLU) {
        const int hc = tc % (BNB / 2);   // the gate or up column within the tile
        ok = t.n0 + hc < N;
        gcol = tiled ? ((tc < BNB / 2) ? hc : t_width / 2 + hc) : ((tc < BNB / 2) ? t.n0 + hc : N + t.n0 + hc);
      } else {
        gcol = tiled ? tc : t.n0 + tc;
        ok = t.n0 + tc < N;
      }
      b_voff[p] = ok ? (uint32_t)(kr * (tiled ? t_width : ldw) + gcol) * 2u : kOutOfRange;
    }
    int k0, k1;
    unit_range(inext_u, k0, k1);
    ka = (uint32_t)k0 * kAStep;
    kb = (uint32_t)k0 * kb_step;
    i_len = k1 - k0;
    const int64_t u = unit_of(i_tile + 1);
    if (u >= 0) {
      inext = decode(unit_tile(u), i_cursor);
      inext_u = u;
      if (row_token) index_dma(inext, (i_tile + 1) % NSLOT);
      if (dyn) {
        int u0, u1;
        unit_range(u, u0, u1);
        total += u1 - u0;
        if (i_tile + 2 >= rs) claim(i_tile + 2);
      }
    }
  };

  // load the next stage of the stream into ring slot SLOT (a constant, so
  // every LDS address below is a fixed offset from the wave's base)
  auto issue = [&](auto slot_c) {
    constexpr int SLOT = decltype(slot_c)::value;
    if (i_k == 0) enter();
    if constexpr (AD) {
      // an odd stage of the stream (every tile has an even number of stages
      // and starts at an even one): the activations of this stage and the
      // one before, into double-stage slot SLOT / 2, ahead of the weights
      if constexpr (SLOT % 2 == 1) {
        constexpr int DOFF = (SLOT / 2) * A_DSTAGE;
#pragma unroll
        for (int p = 0; p < A_INSTR_D; ++p)
          dma16s(a_rsrc, a_lds0 + DOFF + p * WAVES * 1024, a_voff[p], ka - kAStep);
        // in every double-stage, tall tile or not, so that waves 0 .. 3
        // always count exactly one load more
        if constexpr (TALL)
          if (wave < XR_WAVES) dma16s(a_rsrc, a_lds0 + DOFF + BM * AD_ROW, ax_voff, ka - kAStep);
      }
    } else {
#pragma unroll
      for (int p = 0; p < GE::A_INSTR; ++p)
        dma16s(a_rsrc, a_lds0 + SLOT * A_STAGE + p * WAVES * 1024, a_voff[p], ka);
      // in every stage, tall tile or not, so that waves 0 and 1 always count
      // exactly one load more per stage (past the tile's rows it fetches nothing)
      if constexpr (TALL)
        if (wave < 2) dma16s(a_rsrc, a_lds0 + SLOT * A_STAGE + GE::A_BYTES, ax_voff, ka);
    }
    // Tall tiles are chosen when an expert holds one or two tiles of rows,
    // so a weight slice is read by about one tile: a stream read once, loaded
    // non-temporal so that it does not evict the activation rows the
    // expert's other column tiles will read (measured: layer -1.5% on the
    // 128-expert layer; with many row tiles per expert, where row tiles
    // share a slice through L2, the same policy was 5% slower).
#pragma unroll
    for (int p = 0; p < GE::B_INSTR; ++p) {
      if constexpr (TALL) dma16s_nt(b_rsrc, b_lds0 + SLOT * GE::B_BYTES + p * WAVES * 1024, b_voff[p], kb);
      else dma16s(b_rsrc, b_lds0 + SLOT * GE::B_BYTES + p * WAVES * 1024, b_voff[p], kb);
    }
    ka += kAStep;
    kb += kb_step;
    if (++i_k == i_len) {
      i_k = 0;
      ++i_tile;
    }
  };

  // ---- compute side ----
  f32x16 acc[NJ][2];
  f32x16 acc_x;           // tall tiles: rows BM .. BM + 31 times the wave's extra columns
  bool cur_tall = false;  // the tile being multiplied has rows past BM
  auto zero_acc = [&]() {
    if constexpr (TALL) {
#pragma unroll
      for (int q = 0; q < 16; ++q) acc_x[q] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[j][i][q] = 0.f;
  };

  struct Frag {
    bf16x8 a[2], b[NJ];
    bf16x8 ax;  // tall tiles: the extra rows
    bf16x8 bx;  // tall tiles: the weight fragment of the extra rows
  };
  // Per-lane LDS addresses of this wave's fragment reads in ring slot 0 at
  // k-step 0.  Every read of the stage loop sits a constant offset from one
  // of them (ring slot, k-step, 32-row block, and for gate/up the up half of
  // the columns), which the read takes as its immediate offset.  The XOR
  // swizzles hide that linearity from the compiler, which otherwise keeps a
  // register or two per read; the empty asm statements make each base an
  // opaque value, computed once.
  constexpr int NFB = SWIGLU ? NJ / 2 : NJ;  // distinct weight-read bases (BT: none, see read_frag)
  uint32_t fa[2], fb[NFB], fax[2] = {0u, 0u}, fbx = 0u;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    // (double-stages: the even stage's chunks; the odd stage's chunk c + 4
    // of a row sits at the address XOR 64, see read_frag)
    fa[ks] = lds_address(sA) + (AD ? GD::a_byte(64 * wm + lane % 32, ks * 2 + lane / 32)
                                   : GE::a_byte(64 * wm + lane % 32, ks * 2 + lane / 32));
    asm("" : "+v"(fa[ks]));
    if constexpr (TALL) {
      fax[ks] = lds_address(sA) + (AD ? GD::a_byte(BM + lane % 32, ks * 2 + lane / 32)
                                      : GE::a_byte(BM + lane % 32, ks * 2 + lane / 32));
      asm("" : "+v"(fax[ks]));
    }
  }
#pragma unroll
  for (int j = 0; j < NFB; ++j) {
    if constexpr (!BT) {
      const int kr = (g16 / 2) * 8 + L / 4;
      const int col = col_base(j) + (g16 % 2) * 16 + 4 * (L % 4);
      fb[j] = lds_address(sB) + GE::b_byte(kr, col >> 3) + ((col >> 2) & 1) * 8;
      asm("" : "+v"(fb[j]));
    }
  }
  if constexpr (TALL && SWIGLU) {
    // the wave's 16 gate columns (WCOL / 2) wn + 16 wm + 0..15 in the extra
    // fragment's first 16 columns, their up columns in its last 16
    const int kr = (g16 / 2) * 8 + L / 4;
    const int col = (WCOL / 2) * wn + 16 * wm + (g16 % 2) * (BNB / 2) + 4 * (L % 4);
    fbx = lds_address(sB) + GE::b_byte(kr, col >> 3) + ((col >> 2) & 1) * 8;
    asm("" : "+v"(fbx));
  } else if constexpr (TALL) {
    // the wave's wm-th column block (selected without indexing the bases at
    // run time, which would put them in scratch memory)
    fbx = fb[0];
#pragma unroll
    for (int j = 1; j < NFB; ++j) fbx = wm == j ? fb[j] : fbx;
    asm("" : "+v"(fbx));
  }
  typedef __attribute__((address_space(3))) const char lds_char;
  auto lds_at = [](uint32_t a) { return (lds_char*)(uintptr_t)a; };
  auto read_a = [&](uint32_t base, int off) { return *(const __attribute__((address_space(3))) bf16x8*)(lds_at(base) + off); };
  auto read_b = [&](uint32_t base, int off) {
    lds_char* p = lds_at(base) + off;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * GE::BROW));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // The activation fragment base of ring slot SLOT.  With double-stages,
  // an odd stage reads chunk c + 4 = c ^ 4 of the rows the even stage reads
  // at chunk c (c < 4), which the swizzle puts at the even stage's address
  // XOR 64 (every other offset added to a base is a multiple of 128); the
  // XOR is issued at each use, so that no second set of bases stays live.
  auto a_base = [&](auto slot_c, uint32_t base) {
    constexpr int SLOT = decltype(slot_c)::value;
    if constexpr (AD && SLOT % 2 == 1) asm volatile("v_xor_b32 %0, 64, %0" : "+v"(base));
    return base;
  };
  // LDS offset of ring slot SLOT's activations, and of the second 32-row block
  auto a_off = [&](auto slot_c) {
    constexpr int SLOT = decltype(slot_c)::value;
    return AD ? (SLOT / 2) * A_DSTAGE : SLOT * A_STAGE;
  };
  constexpr int A_BLK32 = 32 * (AD ? AD_ROW : BK * 2);
  // the stage in ring slot SLOT, k-step ks
  auto read_frag = [&](auto slot_c, int ks, Frag& f) {
    constexpr int SLOT = decltype(slot_c)::value;
    constexpr int B_OFF = SLOT * GE::B_BYTES;
    const uint32_t ab = a_base(slot_c, fa[ks]);
#pragma unroll
    for (int i = 0; i < 2; ++i) f.a[i] = read_a(ab, a_off(slot_c) + i * A_BLK32);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if constexpr (BT) {
        // weight rows held like activation rows (the backward's products)
        f.b[j] = *(const bf16x8*)(sB + B_OFF + GE::a_byte(col_base(j) + lane % 32, ks * 2 + lane / 32));
        continue;
      }
      const bool up = SWIGLU && j >= NJ / 2;  // the up half: BNB / 2 columns = BNB bytes on
      f.b[j] = read_b(fb[up ? j - NJ / 2 : j], B_OFF + ks * 16 * GE::BROW + (up ? BNB : 0));
    }
  };
  // tall tiles: the extra rows' fragment and the weight fragment it meets
  // (gate/up: 16 gate and their 16 up columns; down: the wm-th column
  // block, read a second time), after the stage's other reads
  auto read_x = [&](auto slot_c, int ks, Frag& f) {
    constexpr int SLOT = decltype(slot_c)::value;
    f.ax = read_a(a_base(slot_c, fax[ks]), a_off(slot_c));
    f.bx = read_b(fbx, SLOT * GE::B_BYTES + ks * 16 * GE::BROW);
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[j][i], 0, 0, 0);
  };
  // tall tiles: the extra rows' MFMA of one k-step, after the stage's others
  // (one branch per stage around both k-steps, none between the others)
  auto mma_x = [&](const Frag& f) { acc_x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.bx, f.ax, acc_x, 0, 0, 0); };

  // acc[j][i] holds output row 64 wm + 32 i + lane % 32, columns
  // col_base(j) + 8 q4 + 4 (lane / 32) + {0..3}
  auto epilogue = [&](const Tile& t, int split, int slot) {
    // (the lane index is re-read here, through a volatile asm, so that the
    // compiler does not hoist the epilogue's per-lane column offsets out of
    // the tile loop and hold them in registers across every stage)
    int elane;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(elane));
    const int lr = elane % 32, lc = 4 * (elane / 32);
    // silu(g) u for two outputs, packed: silu(g) = g / (1 + e^-g) with the
    // hardware reciprocal (about 1 ulp in float32, far below the bf16
    // rounding of h)
    auto swiglu2 = [](float g0, float u0, float g1, float u1) {
      return pack_bf16x2(g0 * __builtin_amdgcn_rcpf(1.f + __expf(-g0)) * u0,
                         g1 * __builtin_amdgcn_rcpf(1.f + __expf(-g1)) * u1);
    };
    // With two 4-column groups 8 columns apart in each of lanes l and l + 32
    // (the same row), one lane swap (v_permlane32_swap) gives lane l the
    // first group's 8 consecutive columns and lane l + 32 the second's: one
    // 16-byte store per lane instead of two 8-byte ones.  pk[g][w] is dword w
    // of group g; every lane takes part in the swap.
    auto swap_store = [&](uint32_t (&pk)[2][2], bf16_t* orow, int c, bool ok) {
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const auto sw = __builtin_amdgcn_permlane32_swap(pk[0][w], pk[1][w], false, false);
        pk[0][w] = sw[0];
        pk[1][w] = sw[1];
      }
      if (ok) *(uint4*)(orow + c) = make_uint4(pk[0][0], pk[0][1], pk[1][0], pk[1][1]);
    };
    if constexpr (EPI == kEpiSwiglu) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (64 * wm + 32 * i >= t.rows) continue;  // (wave-uniform: the whole block is past the rows)
        const int r = 64 * wm + 32 * i + lr;
        bf16_t* orow = Out + (t.row0 + r) * N;
#pragma unroll
        for (int j = 0; j < NJ / 2; ++j)
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            // groups q4 = 2 p, 2 p + 1 (columns 8 q4 + lc + 0..3)
            uint32_t pk[2][2];
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
              for (int w = 0; w < 2; ++w) {
                const int q = 4 * (2 * p + g) + 2 * w;
                pk[g][w] = swiglu2(acc[j][i][q], acc[j + NJ / 2][i][q], acc[j][i][q + 1], acc[j + NJ / 2][i][q + 1]);
              }
            const int c = t.n0 + (WCOL / 2) * wn + 32 * j + 16 * p + 2 * lc;
            swap_store(pk, orow, c, r < t.rows && c < N);
          }
      }
    } else if constexpr (EPI == kEpiPlain || EPI == kEpiScatter) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (64 * wm + 32 * i >= t.rows) continue;  // (wave-uniform)
        const int r = 64 * wm + 32 * i + lr;
        bf16_t* orow = Out + (t.row0 + r) * N;
        bool ok = r < t.rows;
        float wr = 0.f;
        if constexpr (EPI == kEpiScatter) {
          // the row's token gets the row rounded to bf16 times its routing
          // weight, rounded again (what the combine computes for one pair);
          // the index slot holds zeros past the tile's rows
          const int tok = s_rt[slot][r];
          wr = s_rw[slot][r];
          ok = ok && tok >= 0 && tok < a_rows;
          orow = Out + (int64_t)(ok ? tok : 0) * N;
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            uint32_t pk[2][2];
#pragma unroll
            for (int g = 0; g < 2; ++g) {
              const int q = 4 * (2 * p + g);
              const uint2 y = make_uint2(pack_bf16x2(acc[j][i][q], acc[j][i][q + 1]),
                                         pack_bf16x2(acc[j][i][q + 2], acc[j][i][q + 3]));
              if constexpr (EPI == kEpiScatter) {
                float f[4];
                unpack4(y, f);
#pragma unroll
                for (int v = 0; v < 4; ++v) f[v] = fmaf(wr, f[v], 0.f);
                const uint2 z = pack4(f);
                pk[g][0] = z.x;
                pk[g][1] = z.y;
              } else {
                pk[g][0] = y.x;
                pk[g][1] = y.y;
              }
            }
            const int c = t.n0 + WCOL * wn + 32 * j + 16 * p + 2 * lc;
            swap_store(pk, orow, c, ok && c < N);
          }
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (EPI == kEpiSwiglu || EPI == kEpiPlain || EPI == kEpiScatter) break;
      const int r = 64 * wm + 32 * i + lr;
      if (r >= t.rows) continue;
      bf16_t* orow = Out + (t.row0 + r) * N;
      if (SWIGLU) {
#pragma unroll
        for (int j = 0; j < NJ / 2; ++j)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int c = t.n0 + (WCOL / 2) * wn + 32 * j + 8 * q4 + lc;
            if (c >= N) continue;
            uint32_t packed[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              float hv[2];
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const float gt = acc[j][i][4 * q4 + 2 * h2 + u], up = acc[j + NJ / 2][i][4 * q4 + 2 * h2 + u];
                // silu(g) = g / (1 + e^-g), with the hardware reciprocal
                // (about 1 ulp in float32, far below the bf16 rounding of h)
                hv[u] = gt * __builtin_amdgcn_rcpf(1.f + __expf(-gt)) * up;
              }
              packed[h2] = pack_bf16x2(hv[0], hv[1]);
            }
            *(uint2*)(orow + c) = make_uint2(packed[0], packed[1]);
            if constexpr (EPI == kEpiSwigluSave) {
              // the pre-activations too: gate at column c, up at column N + c
              bf16_t* srow = Out2 + (t.row0 + r) * 2 * N;
              float gq[4], uq[4];
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                gq[v] = acc[j][i][4 * q4 + v];
                uq[v] = acc[j + NJ / 2][i][4 * q4 + v];
              }
              *(uint2*)(srow + c) = pack4(gq);
              *(uint2*)(srow + N + c) = pack4(uq);
            }
          }
      } else if constexpr (EPI == kEpiPartial) {
        // this range's float32 partial sums of the row
        float* prow = Part + ((int64_t)split * max_rows + t.row0 + r) * N;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int c = t.n0 + WCOL * wn + 32 * j + 8 * q4 + lc;
            if (c >= N) continue;
            *(f32x4*)(prow + c) = f32x4{acc[j][i][4 * q4], acc[j][i][4 * q4 + 1], acc[j][i][4 * q4 + 2],
                                        acc[j][i][4 * q4 + 3]};
          }
      } else if constexpr (EPI == kEpiScatter) {
        // the row's token gets the row rounded to bf16 times its routing
        // weight, rounded again (what the combine computes for one pair)
        const int tok = s_rt[slot][r];
        const float wr = s_rw[slot][r];
        if (tok < 0 || tok >= a_rows) continue;
        bf16_t* trow = Out + (int64_t)tok * N;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int c = t.n0 + WCOL * wn + 32 * j + 8 * q4 + lc;
            if (c >= N) continue;
            float f[4];
            unpack4(make_uint2(pack_bf16x2(acc[j][i][4 * q4], acc[j][i][4 * q4 + 1]),
                               pack_bf16x2(acc[j][i][4 * q4 + 2], acc[j][i][4 * q4 + 3])),
                    f);
#pragma unroll
            for (int v = 0; v < 4; ++v) f[v] = fmaf(wr, f[v], 0.f);
            *(uint2*)(trow + c) = pack4(f);
          }
      } else if constexpr (EPI == kEpiSwigluBwd) {
        // acc is dh; with the saved pre-activations g, u of the row:
        // dg = dh u s (1 + g (1 - s)), du = dh g s, s = sigmoid(g)
        const bf16_t* grow = Aux + (t.row0 + r) * 2 * N;
        bf16_t* drow = Out + (t.row0 + r) * 2 * N;
        // g, u of one column block first (one round trip for its eight
        // loads), then its arithmetic
#pragma unroll
        for (int j0 = 0; j0 < NJ; j0 += kBwdBlocks) {
          uint2 gq[kBwdBlocks][4], uq[kBwdBlocks][4];
#pragma unroll
          for (int jj = 0; jj < kBwdBlocks; ++jj)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const int c = t.n0 + WCOL * wn + 32 * (j0 + jj) + 8 * q4 + lc;
              gq[jj][q4] = c < N ? *(const uint2*)(grow + c) : make_uint2(0u, 0u);
              uq[jj][q4] = c < N ? *(const uint2*)(grow + N + c) : make_uint2(0u, 0u);
            }
#pragma unroll
          for (int jj = 0; jj < kBwdBlocks; ++jj)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int j = j0 + jj;
            const int c = t.n0 + WCOL * wn + 32 * j + 8 * q4 + lc;
            if (c >= N) continue;
            float g[4], u[4], dg[4], du[4];
            unpack4(gq[jj][q4], g);
            unpack4(uq[jj][q4], u);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float dh = acc[j][i][4 * q4 + v];
              const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-g[v]));
              dg[v] = dh * u[v] * sg * (1.f + g[v] * (1.f - sg));
              du[v] = dh * g[v] * sg;
            }
            *(uint2*)(drow + c) = pack4(dg);
            *(uint2*)(drow + N + c) = pack4(du);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int c = t.n0 + WCOL * wn + 32 * j + 8 * q4 + lc;
            if (c >= N) continue;
            const uint32_t p0 = pack_bf16x2(acc[j][i][4 * q4], acc[j][i][4 * q4 + 1]);
            const uint32_t p1 = pack_bf16x2(acc[j][i][4 * q4 + 2], acc[j][i][4 * q4 + 3]);
            *(uint2*)(orow + c) = make_uint2(p0, p1);
          }
      }
    }
    if constexpr (TALL) {
      // the extra rows: acc_x holds row BM + lane % 32, the wave's wm-th
      // column block
      const int r = BM + lr;
      if (SWIGLU && t.rows > BM) {
        // acc_x[4 q4 + v] is gate column (WCOL / 2) wn + 16 wm + 8 q4 + lc + v
        // for q4 < 2 and the matching up column for q4 + 2
        bf16_t* orow = Out + (t.row0 + r) * N;
        uint32_t pk[2][2];
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            const int q = 4 * g + 2 * w;
            pk[g][w] = swiglu2(acc_x[q], acc_x[q + 8], acc_x[q + 1], acc_x[q + 9]);
          }
        const int c = t.n0 + (WCOL / 2) * wn + 16 * wm + 2 * lc;
        swap_store(pk, orow, c, r < t.rows && c < N);
      } else if (!SWIGLU && t.rows > BM) {
        // the wave's wm-th column block
        bf16_t* orow = Out + (t.row0 + r) * N;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          uint32_t pk[2][2];
#pragma unroll
          for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int w = 0; w < 2; ++w) {
              const int q = 4 * (2 * p + g) + 2 * w;
              pk[g][w] = pack_bf16x2(acc_x[q], acc_x[q + 1]);
            }
          const int c = t.n0 + WCOL * wn + 32 * wm + 16 * p + 2 * lc;
          swap_store(pk, orow, c, r < t.rows && c < N);
        }
      }
    }
  };

  // A piece of a split tail tile: its float32 partial tile (the tile's rows,
  // all BNB columns, tall rows included) goes to piece slot xt tS + piece
  // of the tail workspace; piece 0 records where the tile lies.
  auto tail_piece = [&](const Tile& t, int64_t xt, int piece) {
    if constexpr (TAIL) {
      static_assert(BM + XR <= 288 && BNB == 256, "the tail workspace holds 288 x 256 partial tiles");
      int elane;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(elane));
      const int lr = elane % 32, lc = 4 * (elane / 32);
      if (piece == 0 && tid == 0) {
        int32_t* rec = (int32_t*)Part + kTailHdrWords + 4 * xt;
        rec[0] = t.e;
        rec[1] = (int)t.row0;
        rec[2] = t.rows;
        rec[3] = t.n0;
      }
      float* pt = Part + kTailPartOff + ((int64_t)xt * tS + piece) * kTailPieceFloats;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 64 * wm + 32 * i + lr;
        if (r >= t.rows) continue;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            *(f32x4*)(pt + r * BNB + WCOL * wn + 32 * j + 8 * q4 + lc) =
                f32x4{acc[j][i][4 * q4], acc[j][i][4 * q4 + 1], acc[j][i][4 * q4 + 2], acc[j][i][4 * q4 + 3]};
      }
      if (TALL && t.rows > BM && BM + lr < t.rows) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *(f32x4*)(pt + (BM + lr) * BNB + WCOL * wn + 32 * wm + 8 * q4 + lc) =
              f32x4{acc_x[4 * q4], acc_x[4 * q4 + 1], acc_x[4 * q4 + 2], acc_x[4 * q4 + 3]};
      }
    }
  };

  // ---- the stage stream ----
  // Stage g of the stream lives in ring slot g % NS.  The compute side walks
  // its tiles; within a tile the stages run through NS copies of the stage
  // body, one per ring slot, entered at the slot of the tile's first stage
  // (so every slot index, LDS address and load count is a constant), and the
  // epilogue runs once per tile after its last stage.  Every tile has at
  // least NS - 1 stages (the host guarantees it), so the token index of the
  // next tile, fetched when a tile is entered, has landed and is visible by
  // the time the next tile is entered.
  auto barrier = [&]() { stage_barrier(); };
  if (row_token) {
    // the first tile's index, before anything else is in flight
    index_dma(inext, 0);
    wait_vmcnt<0>();
    barrier();
  }
  issue(std::integral_constant<int, 0>{});
  if (1 < total) issue(std::integral_constant<int, 1>{});
  if constexpr (NS > 3) {
    if (2 < total) issue(std::integral_constant<int, 2>{});
  }
  if constexpr (NS > 4) {
    if (3 < total) issue(std::integral_constant<int, 3>{});
  }

  int g = 0;
  int c_cursor = 0;
  Tile cur = decode(unit_tile(vb), c_cursor);
  int64_t cur_u = vb;
  Frag f0, f1;
  zero_acc();

  // One stage of the stream in ring slot SLOT; returns false after the
  // tile's last stage.
  auto stage = [&](auto slot_c, bool active, int& left) {
    constexpr int SLOT = decltype(slot_c)::value;
    constexpr int ISSUE = (SLOT + NS - 1) % NS;  // the slot stage g + NS - 1 lands in
    const bool more = g + NS - 1 < total;
    if constexpr (!PP) {
      // this wave's loads of stage g are done (NS - 2 later stages may still
      // be in flight); after the barrier every wave's are, and every wave is
      // done reading stage g - 1, whose slot then receives stage g + NS - 1
      if (g + NS - 2 < total) wait_vmcnt<(NS - 2) * GE::PER_STAGE>();
      else wait_vmcnt<0>();
      barrier();
      if (more) issue(std::integral_constant<int, ISSUE>{});
      // all of the stage's fragments first, then its multiplications: the
      // reads of the second k-step are in flight during the first k-step's
      // MFMAs.  A wave whose 64 rows are all past the tile's rows has nothing
      // to multiply.
      if (active) {
        read_frag(slot_c, 0, f0);
        read_frag(slot_c, 1, f1);
        if (TALL && cur_tall) {
          read_x(slot_c, 0, f0);
          read_x(slot_c, 1, f1);
        }
        __builtin_amdgcn_sched_barrier(0);
        mma(f0);
        mma(f1);
        if (TALL && cur_tall) {
          mma_x(f0);
          mma_x(f1);
        }
      }
    } else {
      // Ping-pong: waves 0-3 and waves 4-7 (one of each per SIMD) run the
      // same body -- read the stage's fragments (and issue the loads of stage
      // g + NS - 1), barrier, multiply, barrier -- with waves 4-7 one barrier
      // behind, so that on every SIMD one wave multiplies while the other
      // reads.  Stage g is read by waves 0-3 between barriers 2g and 2g+1 and
      // by waves 4-7 between 2g+1 and 2g+2; its slot is refilled (with stage
      // g + NS) in the read phase of stage g + 1, which starts after barrier
      // 2g + 2.  Each wave waits for its own loads of stage g + 1 before the
      // barrier that ends its read phase of stage g, so every wave's share of
      // stage g + 1 has landed before barrier 2g + 2.
      if (more) issue(std::integral_constant<int, ISSUE>{});
      // a wave whose 64 rows are all past the tile's rows has nothing to
      // multiply: its SIMD then serves the other group alone (tiles of an
      // expert's last rows run up to twice as fast)
      if (active) {
        read_frag(slot_c, 0, f0);
        read_frag(slot_c, 1, f1);
        if (TALL && cur_tall) {
          read_x(slot_c, 0, f0);
          read_x(slot_c, 1, f1);
        }
      }
      if constexpr (AD) {
        // Double-stages: stage g + 1 is the weights issued two phases ago and
        // the activations issued with them (g even) or in the last phase (g
        // odd).  Issued since: g even -- the last phase's weights, this
        // phase's activations and weights; g odd -- the last phase's weights
        // and this phase's.  (Tall tiles: waves 0 .. 3 load one more
        // activation instruction per double-stage.)
        constexpr int NW = GE::B_INSTR;
        if (!more) {
          wait_vmcnt<0>();
        } else if constexpr (SLOT % 2 == 0) {
          if (TALL && wave < XR_WAVES) wait_vmcnt<2 * NW + A_INSTR_D + 1>();
          else wait_vmcnt<2 * NW + A_INSTR_D>();
        } else {
          wait_vmcnt<2 * NW>();
        }
      } else if (more) {
        // (tall tiles: waves 0 and 1 issue one load more per stage)
        if (TALL && wave < 2) wait_vmcnt<(NS - 2) * (GE::PER_STAGE + 1)>();
        else wait_vmcnt<(NS - 2) * GE::PER_STAGE>();
      } else {
        wait_vmcnt<0>();
      }
      if (post_cnt > 0 && --post_cnt == 0) post();
      wait_lgkm0();
      barrier();
      if (active) {
        __builtin_amdgcn_s_setprio(1);
        mma(f0);
        mma(f1);
        if (TALL && cur_tall) {
          mma_x(f0);
          mma_x(f1);
        }
        __builtin_amdgcn_s_setprio(0);
      }
      barrier();
    }
    ++g;
    return --left > 0;
  };

  if constexpr (PP) {
    // waves 4-7 start one barrier behind (see the stage body).  Stage 0 has
    // landed once at most the loads of stages 1 and 2 are outstanding (with
    // double-stages: the weights of stages 1 and 2, issued after stage 0's
    // activations).
    if (AD && 2 < total) wait_vmcnt<2 * GE::B_INSTR>();
    else if (AD) wait_vmcnt<0>();
    else wait_vmcnt<(NS - 2) * GE::PER_STAGE>();
    barrier();
    if (wave >= 4) barrier();
  }
  for (int c_tile = 0;; ++c_tile) {
    // A wave whose 64 rows are all past the tile's rows has nothing to
    // multiply -- except in the ping-pong down projection, where a tile of an
    // expert's last rows then finishes with its full sibling on the same
    // weight slice instead of running ahead of it, and the two keep sharing
    // the slice's stages in L2 (measured: the projection 1.4-4.4% faster).
    constexpr bool kKeepPace = PP && (EPI == kEpiPlain || EPI == kEpiScatter);
    const bool active = kKeepPace || 64 * wm < cur.rows;
    cur_tall = TALL && cur.rows > BM;
    int cur_k0, cur_k1;
    const int cur_piece = unit_range(cur_u, cur_k0, cur_k1);
    int left = cur_k1 - cur_k0;
    // the unrolled ring, entered at the slot of the tile's first stage: the
    // copies before it are skipped in the first round only (one entry, so
    // the loop stays reducible and its control flow uniform)
    int first = g % NS;
    while (true) {
      if (first <= 0 && !stage(std::integral_constant<int, 0>{}, active, left)) break;
      if (first <= 1 && !stage(std::integral_constant<int, 1>{}, active, left)) break;
      if constexpr (NS > 2) {
        if (first <= 2 && !stage(std::integral_constant<int, 2>{}, active, left)) break;
      }
      if constexpr (NS > 3) {
        if (first <= 3 && !stage(std::integral_constant<int, 3>{}, active, left)) break;
      }
      if constexpr (NS > 4) {
        if (first <= 4 && !stage(std::integral_constant<int, 4>{}, active, left)) break;
      }
      first = 0;
    }
    if (TAIL && cur_piece >= 0)
      tail_piece(cur, unit_tile(cur_u) - t_full, cur_piece);
    else
      epilogue(cur, (int)(cur_u % n_split), c_tile % NSLOT);
    zero_acc();
    const int64_t u = unit_of(c_tile + 1);
    if (u < 0) break;
    cur = decode(unit_tile(u), c_cursor);
    cur_u = u;
  }
  if constexpr (PP) {
    if (wave < 4) barrier();
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
// Tiles of 64 output rows x 128 columns in k-stages of 64 (the weight
// gradients: stages of 32 rows), four waves (2 x 2) of 32 rows x 64 columns,
// each two 32 x 32 blocks of v_mfma_f32_32x32x2_f32.
// That MFMA takes A (32 x 2) with A[i][k] in lane i + 32 k and B (2 x 32)
// with B[k][j] in lane j + 32 k, and register q of lane l of its 32 x 32
// float32 result holds row 8 (q / 4) + 4 (l / 32) + q % 4, column l % 32.
// Stages are double-buffered in LDS: the next stage's global loads are in
// registers while the current one is multiplied, and one barrier a stage
// separates the two.  At the sizes this path serves a stage waits about one
// memory round trip for its loads, so the products take deep stages: half as
// many round trips as 32-wide ones.  Rows past an operand's end load as zeros.
//
// Operands in LDS, by how they lie in memory:
//   A rows  [64][97]  (the grouped rows, k contiguous);
//   A^T     [32][96]  (the weight gradient's contraction over an expert's
//                      rows: k = row, the output rows contiguous);
//   B       [64][160] (weights [K][ldw], columns contiguous; the weight
//                      gradient's second operand: [32][160]);
//   B^T     [128][97] (weights read as [N][K], k contiguous: the backward's
//                      products with Wd^T and Wgu^T).
// The pads put the two k-halves of an MFMA operand (lanes 0-31, 32-63) on
// different LDS banks (64 banks of 4 bytes: row i of a k-contiguous operand
// starts at bank 33 i mod 64).
constexpr int kF32Rows = 64, kF32Cols = 128;
constexpr int kF32K = 64;    // k-stage depth of the products
constexpr int kF32WK = 32;   // rows per stage of the weight gradients' contraction
constexpr int kF32Epi = 0, kF32Swiglu = 1, kF32SwigluSave = 2, kF32SwigluBwd = 3;

struct F32Stage {
  static constexpr int LDA = kF32K + 33, LDAT = kF32Rows + 32, LDB = kF32Cols + 32, LDBT = kF32K + 33;
  static constexpr int A_FLOATS = kF32Rows * LDA;                                  // A rows
  static constexpr int B_FLOATS = kF32K * LDB > kF32Cols * LDBT ? kF32K * LDB : kF32Cols * LDBT;
  static constexpr int WA_FLOATS = kF32WK * LDAT, WB_FLOATS = kF32WK * LDB;        // the weight gradients
};

// One stage's MFMAs over KD k-values: a wave's rows 32 wm.., its two column
// blocks cb0, cb1.
template <bool AT, bool BT, int KD>
__device__ __forceinline__ void f32_stage_mma(const float* sA, const float* sB, int wm, int cb0, int cb1, int lane,
                                              f32x16& acc0, f32x16& acc1) {
  typedef F32Stage S;
  const int i = 32 * wm + lane % 32, kh = lane / 32, j = lane % 32;
#pragma unroll
  for (int kk = 0; kk < KD / 2; ++kk) {
    const int k = 2 * kk + kh;
    const float av = AT ? sA[k * S::LDAT + i] : sA[i * S::LDA + k];
    const float b0 = BT ? sB[(cb0 + j) * S::LDBT + k] : sB[k * S::LDB + cb0 + j];
    const float b1 = BT ? sB[(cb1 + j) * S::LDBT + k] : sB[k * S::LDB + cb1 + j];
    acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av, b0, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av, b1, acc1, 0, 0, 0);
  }
}

// The grouped products: row tiles of each expert's grouped rows, numbered
// expert by expert from the device offsets, times column tiles.
//   kF32Epi:        Out = A W                            (N columns)
//   kF32Swiglu:     Out = silu(A Wg) * (A Wu)            (W = [Wg | Wu], 2N columns; a tile takes 64 gate
//                                                          columns and the matching 64 up columns, and a
//                                                          wave's two blocks are gate columns j and up
//                                                          columns j, so each pair meets in one register)
//   kF32SwigluSave: as kF32Swiglu, and Out2 = [A Wg | A Wu] (row stride 2N)
//   kF32SwigluBwd:  Out = [dg | du] (row stride 2N) from dh = A W and Aux = [g | u]:
//                   dg = dh u s (1 + g (1 - s)), du = dh g s, s = sigmoid(g)
// BT: W is read as [N][K] (row n holds column n of the product's weight).
template <int EPI, bool BT>
__global__ __launch_bounds__(256) void k_grouped_gemm_f32(const float* __restrict__ A,
                                                          const int32_t* __restrict__ offsets, int64_t max_rows,
                                                          int E, int K, int N, const float* __restrict__ W,
                                                          float* __restrict__ Out, float* __restrict__ Out2,
                                                          const float* __restrict__ Aux) {
  constexpr bool GU = EPI == kF32Swiglu || EPI == kF32SwigluSave;   // gate/up column pairs
  static_assert(!(GU && BT), "the gate/up weight is read as [K][2N]");
  constexpr int BM = kF32Rows, BN = kF32Cols, BK = kF32K;
  typedef F32Stage S;
  __shared__ float sA[2][S::A_FLOATS];
  __shared__ __attribute__((aligned(16))) float sB[2][S::B_FLOATS];
  __shared__ int s_wave[4];
  __shared__ int s_tile[3];  // expert, first grouped row, rows
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave / 2, wn = wave % 2;

  // this workgroup's row tile
  int mt = 0, lo = 0, cnt = 0;
  if (tid < E) {
    MOE_DCHECK(0 <= offsets[tid] && offsets[tid] <= offsets[tid + 1] && offsets[tid + 1] <= max_rows);
    lo = (int)clampi<int64_t>(offsets[tid], 0, max_rows);
    cnt = (int)clampi<int64_t>(offsets[tid + 1], lo, max_rows) - lo;
    mt = (int)ceil_div(cnt, BM);
  }
  int total = 0;
  const int before = block_exclusive_scan<4>(mt, s_wave, &total);
  const int u = (int)blockIdx.x;
  if (u >= total) return;  // (the same for the whole workgroup)
  if (tid < E && before <= u && u < before + mt) {
    s_tile[0] = tid;
    s_tile[1] = lo + (u - before) * BM;
    s_tile[2] = min(BM, cnt - (u - before) * BM);
  }
  __syncthreads();
  const int e = s_tile[0], r0 = s_tile[1], rows = s_tile[2];
  const int ldw = BT ? K : GU ? 2 * N : N;
  const int n0 = (int)blockIdx.y * (GU ? BN / 2 : BN);
  const float* We = W + (int64_t)e * K * (GU ? 2 * N : N);

  // the weight column of LDS column cb (a multiple of 4), or -1 past N
  auto gcol = [&](int cb) -> int {
    if (GU) return cb < BN / 2 ? n0 + cb : N + n0 + cb - BN / 2;
    return n0 + cb < N ? n0 + cb : -1;
  };
  // a stage: 64 rows x BK of A (BK / 4 vectors a row), and BK k-rows x 128
  // columns of W (or, BT, 128 weight rows x BK)
  constexpr int VA = BM * BK / 4 / 256, VB = BK * BN / 4 / 256, VR = BK / 4;   // vectors a thread / a k-run
  f32x4 ra[VA], rb[VB];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < VA; ++i) {
      const int q = tid + 256 * i, row = q / VR, c = 4 * (q % VR);
      ra[i] = row < rows ? *(const f32x4*)(A + (int64_t)(r0 + row) * K + k0 + c) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < VB; ++i) {
      const int q = tid + 256 * i;
      if (BT) {   // 128 weight rows (the product's columns) x BK k
        const int n = q / VR, c = 4 * (q % VR);
        rb[i] = n0 + n < N ? *(const f32x4*)(We + (int64_t)(n0 + n) * ldw + k0 + c) : f32x4{0.f, 0.f, 0.f, 0.f};
      } else {    // BK k-rows x 128 columns
        const int k = q / 32, col = gcol(4 * (q % 32));
        rb[i] = col >= 0 ? *(const f32x4*)(We + (int64_t)(k0 + k) * ldw + col) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < VA; ++i) {
      const int q = tid + 256 * i, row = q / VR, c = 4 * (q % VR);
#pragma unroll
      for (int j = 0; j < 4; ++j) sA[buf][row * S::LDA + c + j] = ra[i][j];
    }
#pragma unroll
    for (int i = 0; i < VB; ++i) {
      const int q = tid + 256 * i;
      if (BT) {
        const int n = q / VR, c = 4 * (q % VR);
#pragma unroll
        for (int j = 0; j < 4; ++j) sB[buf][n * S::LDBT + c + j] = rb[i][j];
      } else {
        *(f32x4*)&sB[buf][(q / 32) * S::LDB + 4 * (q % 32)] = rb[i];
      }
    }
  };
  // a wave's two column blocks in LDS
  const int cb0 = GU ? 32 * wn : 64 * wn, cb1 = GU ? BN / 2 + 32 * wn : 64 * wn + 32;
  f32x16 acc0 = {}, acc1 = {};
  const int nk = K / BK;
  load(0);
  store(0);
  __syncthreads();
  for (int st = 0; st < nk; ++st) {
    const int buf = st & 1;
    if (st + 1 < nk) load((st + 1) * BK);
    f32_stage_mma<false, BT, BK>(sA[buf], sB[buf], wm, cb0, cb1, lane, acc0, acc1);
    if (st + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }
  // epilogue: register q of this lane is row 8 (q / 4) + 4 (lane / 32) + q % 4 of the wave's 32 rows
  const int col = lane % 32;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int r = 32 * wm + 8 * (q / 4) + 4 * (lane / 32) + q % 4;
    if (r >= rows) continue;
    const int64_t gr = r0 + r;
    if constexpr (GU) {
      const int n = n0 + 32 * wn + col;
      const float g = acc0[q], up = acc1[q];
      Out[gr * N + n] = g / (1.f + expf(-g)) * up;
      if (EPI == kF32SwigluSave) {
        Out2[gr * 2 * N + n] = g;
        Out2[gr * 2 * N + N + n] = up;
      }
    } else {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int n = n0 + (b ? cb1 : cb0) + col;
        const float v = b ? acc1[q] : acc0[q];
        if (n >= N) continue;
        if (EPI == kF32SwigluBwd) {
          const float g = Aux[gr * 2 * N + n], up = Aux[gr * 2 * N + N + n];
          const float sg = 1.f / (1.f + expf(-g));
          Out[gr * 2 * N + n] = v * up * sg * (1.f + g * (1.f - sg));
          Out[gr * 2 * N + N + n] = v * g * sg;
        } else {
          Out[gr * N + n] = v;
        }
      }
    }
  }
}

// Per-expert weight gradients dW[e] = A_e^T B_e [M][N] ("Expert parallelism",
// "Combining with FSDP2": an expert's gradient sums over every row it served,
// and is zero when it served none), the contraction over expert e's grouped
// rows (A [rows][lda], B [rows][ldb]) in stages of 32 rows; one workgroup per
// (expert, 64-row block, 128-column block) of dW.
__global__ __launch_bounds__(256) void k_wgrad_f32(const float* __restrict__ A, int lda, int M,
                                                   const float* __restrict__ B, int ldb, int N,
                                                   const int32_t* __restrict__ offsets, int64_t max_rows,
                                                   int m_tiles, int n_tiles, float* __restrict__ dW) {
  constexpr int BM = kF32Rows, BN = kF32Cols, BK = kF32WK;
  typedef F32Stage S;
  __shared__ __attribute__((aligned(16))) float sA[2][S::WA_FLOATS];
  __shared__ __attribute__((aligned(16))) float sB[2][S::WB_FLOATS];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave / 2, wn = wave % 2;
  const int per_e = m_tiles * n_tiles;
  const int e = (int)blockIdx.x / per_e, rem = (int)blockIdx.x % per_e;
  const int m0 = (rem % m_tiles) * BM, n0 = (rem / m_tiles) * BN;
  MOE_DCHECK(0 <= offsets[e] && offsets[e] <= offsets[e + 1] && offsets[e + 1] <= max_rows);
  const int64_t lo = clampi<int64_t>(offsets[e], 0, max_rows);
  const int cnt = (int)(clampi<int64_t>(offsets[e + 1], lo, max_rows) - lo);

  f32x4 ra[2], rb[4];
  auto load = [&](int k0) {   // rows k0 .. k0 + 31 of the expert
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 256 * i, kr = q / 16, m = m0 + 4 * (q % 16);
      ra[i] = (k0 + kr < cnt && m < M) ? *(const f32x4*)(A + (lo + k0 + kr) * lda + m) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i, kr = q / 32, n = n0 + 4 * (q % 32);
      rb[i] = (k0 + kr < cnt && n < N) ? *(const f32x4*)(B + (lo + k0 + kr) * ldb + n) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 256 * i;
      *(f32x4*)&sA[buf][(q / 16) * S::LDAT + 4 * (q % 16)] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i;
      *(f32x4*)&sB[buf][(q / 32) * S::LDB + 4 * (q % 32)] = rb[i];
    }
  };
  const int cb0 = 64 * wn, cb1 = 64 * wn + 32;
  f32x16 acc0 = {}, acc1 = {};
  const int nk = (cnt + BK - 1) / BK;
  if (nk > 0) {
    load(0);
    store(0);
  }
  __syncthreads();
  for (int st = 0; st < nk; ++st) {
    const int buf = st & 1;
    if (st + 1 < nk) load((st + 1) * BK);
    f32_stage_mma<true, false, BK>(sA[buf], sB[buf], wm, cb0, cb1, lane, acc0, acc1);
    if (st + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }
  float* out = dW + (int64_t)e * M * N;
  const int col = lane % 32;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int m = m0 + 32 * wm + 8 * (q / 4) + 4 * (lane / 32) + q % 4;
    if (m >= M) continue;
    if (n0 + cb0 + col < N) out[(int64_t)m * N + n0 + cb0 + col] = acc0[q];
    if (n0 + cb1 + col < N) out[(int64_t)m * N + n0 + cb1 + col] = acc1[q];
  }
}

template <int EPI, bool BT = false, int BK = 32, int OCC = 2, int NJ = 4, int WM = 2, int NS = 3, bool PP = false,
          bool TL = false>
hipError_t launch_dma(const bf16_t* a, const int32_t* offsets, int64_t max_rows, int E, int K, int N, int ldw,
                      const bf16_t* w, bf16_t* out, hipStream_t s, const int32_t* row_token = nullptr,
                      int64_t a_rows = 0, bf16_t* out2 = nullptr, const bf16_t* aux = nullptr, int n_split = 1,
                      float* part = nullptr, int32_t* sched = nullptr, const float* row_w = nullptr,
                      bool wtiled = false) {
  constexpr bool SWIGLU = EPI == kEpiSwiglu || EPI == kEpiSwigluSave;
  constexpr int BNO = SWIGLU ? 32 * NJ : 64 * NJ;   // output columns per tile
  if (K / BK / n_split < NS - 1) return hipErrorInvalidValue;  // each range spans at least NS - 1 stages
  const int nt = (int)ceil_div(N, BNO);
  dma::k_grouped_gemm<EPI, BT, BK, OCC, NJ, WM, NS, PP, TL>
      <<<persistent_grid(max_rows, E, 64 * WM, nt * n_split, OCC), 128 * WM, 0, s>>>(
          a, offsets, max_rows, E, K, N, ldw, w, out, nt, row_token, a_rows, out2, aux, n_split, part, sched, row_w,
          wtiled ? 1 : 0);
  return hipGetLastError();
}

// ---- k-split products for few rows ----
// With few rows (decode-sized batches) the weight stream is the whole cost
// and the tiles are too few to keep every CU loading: the down projection's
// k-stages are then cut into n_split ranges, each writing float32 partial
// sums of its rows, and k_split_sum adds the ranges in order (deterministic)
// and rounds the rows to bf16.
constexpr int64_t kSplitMaxRows = 256;
constexpr int kSplitMax = 8;
constexpr int kSplitMinStages = 16;

// One thread per 4 columns of a row.
// With row_token (one pair per token) the rounded row goes, times its
// routing weight row_w[r] and rounded again, to its token's row of out
// ([out_rows, N]) instead of row r.
__global__ __launch_bounds__(256) void k_split_sum(const float* __restrict__ part, int n_split,
                                                   const int32_t* __restrict__ offsets, int E, int64_t max_rows,
                                                   int N, bf16_t* __restrict__ out,
                                                   const int32_t* __restrict__ row_token,
                                                   const float* __restrict__ row_w, int64_t out_rows) {
  const int64_t r = blockIdx.y;
  const int c = 4 * (blockIdx.x * blockDim.x + threadIdx.x);
  const int64_t n_rows = clampi<int64_t>(offsets[E], 0, max_rows);
  if (r >= n_rows || c >= N) return;
  f32x4 sum = *(const f32x4*)(part + r * N + c);
  for (int sp = 1; sp < n_split; ++sp) sum += *(const f32x4*)(part + ((int64_t)sp * max_rows + r) * N + c);
  const uint2 y = make_uint2(pack_bf16x2(sum[0], sum[1]), pack_bf16x2(sum[2], sum[3]));
  if (!row_token) {
    *(uint2*)(out + r * N + c) = y;
    return;
  }
  const int64_t t = row_token[r];
  if (t < 0 || t >= out_rows) return;
  const float w = row_w[r];
  float f[4];
  unpack4(y, f);
#pragma unroll
  for (int v = 0; v < 4; ++v) f[v] = fmaf(w, f[v], 0.f);
  *(uint2*)(out + t * N + c) = pack4(f);
}

// The split tail's sums: block (x, y) takes rows 4 y .. 4 y + 3 of split
// tile x, one thread per 4 columns; it adds the tile's pieces in piece order
// (deterministic) and applies the down projection's epilogue -- the row
// rounded to bf16, or with row_token (one pair per token) that times the
// row's routing weight, rounded again, into its token's row of out.  The
// header says how many tiles were split (none: every block returns).
constexpr int kTailSumRows = 4;
__global__ __launch_bounds__(256) void k_tail_sum(const float* __restrict__ ws, int N, bf16_t* __restrict__ out,
                                                  const int32_t* __restrict__ row_token,
                                                  const float* __restrict__ row_w, int64_t out_rows) {
  const int32_t* hdr = (const int32_t*)ws;
  const int n_exc = hdr[0], n_pc = hdr[1];
  const int b = blockIdx.x;
  if (b >= n_exc) return;
  const int32_t* rec = hdr + kTailHdrWords + 4 * b;
  const int64_t row0 = rec[1];
  const int rows = rec[2], n0 = rec[3];
  const int r = kTailSumRows * blockIdx.y + threadIdx.x / 64, c = 4 * (threadIdx.x % 64);
  if (r >= rows || n0 + c >= N) return;
  {
    const float* part = ws + kTailPartOff + (int64_t)b * n_pc * kTailPieceFloats + r * 256 + c;
    f32x4 p[kTailMaxSplit];
#pragma unroll
    for (int pc = 0; pc < kTailMaxSplit; ++pc)
      if (pc < n_pc) p[pc] = *(const f32x4*)(part + (int64_t)pc * kTailPieceFloats);
    f32x4 sum = p[0];
#pragma unroll
    for (int pc = 1; pc < kTailMaxSplit; ++pc)
      if (pc < n_pc) sum += p[pc];
    const uint2 y = make_uint2(pack_bf16x2(sum[0], sum[1]), pack_bf16x2(sum[2], sum[3]));
    if (!row_token) {
      *(uint2*)(out + (row0 + r) * N + n0 + c) = y;
      return;
    }
    const int64_t t = row_token[row0 + r];
    if (t < 0 || t >= out_rows) return;
    const float w = row_w[row0 + r];
    float f[4];
    unpack4(y, f);
#pragma unroll
    for (int v = 0; v < 4; ++v) f[v] = fmaf(w, f[v], 0.f);
    *(uint2*)(out + t * N + n0 + c) = pack4(f);
  }
}

// Ranges per tile for a product with few rows (1: no split).  Tiles are
// counted for the worst case of the offsets (every expert non-empty); the
// split that needs the fewest rounds of CU slots per unit of work wins.
int choose_split(int64_t max_rows, int E, int K, int N, int bm, int occ) {
  if (max_rows > kSplitMaxRows || N % 4 != 0) return 1;
  const int64_t tiles = (max_rows / bm + (E < max_rows ? E : max_rows)) * ceil_div(N, 256);
  const int64_t slots = (int64_t)occ * num_cus();
  int best = 1;
  double best_cost = (double)ceil_div(tiles, slots);
  for (int sp = 2; sp <= kSplitMax && (K / 32) / sp >= kSplitMinStages; ++sp) {
    const double cost = (double)ceil_div(tiles * sp, slots) / sp;
    if (cost < 0.95 * best_cost) {
      best = sp;
      best_cost = cost;
    }
  }
  return best;
}

// One grouped product in the tile shape big_tiles picks.
template <int EPI, bool BT>
hipError_t launch_auto(const bf16_t* a, const int32_t* offsets, int64_t max_rows, int E, int K, int N, int ldw,
                       const bf16_t* w, bf16_t* out, hipStream_t s, const int32_t* row_token = nullptr,
                       int64_t a_rows = 0, bf16_t* out2 = nullptr, const bf16_t* aux = nullptr,
                       int32_t* sched = nullptr, float* tail_ws = nullptr, bool allow_tall = true,
                       bool wtiled = false);

// 256-row tiles (8 waves in ping-pong, one workgroup per CU: each weight
// stage feeds twice the rows) once the experts hold 128 rows or more on
// average and K spans at least three stages; 128-row tiles (two workgroups
// per CU) below that.
bool big_tiles(int64_t max_rows, int E, int K) { return max_rows >= 128 * (int64_t)E && K >= 96; }

// 64-row tiles (two waves, two workgroups per CU) when the experts hold at
// most 64 rows on average (decode-sized batches): the product is a weight
// stream, and a 128-row tile would stage and multiply mostly empty rows.
// The tile list is set up with one thread per expert, so E <= 128.
bool small_tiles(int64_t max_rows, int E) { return max_rows <= 64 * (int64_t)E && E <= 128; }

// Tall 256-row tiles for the down and gate/up projections when the experts
// hold at most 384 rows on average: an expert then has one or two tiles, and
// a second tile of a few rows would cost about half a full one (measured on
// the 128-expert layer: down 881 -> 743 us, gate/up 1470 -> 1259 us).  With
// more rows per expert such tails are rare and the always-issued extra load
// costs more than it saves (down 74 -> 86 us at 512 rows per expert).
bool tall_tiles(int64_t max_rows, int E) { return max_rows <= 384 * (int64_t)E; }

template <int EPI, bool BT>
hipError_t launch_auto(const bf16_t* a, const int32_t* offsets, int64_t max_rows, int E, int K, int N, int ldw,
                       const bf16_t* w, bf16_t* out, hipStream_t s, const int32_t* row_token, int64_t a_rows,
                       bf16_t* out2, const bf16_t* aux, int32_t* sched, float* tail_ws, bool allow_tall,
                       bool wtiled) {
  if constexpr (EPI == kEpiPlain && !BT) {
    if (allow_tall && big_tiles(max_rows, E, K) && tall_tiles(max_rows, E) && row_token == nullptr)
      return launch_dma<EPI, BT, 32, 1, 4, 4, 4, true, true>(a, offsets, max_rows, E, K, N, ldw, w, out, s, nullptr,
                                                             0, out2, aux, 1, tail_ws, sched, nullptr, wtiled);
  }
  if constexpr (EPI == kEpiSwiglu && !BT) {
    if (big_tiles(max_rows, E, K) && tall_tiles(max_rows, E))
      return launch_dma<EPI, BT, 32, 1, 4, 4, 4, true, true>(a, offsets, max_rows, E, K, N, ldw, w, out, s, row_token,
                                                             a_rows, out2, aux, 1, nullptr, sched, nullptr, wtiled);
  }
  if (big_tiles(max_rows, E, K))
    return launch_dma<EPI, BT, 32, 1, 4, 4, 4, true>(a, offsets, max_rows, E, K, N, ldw, w, out, s, row_token,
                                                     a_rows, out2, aux, 1, EPI == kEpiPlain && !BT ? tail_ws : nullptr,
                                                     sched, nullptr, wtiled);
  if (small_tiles(max_rows, E))
    return launch_dma<EPI, BT, 32, 2, 4, 1, 3, false>(a, offsets, max_rows, E, K, N, ldw, w, out, s, row_token,
                                                      a_rows, out2, aux, 1, nullptr, nullptr, nullptr, wtiled);
  return launch_dma<EPI, BT>(a, offsets, max_rows, E, K, N, ldw, w, out, s, row_token, a_rows, out2, aux, 1, nullptr,
                             nullptr, nullptr, wtiled);
}

}  // namespace

__global__ __launch_bounds__(64) void k_sched_reset(int32_t* __restrict__ sched) {
  if (threadIdx.x < kSchedWords) sched[threadIdx.x] = 0;
}

hipError_t launch_sched_reset(int32_t* sched, hipStream_t s) {
  k_sched_reset<<<1, 64, 0, s>>>(sched);
  return hipGetLastError();
}

hipError_t launch_gate_up_bf16(const bf16_t* x, const int32_t* expert_offsets, int64_t max_rows, int E, int d,
                               int I, const bf16_t* w_gate_up, bf16_t* h, hipStream_t s, const int32_t* row_token,
                               int64_t x_rows, int32_t* sched, bool wtiled) {
  return launch_auto<kEpiSwiglu, false>(x, expert_offsets, max_rows, E, d, I, 2 * I, w_gate_up, h, s, row_token,
                                        x_rows, nullptr, nullptr, sched, nullptr, true, wtiled);
}

// Whether the 256-row down projection can have a split tail: only when its
// persistent grid is capped at the CU count (otherwise every tile has a
// workgroup of its own, whatever the offsets).
bool down_tail_possible(int64_t max_rows, int E, int d, int I) {
  const int64_t max_mt = max_rows / 256 + (E < max_rows ? E : max_rows);
  return max_rows > kSplitMaxRows && big_tiles(max_rows, E, I) && max_mt * ceil_div(d, 256) > (int64_t)num_cus();
}

size_t split_workspace(int64_t max_rows, int E, int d, int I) {
  if (max_rows <= kSplitMaxRows) return (size_t)kSplitMax * max_rows * d * sizeof(float);
  return down_tail_possible(max_rows, E, d, I) ? kTailBytes : 0;
}

int down_split(int64_t max_rows, int E, int d, int I, bool have_split_ws) {
  if (!have_split_ws || big_tiles(max_rows, E, I)) return 1;
  return choose_split(max_rows, E, I, d, small_tiles(max_rows, E) ? 64 : 128, 2);
}

bool down_scatters(int64_t max_rows, int E, int d, int I, bool have_split_ws) {
  return big_tiles(max_rows, E, I) || down_split(max_rows, E, d, I, have_split_ws) > 1;
}

hipError_t launch_down_bf16(const bf16_t* h, const int32_t* expert_offsets, int64_t max_rows, int E, int d,
                            int I, const bf16_t* w_down, bf16_t* y_perm, hipStream_t s, float* split_ws,
                            int32_t* sched, const DownScatter* sc, bool scatter_tiles, bool wtiled) {
  if (sc && !down_scatters(max_rows, E, d, I, split_ws != nullptr)) return hipErrorInvalidValue;
  {
    const bool small = small_tiles(max_rows, E);
    const int n_split = down_split(max_rows, E, d, I, split_ws != nullptr);
    if (n_split > 1) {
      const hipError_t e =
          small ? launch_dma<kEpiPartial, false, 32, 2, 4, 1, 3, false>(h, expert_offsets, max_rows, E, I, d, d,
                                                                        w_down, nullptr, s, nullptr, 0, nullptr,
                                                                        nullptr, n_split, split_ws, nullptr, nullptr,
                                                                        wtiled)
                : launch_dma<kEpiPartial>(h, expert_offsets, max_rows, E, I, d, d, w_down, nullptr, s, nullptr, 0,
                                          nullptr, nullptr, n_split, split_ws, nullptr, nullptr, wtiled);
      if (e != hipSuccess) return e;
      const dim3 grid((unsigned)ceil_div(d / 4, 256), (unsigned)max_rows);
      k_split_sum<<<grid, 256, 0, s>>>(split_ws, n_split, expert_offsets, E, max_rows, d, sc ? sc->out : y_perm,
                                       sc ? sc->row_token : nullptr, sc ? sc->row_w : nullptr, sc ? sc->T : 0);
      return hipGetLastError();
    }
  }
  int32_t* dn_sched = sched ? sched + kSchedDown : nullptr;
  // the split tail (256-row tiles, with a workspace, when the grid is capped)
  float* tail_ws = split_ws && down_tail_possible(max_rows, E, d, I) ? split_ws : nullptr;
  hipError_t e;
  if (sc)   // 256-row tiles (down_scatters)
    e = launch_dma<kEpiScatter, false, 32, 1, 4, 4, 4, true>(h, expert_offsets, max_rows, E, I, d, d, w_down,
                                                              sc->out, s, sc->row_token, sc->T, nullptr, nullptr, 1,
                                                              tail_ws, dn_sched, sc->row_w, wtiled);
  else
    e = launch_auto<kEpiPlain, false>(h, expert_offsets, max_rows, E, I, d, d, w_down, y_perm, s, nullptr, 0,
                                      nullptr, nullptr, dn_sched, tail_ws, !scatter_tiles, wtiled);
  if (e != hipSuccess || tail_ws == nullptr) return e;
  k_tail_sum<<<dim3(kTailPieces / 2, 288 / kTailSumRows), 256, 0, s>>>(
      tail_ws, d, sc ? sc->out : y_perm, sc ? sc->row_token : nullptr, sc ? sc->row_w : nullptr, sc ? sc->T : 0);
  return hipGetLastError();
}

hipError_t launch_gate_up_save_bf16(const bf16_t* x, const int32_t* expert_offsets, int64_t max_rows, int E, int d,
                                    int I, const bf16_t* w_gate_up, bf16_t* h, bf16_t* gu, hipStream_t s,
                                    const int32_t* row_token, int64_t x_rows, int32_t* sched) {
  return launch_auto<kEpiSwigluSave, false>(x, expert_offsets, max_rows, E, d, I, 2 * I, w_gate_up, h, s, row_token,
                                            x_rows, gu, nullptr, sched);
}

hipError_t launch_down_dgrad_swiglu_bf16(const bf16_t* dy, const int32_t* expert_offsets, int64_t max_rows, int E,
                                         int d, int I, const bf16_t* w_down, const bf16_t* gu, bf16_t* dgu,
                                         hipStream_t s) {
  // dh = dy Wd^T: Wd [I][d] is the [N][K] weight of a product with K = d, N = I
  return launch_auto<kEpiSwigluBwd, true>(dy, expert_offsets, max_rows, E, d, I, d, w_down, dgu, s, nullptr, 0,
                                          nullptr, gu);
}

hipError_t launch_gate_up_dgrad_bf16(const bf16_t* dgu, const int32_t* expert_offsets, int64_t max_rows, int E,
                                     int d, int I, const bf16_t* w_gate_up, bf16_t* dx_perm, hipStream_t s) {
  // dx = [dg | du] Wgu^T: Wgu [d][2I] is the [N][K] weight of a product with K = 2I, N = d
  return launch_auto<kEpiPlain, true>(dgu, expert_offsets, max_rows, E, 2 * I, d, 2 * I, w_gate_up, dx_perm, s);
}

// ---- column-tiled weights -------------------------------------------------
// One expert's [K][ldw] weight as the products' column tiles read it: block
// c (c = 0, 1, ...) holds the tile's columns as [K][width], width = the
// tile's weight columns, blocks in column order; for gate/up (ldw = 2N) a
// tile is TC gate columns n0 .. n0 + w - 1 and the same up columns, stored
// gate first (width 2w), for down (ldw = N) TC columns (width w).  Every
// block but the last is full, so block c starts at element K * c * TC
// (gate/up: K * 2 c * TC).  One wave copies one row of one block, 16 bytes
// a lane.
__global__ __launch_bounds__(256) void k_tile_weights(const bf16_t* __restrict__ w, int E, int K, int N, int tc,
                                                      bool gate_up, bf16_t* __restrict__ out) {
  const int lane = threadIdx.x % kWave;
  const int nb = (int)ceil_div(N, tc);
  const int64_t rows = (int64_t)E * nb * K;
  const int ldw = gate_up ? 2 * N : N;
  for (int64_t q = (int64_t)blockIdx.x * (256 / kWave) + threadIdx.x / kWave; q < rows;
       q += (int64_t)gridDim.x * (256 / kWave)) {
    const int e = (int)(q / ((int64_t)nb * K));
    const int c = (int)(q / K % nb);
    const int k = (int)(q % K);
    const int n0 = c * tc, wc = min(tc, N - n0);
    const int width = gate_up ? 2 * wc : wc;
    const bf16_t* src = w + ((int64_t)e * K + k) * ldw;
    bf16_t* dst = out + (int64_t)e * K * ldw + (int64_t)K * (gate_up ? 2 * n0 : n0) + (int64_t)k * width;
    for (int v = lane * 8; v < width; v += kWave * 8) {
      // (wc is a multiple of 8: a vector never straddles the gate and up halves)
      const int col = (gate_up && v >= wc) ? N + n0 + (v - wc) : n0 + v;
      *(uint4*)(dst + v) = *(const uint4*)(src + col);
    }
  }
}

hipError_t launch_tile_weights_bf16(const bf16_t* w_gate_up, const bf16_t* w_down, int E, int d, int I,
                                    bf16_t* wgu_tiled, bf16_t* wd_tiled, hipStream_t s) {
  const int64_t rows_gu = (int64_t)E * ceil_div(I, kTileGateCols) * d;
  const int64_t rows_dn = (int64_t)E * ceil_div(d, kTileDownCols) * I;
  const unsigned cap = 65535u * 4u;
  k_tile_weights<<<(unsigned)std::min<int64_t>(ceil_div(rows_gu, 4), cap), 256, 0, s>>>(w_gate_up, E, d, I,
                                                                                       kTileGateCols, true, wgu_tiled);
  k_tile_weights<<<(unsigned)std::min<int64_t>(ceil_div(rows_dn, 4), cap), 256, 0, s>>>(w_down, E, I, d,
                                                                                       kTileDownCols, false, wd_tiled);
  return hipGetLastError();
}

// row tiles a float32 launch may need: ceil(rows_e / 64) summed over the experts
static unsigned f32_row_tiles(int64_t max_rows, int E) {
  return (unsigned)(max_rows / kF32Rows + (E < max_rows ? E : max_rows));
}

template <int EPI, bool BT>
static hipError_t launch_f32(const float* a, const int32_t* offsets, int64_t max_rows, int E, int K, int N,
                             const float* w, float* out, hipStream_t s, float* out2 = nullptr,
                             const float* aux = nullptr) {
  constexpr bool GU = EPI == kF32Swiglu || EPI == kF32SwigluSave;
  const dim3 g(f32_row_tiles(max_rows, E), (unsigned)ceil_div(N, GU ? kF32Cols / 2 : kF32Cols));
  if (g.x == 0 || g.y == 0) return hipSuccess;
  if (K % kF32K != 0) return hipErrorInvalidValue;
  k_grouped_gemm_f32<EPI, BT><<<g, 256, 0, s>>>(a, offsets, max_rows, E, K, N, w, out, out2, aux);
  return hipGetLastError();
}

hipError_t launch_gate_up_f32(const float* x_perm, const int32_t* expert_offsets, int64_t max_rows, int E,
                              int d, int I, const float* w_gate_up, float* h, hipStream_t s) {
  return launch_f32<kF32Swiglu, false>(x_perm, expert_offsets, max_rows, E, d, I, w_gate_up, h, s);
}

hipError_t launch_down_f32(const float* h, const int32_t* expert_offsets, int64_t max_rows, int E, int d,
                           int I, const float* w_down, float* y_perm, hipStream_t s) {
  return launch_f32<kF32Epi, false>(h, expert_offsets, max_rows, E, I, d, w_down, y_perm, s);
}

hipError_t launch_gate_up_save_f32(const float* x_perm, const int32_t* expert_offsets, int64_t max_rows, int E,
                                   int d, int I, const float* w_gate_up, float* h, float* gu, hipStream_t s) {
  return launch_f32<kF32SwigluSave, false>(x_perm, expert_offsets, max_rows, E, d, I, w_gate_up, h, s, gu);
}

hipError_t launch_down_dgrad_swiglu_f32(const float* dy, const int32_t* expert_offsets, int64_t max_rows, int E,
                                        int d, int I, const float* w_down, const float* gu, float* dgu,
                                        hipStream_t s) {
  // dh = dy Wd^T: Wd [I][d] is the [N][K] weight of a product with K = d, N = I
  return launch_f32<kF32SwigluBwd, true>(dy, expert_offsets, max_rows, E, d, I, w_down, dgu, s, nullptr, gu);
}

hipError_t launch_gate_up_dgrad_f32(const float* dgu, const int32_t* expert_offsets, int64_t max_rows, int E,
                                    int d, int I, const float* w_gate_up, float* dx_perm, hipStream_t s) {
  // dx = [dg | du] Wgu^T: Wgu [d][2I] is the [N][K] weight of a product with K = 2I, N = d
  return launch_f32<kF32Epi, true>(dgu, expert_offsets, max_rows, E, 2 * I, d, w_gate_up, dx_perm, s);
}

hipError_t launch_wgrad_f32(const float* a, int lda, int M, const float* b, int ldb, int N,
                            const int32_t* expert_offsets, int64_t max_rows, int E, float* dw, hipStream_t s) {
  if (M % 4 != 0 || N % 4 != 0 || lda < M || ldb < N) return hipErrorInvalidValue;
  const int m_tiles = (int)ceil_div(M, kF32Rows), n_tiles = (int)ceil_div(N, kF32Cols);
  const int64_t blocks = (int64_t)E * m_tiles * n_tiles;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  k_wgrad_f32<<<(unsigned)blocks, 256, 0, s>>>(a, lda, M, b, ldb, N, expert_offsets, max_rows, m_tiles, n_tiles, dw);
  return hipGetLastError();
}

hipError_t launch_grouped_ffn_bf16(const bf16_t* x_perm, const int32_t* expert_offsets, int64_t max_rows,
                                   int E, int d, int I, const bf16_t* w_gate_up, const bf16_t* w_down,
                                   bf16_t* h, bf16_t* y_perm, hipStream_t s, float* split_ws, int32_t* sched,
                                   bool wtiled) {
  const hipError_t e =
      launch_gate_up_bf16(x_perm, expert_offsets, max_rows, E, d, I, w_gate_up, h, s, nullptr, 0, sched, wtiled);
  if (e != hipSuccess) return e;
  return launch_down_bf16(h, expert_offsets, max_rows, E, d, I, w_down, y_perm, s, split_ws, sched, nullptr, false,
                          wtiled);
}

hipError_t launch_grouped_ffn_f32(const float* x_perm, const int32_t* expert_offsets, int64_t max_rows, int E,
                                  int d, int I, const float* w_gate_up, const float* w_down, float* h,
                                  float* y_perm, hipStream_t s) {
  const hipError_t e = launch_gate_up_f32(x_perm, expert_offsets, max_rows, E, d, I, w_gate_up, h, s);
  if (e != hipSuccess) return e;
  return launch_down_f32(h, expert_offsets, max_rows, E, d, I, w_down, y_perm, s);
}

}  // namespace tre
