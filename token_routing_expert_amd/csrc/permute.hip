// permute.hip -- group (token, expert) pairs by expert and move token rows.
//
// "Expert parallelism" (Hugging Face Transformers docs), section "Token
// dispatch": each (token, expert) pair is sent to the expert's owner, which
// runs the expert on the rows it received.  On one device this is a stable
// counting sort of the pairs by expert followed by a row gather:
//   expert e owns rows [offsets[e], offsets[e+1]) in increasing pair order,
//   row_token[r] = token of row r, pair_row[p] = row of pair p (-1: dropped),
//   x_perm[r] = x[row_token[r]].
//
// Index kernels, all deterministic (integer counts only; no result depends on
// the order of atomics):
//   hist     one workgroup per chunk of kPermuteChunk pairs counts its pairs
//            per expert in LDS;
//   scatter  every workgroup first sums the counts of the chunks before its
//            own and of all chunks (expert offsets and its chunk's starting
//            row per expert, with no scan kernel in between), then walks its
//            pairs in order, 256 at a time: a pair's row is its chunk's
//            running row for the expert, plus the matching pairs in earlier
//            waves of the step, plus its rank among equal experts in its own
//            wave (eight ballots over the expert id bits);
//   scan     only when there are many chunks (the sums above would grow as
//            chunks^2): one workgroup writes the offsets and every chunk's
//            starting rows, which the scatter then reads.
//   small    up to kSmallPairs pairs: one workgroup does all of the above in
//            one launch.
//   rows     the scatter and the row move in one kernel (after hist): each
//            workgroup places the pairs of a few tokens (summing the counts
//            it needs itself) while its first row loads are in flight, then
//            writes the tokens' rows to their grouped rows.
// Without that fusion (decode-sized batches, more than 64 pairs a token) the
// row move is its own bandwidth-bound kernel: one wave per token, its row read
// once in 16-byte vectors and written to each of its grouped rows.
#include "common.hpp"

namespace tre {
namespace {

constexpr int kThreads = 256;

// Adds 1 to cnt[e] (LDS) for every expert id e in [0, E) among
// pair_expert[lo, hi), the workgroup's threads striding over the range.  A
// thread's ids are read kCountBatch at a time with every load in flight
// together (an id's load and its count in turn would wait a full memory
// round trip per id); lanes past hi re-read pair_expert[lo] and count
// nothing.
constexpr int kCountBatch = 8;   // (the asm below names each of the 8)

__device__ __forceinline__ void count_ids(const int32_t* __restrict__ pair_expert, int64_t lo, int64_t hi, int E,
                                          int* cnt) {
  for (int64_t q0 = lo + threadIdx.x; q0 < hi; q0 += (int64_t)kCountBatch * kThreads) {
    int ev[kCountBatch];
#pragma unroll
    for (int u = 0; u < kCountBatch; ++u) {
      const int64_t q = q0 + (int64_t)u * kThreads;
      ev[u] = pair_expert[q < hi ? q : lo];
    }
    // (without this the compiler waits for the first id before issuing the
    // other loads, to test it early)
    asm volatile("" : "+v"(ev[0]), "+v"(ev[1]), "+v"(ev[2]), "+v"(ev[3]), "+v"(ev[4]), "+v"(ev[5]), "+v"(ev[6]),
                 "+v"(ev[7]));
#pragma unroll
    for (int u = 0; u < kCountBatch; ++u) {
      const int64_t q = q0 + (int64_t)u * kThreads;
      if (q >= hi) continue;
      MOE_DCHECK(ev[u] >= -1 && ev[u] < E);   // an expert id, or -1 for a masked pair
      if (ev[u] >= 0 && ev[u] < E) atomicAdd(&cnt[ev[u]], 1);
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_perm_hist(const int32_t* __restrict__ pair_expert, int64_t P,
                                                        int E, int chunk_pairs, int32_t* __restrict__ chunk_count,
                                                        int32_t* __restrict__ sched) {
  __shared__ int cnt[kMaxExperts];
  const int tid = threadIdx.x;
  if (sched && blockIdx.x == 0 && tid < kSchedWords) sched[tid] = 0;
  if (tid < E) cnt[tid] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * chunk_pairs;
  count_ids(pair_expert, base, min(P, base + chunk_pairs), E, cnt);
  __syncthreads();
  if (tid < E) chunk_count[(int64_t)blockIdx.x * E + tid] = cnt[tid];
}

// Exclusive prefix over the 256 threads of a block; *total gets the sum.
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
  for (int w = 0; w < kThreads / kWave; ++w) {
    before += (w < wave) ? s_wave[w] : 0;
    all += s_wave[w];
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

__global__ __launch_bounds__(kThreads) void k_perm_scan(const int32_t* __restrict__ chunk_count, int n_chunks,
                                                        int E, int32_t* __restrict__ chunk_base,
                                                        int32_t* __restrict__ offsets) {
  __shared__ int s_wave[kThreads / kWave];
  const int e = threadIdx.x;
  int total = 0;
  if (e < E)
    for (int b = 0; b < n_chunks; ++b) total += chunk_count[(int64_t)b * E + e];
  int all = 0;
  const int start = block_exclusive_scan(e < E ? total : 0, s_wave, &all);
  if (e < E) {
    offsets[e] = start;
    int run = start;
    for (int b = 0; b < n_chunks; ++b) {
      chunk_base[(int64_t)b * E + e] = run;
      run += chunk_count[(int64_t)b * E + e];
    }
  }
  if (e == 0) offsets[E] = all;
}

// chunk_base != nullptr: the chunk starting rows come from k_perm_scan.
// Otherwise they (and the offsets, written by workgroup 0) are summed here
// from all n_chunks * E counts.
__global__ __launch_bounds__(kThreads) void k_perm_scatter(const int32_t* __restrict__ pair_expert, int64_t P,
                                                           int k, int E, int n_chunks,
                                                           const int32_t* __restrict__ chunk_count,
                                                           const int32_t* __restrict__ chunk_base,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ pair_row,
                                                           int32_t* __restrict__ row_token,
                                                           const float* __restrict__ pair_w,
                                                           float* __restrict__ row_w) {
  __shared__ int running[kMaxExperts];
  __shared__ int s_before[kMaxExperts];
  __shared__ int s_total[kMaxExperts];
  __shared__ int wave_count[kThreads / kWave][kMaxExperts];
  __shared__ int s_wave[kThreads / kWave];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int chunk = blockIdx.x;
  const int64_t base = (int64_t)chunk * kPermuteChunk;
  const int64_t end = min(P, base + kPermuteChunk);
  // the first step's expert id, loaded before the counts are summed
  int e_next = (base + tid < end) ? pair_expert[base + tid] : -1;
  if (chunk_base) {
    if (tid < E) running[tid] = chunk_base[(int64_t)chunk * E + tid];
  } else {
    if (tid < E) s_before[tid] = s_total[tid] = 0;
    __syncthreads();
    // kThreads / E threads share an expert's chunks, all of a thread's loads
    // in flight together
    const int parts = kThreads / E;
    if (tid < parts * E) {
      const int ex = tid % E;
      int before = 0, total = 0;
#pragma unroll 16
      for (int b = tid / E; b < n_chunks; b += parts) {
        const int v = chunk_count[(int64_t)b * E + ex];
        total += v;
        before += b < chunk ? v : 0;
      }
      atomicAdd(&s_total[ex], total);
      atomicAdd(&s_before[ex], before);
    }
    __syncthreads();
    const int total = tid < E ? s_total[tid] : 0;
    int all = 0;
    const int start = block_exclusive_scan(total, s_wave, &all);
    if (tid < E) running[tid] = start + s_before[tid];
    if (chunk == 0) {
      if (tid < E) offsets[tid] = start;
      if (tid == 0) offsets[E] = all;
    }
  }
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int step = 0; step < kPermuteChunk; step += kThreads) {
    if (tid < E) {
#pragma unroll
      for (int w = 0; w < kThreads / kWave; ++w) wave_count[w][tid] = 0;
    }
    __syncthreads();
    const int64_t p = base + step + tid;
    const int e = e_next;
    if (step + kThreads < kPermuteChunk) e_next = (p + kThreads < end) ? pair_expert[p + kThreads] : -1;
    const bool valid = e >= 0 && e < E;
    // lanes of this wave holding the same expert: eight ballots over the id bits
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool set = (e >> bit) & 1;
      const uint64_t b = __ballot(set);
      peers &= set ? b : ~b;
    }
    const int rank = __popcll(peers & lt_mask);
    if (valid && rank == 0) wave_count[wave][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int r = running[e] + rank;
      for (int w = 0; w < wave; ++w) r += wave_count[w][e];
      pair_row[p] = r;
      if (r >= 0 && r < P) {
        row_token[r] = (int32_t)(p / k);
        if (row_w) row_w[r] = pair_w[p];
      }
    } else if (p < end) {
      pair_row[p] = -1;
    }
    __syncthreads();
    if (tid < E) {
      int add = 0;
#pragma unroll
      for (int w = 0; w < kThreads / kWave; ++w) add += wave_count[w][tid];
      running[tid] += add;
    }
    // the next step's zeroing is ordered after this update by its own barrier
    __syncthreads();
  }
}

// Small batches (P <= kSmallPairs, decode-sized): one workgroup of 1024 threads does the
// whole grouping -- counts in LDS, the exclusive scan, then the same stable
// scatter as k_perm_scatter, 1024 pairs per step (rank = running row of the
// expert + matching pairs in earlier waves of the step + rank among equal
// ids in the wave) -- in one launch instead of two.
constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / kWave;
constexpr int kSmallSteps = 2;  // pairs per thread: up to kSmallSteps * kSmallThreads pairs

__global__ __launch_bounds__(kSmallThreads) void k_perm_small(const int32_t* __restrict__ pair_expert, int P,
                                                               int k, int E, int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ pair_row,
                                                               int32_t* __restrict__ row_token,
                                                               int32_t* __restrict__ sched,
                                                               const float* __restrict__ pair_w,
                                                               float* __restrict__ row_w) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int running[kMaxExperts];
  __shared__ int wave_count[kSmallWaves][kMaxExperts];
  __shared__ int s_wave[kSmallWaves];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  if (sched && tid < kSchedWords) sched[tid] = 0;
  // every id is read once, up front (one round trip), and kept in registers:
  // id j of this thread is pair j * kSmallThreads + tid
  int ids[kSmallSteps];
#pragma unroll
  for (int j = 0; j < kSmallSteps; ++j) {
    const int p = j * kSmallThreads + tid;
    ids[j] = p < P ? pair_expert[p] : -1;
    MOE_DCHECK(ids[j] >= -1 && ids[j] < E);   // an expert id, or -1 for a masked pair
  }
  if (tid < E) cnt[tid] = 0;
  lds_barrier();
#pragma unroll
  for (int j = 0; j < kSmallSteps; ++j)
    if (ids[j] >= 0 && ids[j] < E) atomicAdd(&cnt[ids[j]], 1);
  lds_barrier();
  // exclusive scan of the counts (E <= 256: the first four waves)
  {
    const int v = tid < E ? cnt[tid] : 0;
    int x = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(x, off, kWave);
      if (lane >= off) x += y;
    }
    if (lane == kWave - 1 && wave < 4) s_wave[wave] = x;
    lds_barrier();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      before += (w < wave) ? s_wave[w] : 0;
      all += s_wave[w];
    }
    if (tid < E) {
      running[tid] = before + x - v;
      offsets[tid] = before + x - v;
    }
    if (tid == 0) offsets[E] = all;
  }
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
#pragma unroll
  for (int j = 0; j < kSmallSteps; ++j) {
    const int base = j * kSmallThreads;
    if (base >= P) break;
    for (int i = tid; i < kSmallWaves * E; i += kSmallThreads) (&wave_count[0][0])[(i / E) * kMaxExperts + i % E] = 0;
    lds_barrier();
    const int p = base + tid;
    const int e = ids[j];
    const bool valid = e >= 0 && e < E;
    // lanes of this wave holding the same expert: eight ballots over the id bits
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool set = (e >> bit) & 1;
      const uint64_t b = __ballot(set);
      peers &= set ? b : ~b;
    }
    const int rank = __popcll(peers & lt_mask);
    if (valid && rank == 0) wave_count[wave][e] = __popcll(peers);
    lds_barrier();
    if (valid) {
      int r = running[e] + rank;
      for (int w = 0; w < wave; ++w) r += wave_count[w][e];
      pair_row[p] = r;
      if (r >= 0 && r < P) {
        row_token[r] = p / k;
        if (row_w) row_w[r] = pair_w[p];
      }
    } else if (p < P) {
      pair_row[p] = -1;
    }
    lds_barrier();
    if (tid < E) {
      int add = 0;
#pragma unroll
      for (int w = 0; w < kSmallWaves; ++w) add += wave_count[w][tid];
      running[tid] += add;
    }
    // the next step's zeroing is ordered after this update by its own barrier
    lds_barrier();
  }
}

// One wave per token: the token's row is read once, in pieces of up to
// kMoveVec 16-byte vectors per lane held in registers, and each piece is
// written to every grouped row the token's pairs landed in (pair_row; -1 and
// rows past max_rows are skipped).  Every byte of x is read once and every
// byte of x_perm written once, all in full 16-byte vectors.
constexpr int kMoveVec = 8;

__global__ __launch_bounds__(kThreads) void k_move_rows(const u32x4* __restrict__ x, int64_t T, int64_t vec_per_row,
                                                        const int32_t* __restrict__ pair_row, int k,
                                                        int64_t max_rows, u32x4* __restrict__ x_perm) {
  const int64_t t = (int64_t)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  const int lane = threadIdx.x % kWave;
  const u32x4* src = x + t * vec_per_row;
  for (int64_t base = 0; base < vec_per_row; base += kMoveVec * kWave) {
    u32x4 piece[kMoveVec];
#pragma unroll
    for (int i = 0; i < kMoveVec; ++i) {
      const int64_t v = base + i * kWave + lane;
      if (v < vec_per_row) piece[i] = __builtin_nontemporal_load(&src[v]);   // each token row is read once
    }
    for (int j = 0; j < k; ++j) {
      const int64_t r = pair_row[t * k + j];
      if (r < 0 || r >= max_rows) continue;
      u32x4* dst = x_perm + r * vec_per_row;
#pragma unroll
      for (int i = 0; i < kMoveVec; ++i) {
        const int64_t v = base + i * kWave + lane;
        if (v < vec_per_row) dst[v] = piece[i];
      }
    }
  }
}

// The grouping and the row move in one launch, after k_perm_hist (and, for
// many chunks, k_perm_scan).  A workgroup takes 4 * tpw consecutive tokens
// (wave w: tokens w, w + 4, ...; at most kThreads pairs).  It first issues the
// loads of each wave's first row piece, so that reading the rows overlaps the
// index work.  It then places its own pairs where k_perm_scatter would: the
// expert's offset, plus that expert's pairs in earlier chunks (the counts) and
// in its own chunk before its first pair (counted here from the ids), plus the
// rank among its own pairs (earlier waves' counts, the ballot rank within the
// wave).  Last, every wave writes its tokens' row pieces to their grouped rows,
// the next piece's loads issued before the current one is written.
constexpr int kRowsWaves = kThreads / kWave;
constexpr int kRowsVec = 8;   // 16-byte vectors a lane per row piece

__global__ __launch_bounds__(kThreads) void k_perm_rows(
    const int32_t* __restrict__ pair_expert, int64_t T, int k, int E, int chunk_pairs, int n_chunks,
    const int32_t* __restrict__ chunk_count, const int32_t* __restrict__ chunk_base, int32_t* __restrict__ offsets,
    int32_t* __restrict__ pair_row, int32_t* __restrict__ row_token, const u32x4* __restrict__ x,
    int64_t vec_per_row, int tpw, u32x4* __restrict__ x_perm) {
  __shared__ int running[kMaxExperts];
  __shared__ int s_before[kMaxExperts];
  __shared__ int s_total[kMaxExperts];
  __shared__ int wave_count[kRowsWaves][kMaxExperts];
  __shared__ int s_wave[kRowsWaves];
  __shared__ int s_row[kThreads];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int64_t P = T * k;
  const int64_t t0 = (int64_t)blockIdx.x * (kRowsWaves * tpw);
  const int n_tok = (int)min((int64_t)kRowsWaves * tpw, T - t0);
  const int64_t p0 = t0 * k;
  const int np = n_tok * k;
  // work items of this wave: (token j, piece) for its tokens t0 + wave + 4 j
  const int n_pieces = (int)ceil_div(vec_per_row, kRowsVec * kWave);
  const int my_tok = n_tok > wave ? (n_tok - wave + kRowsWaves - 1) / kRowsWaves : 0;
  const int items = my_tok * n_pieces;
  u32x4 buf_a[kRowsVec], buf_b[kRowsVec];
  auto load_item = [&](int i, u32x4(&buf)[kRowsVec]) {
    const int j = i / n_pieces;
    const u32x4* src = x + (t0 + wave + kRowsWaves * j) * vec_per_row;
    const int64_t base = (int64_t)(i - j * n_pieces) * (kRowsVec * kWave);
#pragma unroll
    for (int u = 0; u < kRowsVec; ++u) {
      const int64_t v = base + u * kWave + lane;
      if (v < vec_per_row) buf[u] = __builtin_nontemporal_load(&src[v]);   // each token row is read once
    }
  };
  auto store_item = [&](int i, const u32x4(&buf)[kRowsVec]) {
    const int j = i / n_pieces;
    const int lt = wave + kRowsWaves * j;
    const int64_t base = (int64_t)(i - j * n_pieces) * (kRowsVec * kWave);
    for (int q = 0; q < k; ++q) {
      const int r = s_row[lt * k + q];
      if (r < 0 || r >= P) continue;
      u32x4* dst = x_perm + (int64_t)r * vec_per_row;
#pragma unroll
      for (int u = 0; u < kRowsVec; ++u) {
        const int64_t v = base + u * kWave + lane;
        if (v < vec_per_row) dst[v] = buf[u];
      }
    }
  };
  if (items > 0) load_item(0, buf_a);
  const int e = tid < np ? pair_expert[p0 + tid] : -1;
  // each expert's pairs before this workgroup's first pair: in earlier chunks
  // (with few experts, kThreads / E threads share an expert's chunks) ...
  const int c0 = (int)(p0 / chunk_pairs);
  if (tid < E) s_before[tid] = s_total[tid] = 0;
  __syncthreads();
  if (chunk_base) {
    if (tid < E) atomicAdd(&s_before[tid], chunk_base[(int64_t)c0 * E + tid]);   // includes the expert's offset
  } else {
    const int parts = kThreads / E;
    if (tid < parts * E) {
      const int ex = tid % E;
      int before = 0, total = 0;
#pragma unroll 16
      for (int b = tid / E; b < n_chunks; b += parts) {
        const int v = chunk_count[(int64_t)b * E + ex];
        total += v;
        before += b < c0 ? v : 0;
      }
      atomicAdd(&s_total[ex], total);
      atomicAdd(&s_before[ex], before);
    }
  }
  // ... and in this chunk
  count_ids(pair_expert, (int64_t)c0 * chunk_pairs, p0, E, s_before);
  __syncthreads();
  if (chunk_base) {
    if (tid < E) running[tid] = s_before[tid];
  } else {
    int all = 0;
    const int start = block_exclusive_scan(tid < E ? s_total[tid] : 0, s_wave, &all);
    if (tid < E) running[tid] = start + s_before[tid];
    if (blockIdx.x == 0) {
      if (tid < E) offsets[tid] = start;
      if (tid == 0) offsets[E] = all;
    }
  }
  if (tid < E) {
#pragma unroll
    for (int w = 0; w < kRowsWaves; ++w) wave_count[w][tid] = 0;
  }
  __syncthreads();
  const bool valid = e >= 0 && e < E;
  // lanes of this wave holding the same expert: eight ballots over the id bits
  uint64_t peers = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const bool set = (e >> bit) & 1;
    const uint64_t b = __ballot(set);
    peers &= set ? b : ~b;
  }
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  const int rank = __popcll(peers & lt_mask);
  if (valid && rank == 0) wave_count[wave][e] = __popcll(peers);
  __syncthreads();
  if (tid < np) {
    int r = -1;
    if (valid) {
      r = running[e] + rank;
      for (int w = 0; w < wave; ++w) r += wave_count[w][e];
      if (r >= 0 && r < P) row_token[r] = (int32_t)(t0 + tid / k);
    }
    pair_row[p0 + tid] = r;
    s_row[tid] = r;
  }
  __syncthreads();
  for (int i = 0; i < items; i += 2) {
    if (i + 1 < items) load_item(i + 1, buf_b);
    store_item(i, buf_a);
    if (i + 1 < items) {
      if (i + 2 < items) load_item(i + 2, buf_a);
      store_item(i + 1, buf_b);
    }
  }
}

}  // namespace

// Chunk counts up to this many are summed by every scatter workgroup.
constexpr int64_t kFusedScanMax = 16384;

size_t permute_index_workspace(int64_t P, int E) {
  const int64_t n_chunks = ceil_div(P, kPermuteChunk);
  return (size_t)round_up(2 * n_chunks * E * (int64_t)sizeof(int32_t), 256);
}

// Pair counts up to this many are grouped by the one-workgroup kernel.
constexpr int64_t kSmallPairs = kSmallSteps * kSmallThreads;

hipError_t launch_permute_index(const int32_t* pair_expert, int64_t P, int k, int E, int32_t* row_token,
                                int32_t* pair_row, int32_t* expert_offsets, void* ws, hipStream_t s, int32_t* sched,
                                const float* pair_w, float* row_w) {
  if (P <= kSmallPairs) {
    k_perm_small<<<1, kSmallThreads, 0, s>>>(pair_expert, (int)P, k, E, expert_offsets, pair_row, row_token, sched,
                                             pair_w, row_w);
    return hipGetLastError();
  }
  const int n_chunks = (int)ceil_div(P, kPermuteChunk);
  int32_t* chunk_count = (int32_t*)ws;
  int32_t* chunk_base = nullptr;
  k_perm_hist<<<n_chunks, kThreads, 0, s>>>(pair_expert, P, E, kPermuteChunk, chunk_count, sched);
  if ((int64_t)n_chunks * E > kFusedScanMax) {
    chunk_base = chunk_count + (int64_t)n_chunks * E;
    k_perm_scan<<<1, kThreads, 0, s>>>(chunk_count, n_chunks, E, chunk_base, expert_offsets);
  }
  k_perm_scatter<<<n_chunks, kThreads, 0, s>>>(pair_expert, P, k, E, n_chunks, chunk_count, chunk_base,
                                               expert_offsets, pair_row, row_token, pair_w, row_w);
  return hipGetLastError();
}

// The grouping with its row move: k_perm_hist with chunks of up to
// kRowsChunkMax pairs (at most kRowsChunks of them, else the one-workgroup
// scan runs too), then k_perm_rows.  Small batches, and more than 64 pairs a
// token, take the index kernels and k_move_rows.
constexpr int kRowsChunks = 32;
constexpr int kRowsChunkMax = 4096;

hipError_t launch_permute_rows(const int32_t* pair_expert, int64_t T, int k, int E, int32_t* row_token,
                               int32_t* pair_row, int32_t* expert_offsets, void* ws, hipStream_t s, int32_t* sched,
                               const void* x, int64_t row_bytes, void* x_perm) {
  const int64_t P = T * k;
  if (P <= kSmallPairs || k > kThreads / kRowsWaves) {
    const hipError_t err = launch_permute_index(pair_expert, P, k, E, row_token, pair_row, expert_offsets, ws, s,
                                                sched);
    if (err != hipSuccess) return err;
    return launch_move_rows(x, T, k, row_bytes, pair_row, P, x_perm, s);
  }
  int64_t chunk = kPermuteChunk;
  while (ceil_div(P, chunk) > kRowsChunks && chunk < kRowsChunkMax) chunk *= 2;
  const int n_chunks = (int)ceil_div(P, chunk);   // <= ceil(P / kPermuteChunk): fits the workspace
  int32_t* chunk_count = (int32_t*)ws;
  int32_t* chunk_base = nullptr;
  k_perm_hist<<<n_chunks, kThreads, 0, s>>>(pair_expert, P, E, (int)chunk, chunk_count, sched);
  if (n_chunks > kRowsChunks) {
    chunk_base = chunk_count + (int64_t)n_chunks * E;
    k_perm_scan<<<1, kThreads, 0, s>>>(chunk_count, n_chunks, E, chunk_base, expert_offsets);
  }
  const int tpw = k >= 8 ? 1 : 8 / k;
  const int64_t blocks = ceil_div(T, kRowsWaves * tpw);
  k_perm_rows<<<(unsigned)blocks, kThreads, 0, s>>>(pair_expert, T, k, E, (int)chunk, n_chunks, chunk_count,
                                                    chunk_base, expert_offsets, pair_row, row_token,
                                                    (const u32x4*)x, row_bytes / 16, tpw, (u32x4*)x_perm);
  return hipGetLastError();
}

hipError_t launch_move_rows(const void* x, int64_t T, int k, int64_t row_bytes, const int32_t* pair_row,
                            int64_t max_rows, void* x_perm, hipStream_t s) {
  const int tokens_per_block = kThreads / kWave;
  const int64_t blocks = ceil_div(T, tokens_per_block);
  k_move_rows<<<(unsigned)blocks, kThreads, 0, s>>>((const u32x4*)x, T, row_bytes / 16, pair_row, k, max_rows,
                                                    (u32x4*)x_perm);
  return hipGetLastError();
}

}  // namespace tre
