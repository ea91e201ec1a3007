// api.hip -- the C ABI (include/moe.h): host-side validation, workspace
// carving and kernel launches.  Every argument is checked before anything
// is enqueued; no call allocates, frees or synchronises.
#include "../../include/moe.h"
#include "common.hpp"

#include <mutex>

using namespace tre;

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 31;  // per-array element limit
constexpr int32_t kMaxRouterWidth = 1 << 22;       // router projection: d below this

size_t elem_size(moe_dtype dt) { return dt == MOE_F32 ? 4 : 2; }
bool dtype_ok(int dt) { return dt == MOE_F32 || dt == MOE_BF16; }
size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

moe_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

moe_status check_experts(int32_t E) {
  if (E < 1) return MOE_ERR_ARG;
  if (E > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_width(int32_t n) {
  if (n < 1) return MOE_ERR_ARG;
  if (n % 64 != 0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

#define TRY(expr)                    \
  do {                               \
    const moe_status st_ = (expr);   \
    if (st_ != MOE_OK) return st_;   \
  } while (0)

// Byte layout of the moe_forward workspace.
struct ForwardLayout {
  size_t pair_row, row_token, offsets, x_perm, h, y_perm, perm_ws, split, sched, row_w, total;
};

ForwardLayout forward_layout(int64_t T, int64_t d, int64_t E, int64_t k, int64_t I, moe_dtype dt) {
  const int64_t P = T * k;
  const size_t s = elem_size(dt);
  ForwardLayout L;
  size_t o = 0;
  L.pair_row = o;  o += align256(P * 4);
  L.row_token = o; o += align256(P * 4);
  L.offsets = o;   o += align256((E + 1) * 4);
  L.x_perm = o;    o += dt == MOE_F32 ? align256(P * d * s) : 0;   // bf16 gathers rows in place
  L.h = o;         o += align256(P * I * s);
  L.y_perm = o;    o += align256(P * d * s);
  L.perm_ws = o;   o += permute_index_workspace(P, (int)E);
  L.split = o;     o += dt == MOE_BF16 ? align256(split_workspace(P, (int)E, (int)d, (int)I)) : 0;
  L.sched = o;     o += dt == MOE_BF16 ? align256(kSchedWords * 4) : 0;
  L.row_w = o;     o += dt == MOE_BF16 && k == 1 ? align256(P * 4) : 0;
  L.total = o;
  return L;
}

// Byte layout of the moe_backward workspace (bf16): the recomputed forward
// intermediates and the row gradients, each 256-byte aligned.
struct BackwardLayout {
  size_t pair_row, row_token, offsets, perm_ws, x_perm, h, gu, y, dy, dgu, dxp, split, sched, total;
};

// s: bytes per element of the activation dtype (the float32 products split
// no k-ranges, so their layout has no split workspace)
BackwardLayout backward_layout(int64_t T, int64_t d, int64_t E, int64_t k, int64_t I, int64_t s) {
  const int64_t P = T * k;
  BackwardLayout L;
  size_t o = 0;
  L.pair_row = o;  o += align256(P * 4);
  L.row_token = o; o += align256(P * 4);
  L.offsets = o;   o += align256((E + 1) * 4);
  L.perm_ws = o;   o += permute_index_workspace(P, (int)E);
  L.x_perm = o;    o += align256(P * d * s);
  L.h = o;         o += align256(P * I * s);
  L.gu = o;        o += align256(P * 2 * I * s);
  L.y = o;         o += align256(P * d * s);
  L.dy = o;        o += align256(P * d * s);
  L.dgu = o;       o += align256(P * 2 * I * s);
  L.dxp = o;       o += align256(P * d * s);
  L.split = o;     o += s == 2 ? align256(split_workspace(P, (int)E, (int)d, (int)I)) : 0;
  L.sched = o;     o += align256(kSchedWords * 4);
  L.total = o;
  return L;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported size (limits: E <= 256, d and I multiples of 64)";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

moe_status moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_idx,
                          float* topk_w, void* stream) {
  if (T < 0) return MOE_ERR_ARG;
  TRY(check_experts(E));
  if (k < 1 || k > E) return MOE_ERR_ARG;
  if ((int64_t)T * E >= kMaxElems) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w) return MOE_ERR_ARG;
  return from_hip(launch_route_topk(logits, T, E, k, topk_idx, topk_w, (hipStream_t)stream));
}

moe_status moe_route_project(const void* x, const void* w_router, moe_dtype dt, int32_t T, int32_t d, int32_t E,
                             int32_t k, float* logits, int32_t* topk_idx, float* topk_w, void* stream) {
  if (!dtype_ok(dt) || T < 0 || k < 1) return MOE_ERR_ARG;
  TRY(check_experts(E));
  if (k > E) return MOE_ERR_ARG;
  TRY(check_width(d));
  if ((int64_t)T * d >= kMaxElems || (int64_t)E * d >= kMaxElems || (int64_t)T * E >= kMaxElems)
    return MOE_ERR_UNSUPPORTED;
  // byte offsets into 256 router rows stay below 2^31
  if (d >= kMaxRouterWidth) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !topk_idx || !topk_w) return MOE_ERR_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (dt == MOE_BF16)
    return from_hip(launch_route_project_bf16((const bf16_t*)x, (const bf16_t*)w_router, T, d, E, k, logits,
                                              topk_idx, topk_w, s));
  return from_hip(launch_route_project_f32((const float*)x, (const float*)w_router, T, d, E, k, logits, topk_idx,
                                           topk_w, s));
}

size_t moe_permute_workspace_size(int32_t T, int32_t k, int32_t E) {
  if (T < 0 || k < 1 || E < 1) return 0;
  return permute_index_workspace((int64_t)T * k, E);
}

moe_status moe_permute(const void* x, moe_dtype dt, int32_t T, int32_t d, int32_t k, const int32_t* pair_expert,
                       int32_t E, void* x_perm, int32_t* row_token, int32_t* pair_row, int32_t* expert_offsets,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dt) || T < 0 || k < 1) return MOE_ERR_ARG;
  TRY(check_experts(E));
  TRY(check_width(d));
  const int64_t P = (int64_t)T * k;
  if (P * d >= kMaxElems) return MOE_ERR_UNSUPPORTED;
  if (!expert_offsets) return MOE_ERR_ARG;
  if (T > 0 && (!pair_expert || !row_token || !pair_row || (x_perm && !x))) return MOE_ERR_ARG;
  if (workspace_bytes < moe_permute_workspace_size(T, k, E) || (T > 0 && !workspace)) return MOE_ERR_WORKSPACE;
  if (T == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  if (!x_perm)   // index only: the caller gathers rows itself
    return from_hip(launch_permute_index(pair_expert, P, k, E, row_token, pair_row, expert_offsets, workspace, s));
  return from_hip(launch_permute_rows(pair_expert, T, k, E, row_token, pair_row, expert_offsets, workspace, s,
                                      nullptr, x, (int64_t)d * elem_size(dt), x_perm));
}

size_t moe_grouped_ffn_workspace_size(int32_t max_rows, int32_t E, int32_t d, int32_t I, moe_dtype dt) {
  if (max_rows < 0 || I < 1 || E < 1 || !dtype_ok(dt)) return 0;
  // h, then (bf16) the down projection's k-split partial sums (few rows) or
  // split-tail partial tiles (many), and the two products' tile counters
  return align256((size_t)max_rows * I * elem_size(dt)) +
         (dt == MOE_BF16 && d > 0 ? align256(split_workspace(max_rows, E, d, I)) + align256(kSchedWords * 4) : 0);
}

moe_status moe_grouped_ffn(const void* x_perm, const int32_t* expert_offsets, int32_t max_rows, int32_t E,
                           int32_t d, int32_t I, const void* w_gate_up, const void* w_down, moe_dtype dt,
                           void* y_perm, void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dt) || max_rows < 0) return MOE_ERR_ARG;
  TRY(check_experts(E));
  TRY(check_width(d));
  TRY(check_width(I));
  if ((int64_t)max_rows * (d > I ? d : I) >= kMaxElems) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)E * d * 2 * I >= 8 * kMaxElems) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)d * I * 4 >= kMaxElems) return MOE_ERR_UNSUPPORTED;   // one expert's weights < 2 GiB
  if (max_rows == 0) return MOE_OK;
  if (!x_perm || !expert_offsets || !w_gate_up || !w_down || !y_perm) return MOE_ERR_ARG;
  if (!workspace || workspace_bytes < moe_grouped_ffn_workspace_size(max_rows, E, d, I, dt)) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if (dt == MOE_BF16) {
    char* split = (char*)workspace + align256((size_t)max_rows * I * 2);
    int32_t* sched = (int32_t*)(split + align256(split_workspace(max_rows, E, d, I)));
    TRY(from_hip(launch_sched_reset(sched, s)));
    return from_hip(launch_grouped_ffn_bf16((const bf16_t*)x_perm, expert_offsets, max_rows, E, d, I,
                                            (const bf16_t*)w_gate_up, (const bf16_t*)w_down, (bf16_t*)workspace,
                                            (bf16_t*)y_perm, s, (float*)split, sched));
  }
  return from_hip(launch_grouped_ffn_f32((const float*)x_perm, expert_offsets, max_rows, E, d, I,
                                         (const float*)w_gate_up, (const float*)w_down, (float*)workspace,
                                         (float*)y_perm, s));
}

namespace {

moe_status check_ffn_half(const void* a, const int32_t* expert_offsets, int32_t max_rows, int32_t E, int32_t d,
                          int32_t I, const void* w, moe_dtype dt, void* out) {
  if (!dtype_ok(dt) || max_rows < 0) return MOE_ERR_ARG;
  TRY(check_experts(E));
  TRY(check_width(d));
  TRY(check_width(I));
  if ((int64_t)max_rows * (d > I ? d : I) >= kMaxElems) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)E * d * 2 * I >= 8 * kMaxElems) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)d * I * 4 >= kMaxElems) return MOE_ERR_UNSUPPORTED;   // one expert's weights < 2 GiB
  if (max_rows > 0 && (!a || !expert_offsets || !w || !out)) return MOE_ERR_ARG;
  return MOE_OK;
}

}  // namespace

moe_status moe_gate_up_swiglu(const void* x, const int32_t* expert_offsets, int32_t max_rows, int32_t E,
                              int32_t d, int32_t I, const void* w_gate_up, moe_dtype dt, const int32_t* row_token,
                              int32_t x_rows, void* h, void* stream) {
  TRY(check_ffn_half(x, expert_offsets, max_rows, E, d, I, w_gate_up, dt, h));
  if (row_token) {
    if (dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (x_rows < 0) return MOE_ERR_ARG;
    if ((int64_t)x_rows * d >= kMaxElems / 2) return MOE_ERR_UNSUPPORTED;
  }
  if (max_rows == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  if (dt == MOE_BF16)
    return from_hip(launch_gate_up_bf16((const bf16_t*)x, expert_offsets, max_rows, E, d, I,
                                        (const bf16_t*)w_gate_up, (bf16_t*)h, s, row_token, x_rows));
  return from_hip(launch_gate_up_f32((const float*)x, expert_offsets, max_rows, E, d, I,
                                     (const float*)w_gate_up, (float*)h, s));
}

moe_status moe_down_proj(const void* h, const int32_t* expert_offsets, int32_t max_rows, int32_t E, int32_t d,
                         int32_t I, const void* w_down, moe_dtype dt, void* y_perm, void* stream) {
  TRY(check_ffn_half(h, expert_offsets, max_rows, E, d, I, w_down, dt, y_perm));
  if (max_rows == 0) return MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  if (dt == MOE_BF16)
    return from_hip(launch_down_bf16((const bf16_t*)h, expert_offsets, max_rows, E, d, I, (const bf16_t*)w_down,
                                     (bf16_t*)y_perm, s));
  return from_hip(launch_down_f32((const float*)h, expert_offsets, max_rows, E, d, I, (const float*)w_down,
                                  (float*)y_perm, s));
}

moe_status moe_combine(const void* y_perm, int32_t max_rows, const int32_t* pair_row, const float* pair_w,
                       int32_t T, int32_t k, int32_t d, moe_dtype dt, void* out, void* stream) {
  if (!dtype_ok(dt) || T < 0 || k < 1 || max_rows < 0) return MOE_ERR_ARG;
  TRY(check_width(d));
  if ((int64_t)T * k * d >= kMaxElems || (int64_t)max_rows * d >= kMaxElems) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!pair_row || !pair_w || !out || (max_rows > 0 && !y_perm)) return MOE_ERR_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (dt == MOE_BF16)
    return from_hip(launch_combine_bf16((const bf16_t*)y_perm, max_rows, pair_row, pair_w, T, k, d, (bf16_t*)out, s));
  return from_hip(launch_combine_f32((const float*)y_perm, max_rows, pair_row, pair_w, T, k, d, (float*)out, s));
}

size_t moe_forward_workspace_size(int32_t T, int32_t d, int32_t E, int32_t k, int32_t I, moe_dtype dt) {
  if (T < 0 || d < 1 || E < 1 || k < 1 || I < 1 || !dtype_ok(dt)) return 0;
  return forward_layout(T, d, E, k, I, dt).total;
}

}  // extern "C"

namespace {

// The layer's arguments, workspace aside (T == 0 is valid: nothing to do).
moe_status check_forward_args(const void* x, const float* logits, int32_t T, int32_t d, int32_t E, int32_t k,
                              int32_t I, const void* w_gate_up, const void* w_down, moe_dtype dt,
                              const int32_t* topk_idx, const float* topk_w, const void* out) {
  if (!dtype_ok(dt) || T < 0 || k < 1) return MOE_ERR_ARG;
  TRY(check_experts(E));
  if (logits && k > E) return MOE_ERR_ARG;
  TRY(check_width(d));
  TRY(check_width(I));
  const int64_t P = (int64_t)T * k;
  if (P * (d > I ? d : I) >= kMaxElems || (int64_t)T * E >= kMaxElems) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)E * d * 2 * I >= 8 * kMaxElems) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)d * I * 4 >= kMaxElems) return MOE_ERR_UNSUPPORTED;   // one expert's weights < 2 GiB
  if ((int64_t)T * d >= kMaxElems / 2) return MOE_ERR_UNSUPPORTED;   // x is addressed with 32-bit byte offsets
  if (T == 0) return MOE_OK;
  if (!x || !w_gate_up || !w_down || !topk_idx || !topk_w || !out) return MOE_ERR_ARG;
  return MOE_OK;
}

// The layer (moe_forward's work) with its scratch in `workspace`.
// wtiled: the expert weights are in the column-tiled layout of moe_tile_weights.
moe_status forward_impl(const void* x, const float* logits, int32_t T, int32_t d, int32_t E, int32_t k, int32_t I,
                        const void* w_gate_up, const void* w_down, moe_dtype dt, int32_t* topk_idx, float* topk_w,
                        int32_t* expert_offsets, int32_t* row_token, int32_t* pair_row, void* out, void* workspace,
                        size_t workspace_bytes, void* stream, bool wtiled = false) {
  TRY(check_forward_args(x, logits, T, d, E, k, I, w_gate_up, w_down, dt, topk_idx, topk_w, out));
  if (T == 0) return MOE_OK;
  const int64_t P = (int64_t)T * k;
  const ForwardLayout L = forward_layout(T, d, E, k, I, dt);
  if (!workspace || workspace_bytes < L.total) return MOE_ERR_WORKSPACE;

  char* ws = (char*)workspace;
  int32_t* p_row = pair_row ? pair_row : (int32_t*)(ws + L.pair_row);
  int32_t* r_tok = row_token ? row_token : (int32_t*)(ws + L.row_token);
  int32_t* offs = expert_offsets ? expert_offsets : (int32_t*)(ws + L.offsets);
  void* x_perm = ws + L.x_perm;
  void* h = ws + L.h;
  void* y_perm = ws + L.y_perm;
  hipStream_t s = (hipStream_t)stream;

  if (logits) TRY(from_hip(launch_route_topk(logits, T, E, k, topk_idx, topk_w, s)));
  int32_t* sched = dt == MOE_BF16 ? (int32_t*)(ws + L.sched) : nullptr;
  // one pair per token: the down projection writes the output rows itself
  // (times the routing weight) where its tile shape allows, and no combine
  // pass runs
  const bool scatter = dt == MOE_BF16 && k == 1 && down_scatters(P, E, d, I, true);
  float* row_w = scatter ? (float*)(ws + L.row_w) : nullptr;
  if (dt == MOE_BF16) {
    TRY(from_hip(launch_permute_index(topk_idx, P, k, E, r_tok, p_row, offs, ws + L.perm_ws, s, sched,
                                      scatter ? topk_w : nullptr, row_w)));
    if (scatter) TRY(from_hip(launch_zero_unrouted_bf16(p_row, P, T, d, (bf16_t*)out, s)));
    // the gate/up projection reads the token rows in place through row_token
    // (no expert-ordered copy of x is materialised)
    TRY(from_hip(launch_gate_up_bf16((const bf16_t*)x, offs, P, E, d, I, (const bf16_t*)w_gate_up, (bf16_t*)h, s,
                                     r_tok, T, sched, wtiled)));
    if (scatter) {
      const DownScatter sc{(bf16_t*)out, r_tok, row_w, T};
      return from_hip(launch_down_bf16((const bf16_t*)h, offs, P, E, d, I, (const bf16_t*)w_down, nullptr, s,
                                       (float*)(ws + L.split), sched, &sc, false, wtiled));
    }
    TRY(from_hip(launch_down_bf16((const bf16_t*)h, offs, P, E, d, I, (const bf16_t*)w_down, (bf16_t*)y_perm, s,
                                  (float*)(ws + L.split), sched, nullptr, false, wtiled)));
    return from_hip(launch_combine_bf16((const bf16_t*)y_perm, P, p_row, topk_w, T, k, d, (bf16_t*)out, s));
  }
  TRY(from_hip(launch_permute_rows(topk_idx, T, k, E, r_tok, p_row, offs, ws + L.perm_ws, s, nullptr, x,
                                   (int64_t)d * elem_size(dt), x_perm)));
  TRY(from_hip(launch_grouped_ffn_f32((const float*)x_perm, offs, P, E, d, I, (const float*)w_gate_up,
                                      (const float*)w_down, (float*)h, (float*)y_perm, s)));
  return from_hip(launch_combine_f32((const float*)y_perm, P, p_row, topk_w, T, k, d, (float*)out, s));
}

// ---- the layer without a workspace: scratch in a static device array ----
//
// Every GPU the library runs on holds its own copy of `scratch` (at its own
// address) until the process ends.  Host code never passes the array's name
// to a kernel or a copy (on the host it is only a stand-in for the symbol):
// the device address is looked up once per device with hipGetSymbolAddress,
// with that device current, and kept.
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on its first use on
// that device.
hipError_t scratch_address(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

moe_status moe_forward(const void* x, const float* logits, int32_t T, int32_t d, int32_t E, int32_t k, int32_t I,
                       const void* w_gate_up, const void* w_down, moe_dtype dt, int32_t* topk_idx, float* topk_w,
                       int32_t* expert_offsets, int32_t* row_token, int32_t* pair_row, void* out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return forward_impl(x, logits, T, d, E, k, I, w_gate_up, w_down, dt, topk_idx, topk_w, expert_offsets, row_token,
                      pair_row, out, workspace, workspace_bytes, stream);
}

moe_status moe_tile_weights(const void* w_gate_up, const void* w_down, int32_t E, int32_t d, int32_t I, moe_dtype dt,
                            void* w_gate_up_tiled, void* w_down_tiled, void* stream) {
  if (!dtype_ok(dt)) return MOE_ERR_ARG;
  TRY(check_experts(E));
  TRY(check_width(d));
  TRY(check_width(I));
  if (dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)d * I * 2 * 2 >= kMaxElems) return MOE_ERR_UNSUPPORTED;   // one expert's gate/up bytes
  if (!w_gate_up || !w_down || !w_gate_up_tiled || !w_down_tiled) return MOE_ERR_ARG;
  return from_hip(launch_tile_weights_bf16((const bf16_t*)w_gate_up, (const bf16_t*)w_down, E, d, I,
                                           (bf16_t*)w_gate_up_tiled, (bf16_t*)w_down_tiled, (hipStream_t)stream));
}

moe_status moe_forward_tiled(const void* x, const float* logits, int32_t T, int32_t d, int32_t E, int32_t k,
                             int32_t I, const void* w_gate_up_tiled, const void* w_down_tiled, moe_dtype dt,
                             int32_t* topk_idx, float* topk_w, int32_t* expert_offsets, int32_t* row_token,
                             int32_t* pair_row, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (dt == MOE_F32) return MOE_ERR_UNSUPPORTED;
  return forward_impl(x, logits, T, d, E, k, I, w_gate_up_tiled, w_down_tiled, dt, topk_idx, topk_w, expert_offsets,
                      row_token, pair_row, out, workspace, workspace_bytes, stream, true);
}

moe_status moe_forward_noalloc(const void* x, const float* logits, int32_t T, int32_t d, int32_t E, int32_t k,
                               int32_t I, const void* w_gate_up, const void* w_down, moe_dtype dt, int32_t* topk_idx,
                               float* topk_w, int32_t* expert_offsets, int32_t* row_token, int32_t* pair_row,
                               void* out, void* stream) {
  // the arguments first, then the size: a layer that needs more scratch
  // than the array holds is refused before anything is looked up or enqueued
  TRY(check_forward_args(x, logits, T, d, E, k, I, w_gate_up, w_down, dt, topk_idx, topk_w, out));
  if (T == 0) return MOE_OK;
  if (forward_layout(T, d, E, k, I, dt).total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return forward_impl(x, logits, T, d, E, k, I, w_gate_up, w_down, dt, topk_idx, topk_w, expert_offsets, row_token,
                      pair_row, out, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}

size_t moe_backward_workspace_size(int32_t T, int32_t d, int32_t E, int32_t k, int32_t I, moe_dtype dt) {
  if (T < 0 || d < 1 || E < 1 || k < 1 || I < 1 || !dtype_ok(dt)) return 0;
  return backward_layout(T, d, E, k, I, elem_size(dt)).total;
}

namespace {

// Validation shared by the training forward and the backward.
moe_status check_train(moe_dtype dt, int32_t T, int32_t d, int32_t E, int32_t k, int32_t I, const float* logits) {
  if (!dtype_ok(dt) || T < 0 || k < 1) return MOE_ERR_ARG;
  TRY(check_experts(E));
  if (logits && k > E) return MOE_ERR_ARG;
  TRY(check_width(d));
  TRY(check_width(I));
  const int64_t P = (int64_t)T * k;
  if (P * (d > 2 * I ? d : 2 * I) >= kMaxElems || (int64_t)T * E >= kMaxElems) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)E * d * 2 * I >= 8 * kMaxElems) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)d * I * 4 >= kMaxElems) return MOE_ERR_UNSUPPORTED;   // one expert's weights < 2 GiB
  return MOE_OK;
}

// The forward with everything the gradients need kept in a backward-layout
// workspace: routing (with logits), grouping, the grouped copy of x, the
// pre-activations g | u, h and the expert outputs y.
moe_status forward_keep(const void* x, const float* logits, int32_t T, int32_t d, int32_t E, int32_t k, int32_t I,
                        const void* w_gate_up, const void* w_down, moe_dtype dt, int32_t* topk_idx, float* topk_w,
                        const BackwardLayout& L, char* ws, hipStream_t s) {
  const int64_t P = (int64_t)T * k;
  int32_t* p_row = (int32_t*)(ws + L.pair_row);
  int32_t* r_tok = (int32_t*)(ws + L.row_token);
  int32_t* offs = (int32_t*)(ws + L.offsets);
  if (logits) TRY(from_hip(launch_route_topk(logits, T, E, k, topk_idx, topk_w, s)));
  int32_t* sched = (int32_t*)(ws + L.sched);
  TRY(from_hip(launch_permute_rows(topk_idx, T, k, E, r_tok, p_row, offs, ws + L.perm_ws, s, sched, x,
                                   (int64_t)d * elem_size(dt), ws + L.x_perm)));
  if (dt == MOE_F32) {
    float* h = (float*)(ws + L.h);
    TRY(from_hip(launch_gate_up_save_f32((const float*)(ws + L.x_perm), offs, P, E, d, I, (const float*)w_gate_up,
                                         h, (float*)(ws + L.gu), s)));
    return from_hip(launch_down_f32(h, offs, P, E, d, I, (const float*)w_down, (float*)(ws + L.y), s));
  }
  bf16_t* x_perm = (bf16_t*)(ws + L.x_perm);
  bf16_t* h = (bf16_t*)(ws + L.h);
  bf16_t* gu = (bf16_t*)(ws + L.gu);
  bf16_t* y = (bf16_t*)(ws + L.y);
  TRY(from_hip(launch_gate_up_save_bf16(x_perm, offs, P, E, d, I, (const bf16_t*)w_gate_up, h, gu, s, nullptr, 0,
                                        sched)));
  // with one pair per token, moe_forward's down projection writes the output
  // rows from its tiles; these rows come from the same tiles (so a split tail
  // cuts the same ones and the output is moe_forward's bit for bit)
  const bool scatter_tiles = k == 1 && down_scatters(P, E, d, I, true);
  return from_hip(launch_down_bf16(h, offs, P, E, d, I, (const bf16_t*)w_down, y, s, (float*)(ws + L.split), sched,
                                   nullptr, scatter_tiles));
}

}  // namespace

moe_status moe_forward_train(const void* x, const float* logits, int32_t T, int32_t d, int32_t E, int32_t k,
                             int32_t I, const void* w_gate_up, const void* w_down, moe_dtype dt, int32_t* topk_idx,
                             float* topk_w, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  TRY(check_train(dt, T, d, E, k, I, logits));
  if (T == 0) return MOE_OK;
  if (!x || !w_gate_up || !w_down || !topk_idx || !topk_w || !out) return MOE_ERR_ARG;
  const BackwardLayout L = backward_layout(T, d, E, k, I, elem_size(dt));
  if (!workspace || workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  TRY(forward_keep(x, logits, T, d, E, k, I, w_gate_up, w_down, dt, topk_idx, topk_w, L, ws, s));
  if (dt == MOE_F32)
    return from_hip(launch_combine_f32((const float*)(ws + L.y), (int64_t)T * k, (const int32_t*)(ws + L.pair_row),
                                       topk_w, T, k, d, (float*)out, s));
  return from_hip(launch_combine_bf16((const bf16_t*)(ws + L.y), (int64_t)T * k, (const int32_t*)(ws + L.pair_row),
                                      topk_w, T, k, d, (bf16_t*)out, s));
}

moe_status moe_backward(const void* x, const float* logits, int32_t T, int32_t d, int32_t E, int32_t k, int32_t I,
                        const void* w_gate_up, const void* w_down, moe_dtype dt, int32_t* topk_idx, float* topk_w,
                        const void* dout, void* dx, void* dw_gate_up, void* dw_down, float* dtopk_w, float* dlogits,
                        int32_t recompute, void* workspace, size_t workspace_bytes, void* stream) {
  TRY(check_train(dt, T, d, E, k, I, logits));
  if (dlogits && !logits) return MOE_ERR_ARG;
  if (recompute != 0 && recompute != 1) return MOE_ERR_ARG;
  const int64_t P = (int64_t)T * k;
  if (T == 0) {
    // no rows: every weight gradient is zero, and nothing else exists (a
    // float32 element is cleared as two bf16 ones)
    if (E > 0 && (!dw_gate_up || !dw_down)) return MOE_ERR_ARG;
    hipStream_t s0 = (hipStream_t)stream;
    const int64_t halves = dt == MOE_F32 ? 2 : 1;
    TRY(from_hip(launch_zero_bf16((bf16_t*)dw_gate_up, (int64_t)E * d * 2 * I * halves, s0)));
    return from_hip(launch_zero_bf16((bf16_t*)dw_down, (int64_t)E * I * d * halves, s0));
  }
  if (!x || !w_gate_up || !w_down || !topk_idx || !topk_w || !dout || !dx || !dw_gate_up || !dw_down || !dtopk_w)
    return MOE_ERR_ARG;
  const BackwardLayout L = backward_layout(T, d, E, k, I, elem_size(dt));
  if (!workspace || workspace_bytes < L.total) return MOE_ERR_WORKSPACE;

  char* ws = (char*)workspace;
  int32_t* p_row = (int32_t*)(ws + L.pair_row);
  int32_t* r_tok = (int32_t*)(ws + L.row_token);
  int32_t* offs = (int32_t*)(ws + L.offsets);
  bf16_t* x_perm = (bf16_t*)(ws + L.x_perm);
  bf16_t* h = (bf16_t*)(ws + L.h);
  bf16_t* gu = (bf16_t*)(ws + L.gu);
  bf16_t* y = (bf16_t*)(ws + L.y);
  bf16_t* dy = (bf16_t*)(ws + L.dy);
  bf16_t* dgu = (bf16_t*)(ws + L.dgu);
  bf16_t* dxp = (bf16_t*)(ws + L.dxp);
  const bf16_t* wgu = (const bf16_t*)w_gate_up;
  const bf16_t* wd = (const bf16_t*)w_down;
  hipStream_t s = (hipStream_t)stream;

  // the forward again, keeping what the gradients need (or, without
  // recompute, what moe_forward_train left in this workspace)
  if (recompute) TRY(forward_keep(x, logits, T, d, E, k, I, w_gate_up, w_down, dt, topk_idx, topk_w, L, ws, s));
  if (dt == MOE_F32) {
    float* fh = (float*)(ws + L.h);
    float* fgu = (float*)(ws + L.gu);
    float* fdy = (float*)(ws + L.dy);
    float* fdgu = (float*)(ws + L.dgu);
    float* fdxp = (float*)(ws + L.dxp);
    const float* fwgu = (const float*)w_gate_up;
    const float* fwd = (const float*)w_down;
    TRY(from_hip(launch_combine_bwd_f32((const float*)dout, (const float*)(ws + L.y), P, p_row, topk_w, topk_idx, T,
                                        k, d, E, fdy, dtopk_w, dlogits, s)));
    TRY(from_hip(launch_down_dgrad_swiglu_f32(fdy, offs, P, E, d, I, fwd, fgu, fdgu, s)));
    TRY(from_hip(launch_wgrad_f32(fh, I, I, fdy, d, d, offs, P, E, (float*)dw_down, s)));
    TRY(from_hip(launch_gate_up_dgrad_f32(fdgu, offs, P, E, d, I, fwgu, fdxp, s)));
    TRY(from_hip(launch_wgrad_f32((const float*)(ws + L.x_perm), d, d, fdgu, 2 * I, 2 * I, offs, P, E,
                                  (float*)dw_gate_up, s)));
    return from_hip(launch_combine_f32(fdxp, P, p_row, nullptr, T, k, d, (float*)dx, s));
  }
  // combine -> routing weights (and logits) and the expert rows' gradient
  TRY(from_hip(launch_combine_bwd_bf16((const bf16_t*)dout, y, P, p_row, topk_w, topk_idx, T, k, d, E, dy, dtopk_w,
                                       dlogits, s)));
  // down projection and SwiGLU
  TRY(from_hip(launch_down_dgrad_swiglu_bf16(dy, offs, P, E, d, I, wd, gu, dgu, s)));
  TRY(from_hip(launch_wgrad_bf16(h, I, I, dy, d, d, offs, P, E, (bf16_t*)dw_down, s)));
  // gate/up projection
  TRY(from_hip(launch_gate_up_dgrad_bf16(dgu, offs, P, E, d, I, wgu, dxp, s)));
  TRY(from_hip(launch_wgrad_bf16(x_perm, d, d, dgu, 2 * I, 2 * I, offs, P, E, (bf16_t*)dw_gate_up, s)));
  // each token's row gradients summed back in token order
  return from_hip(launch_combine_bf16(dxp, P, p_row, nullptr, T, k, d, (bf16_t*)dx, s));
}

}  // extern "C"
