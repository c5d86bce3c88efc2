// C ABI of the MoE verify-pass library: host-side validation, workspace
// sizing, byte accounting and the launches (the operations themselves are
// described in include/moe_verify.h).  Every argument is checked before any
// work is enqueued, so an invalid call enqueues nothing.
#include "moe_verify.h"

#include <mutex>
#include <vector>

#include "common.h"
#include "partition.h"

// moe_verify_layer_noalloc keeps its workspace (control block, hand-over
// flags, H and the slot outputs the caller keeps none of) in this array.
// In host code `scratch` names a host-side stand-in, never the device
// memory: host code uses only the address hipGetSymbolAddress returns for
// the current device, kept per device in g_scratch.
constexpr size_t kScratchBytes = size_t{16} << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

using moe::kCtrlBytes;
using moe::kHOffset;

constexpr int kMaxN = 32, kMaxK = 8, kMaxE = 256, kMaxS = 4, kMaxDim = 65536;
constexpr int kMaxTreeNodes = 1024;
constexpr int kMaxSetWords = 256;          // 64-bit words of one (layer, expert) set
constexpr int kMaxTreeSetWords = 8192;     // N * W: the footprints fit 64 KB of LDS
constexpr int kMaxSequence = 1 << 22;      // positions of a Bellman reference sequence
constexpr int kMaxDraftLength = 32;        // draft lengths of the Bellman policy (one lane each)

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

thread_local hipError_t g_last_hip = hipSuccess;

// MOE_OK, or MOE_ERR_HIP with the HIP error remembered for moe_last_hip_error()
moe_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip = e;
  return MOE_ERR_HIP;
}

int elem_bytes(int dt) {
  switch (dt) {
    case MOE_F32: return 4;
    case MOE_BF16: return 2;
    case MOE_FP8_E4M3: return 1;
    default: return 0;
  }
}

// token storage type of a weight type (f32 for f32 weights, bf16 otherwise)
int token_bytes(int w_dtype) { return w_dtype == MOE_F32 ? 4 : 2; }

moe_status check_shape(const moe_shape* s) {
  if (s == nullptr) return MOE_ERR_ARG;
  if (s->K < 1 || s->K > kMaxK || s->E < s->K || s->E > kMaxE) return MOE_ERR_ARG;
  if (s->S < 0 || s->S > kMaxS) return MOE_ERR_ARG;
  if (s->d < 1 || s->f < 1 || s->d > kMaxDim || s->f > kMaxDim) return MOE_ERR_ARG;
  const bool ok_combo = (s->w_dtype == MOE_F32 && s->x_dtype == MOE_F32) ||
                        (s->w_dtype == MOE_BF16 && s->x_dtype == MOE_BF16) ||
                        (s->w_dtype == MOE_FP8_E4M3 && s->x_dtype == MOE_BF16);
  if (!ok_combo) return MOE_ERR_UNSUPPORTED;
  const int mult = s->w_dtype == MOE_F32 ? 4 : (s->w_dtype == MOE_BF16 ? 8 : 128);
  if (s->d % mult != 0 || s->f % mult != 0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

uint64_t expert_bytes(const moe_shape* s) {
  uint64_t b = 3ull * static_cast<uint64_t>(s->d) * static_cast<uint64_t>(s->f) *
               static_cast<uint64_t>(elem_bytes(s->w_dtype));
  if (s->w_dtype == MOE_FP8_E4M3) b += 3ull * (s->d / 128) * (s->f / 128) * 4ull;
  return b;
}

size_t h_bytes(const moe_shape* s, int n) {
  return static_cast<size_t>(n) * (s->K + s->S) * s->f * token_bytes(s->w_dtype);
}

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// workspace regions of the one-launch pass after kHOffset: H in f32, then the
// slot outputs the caller does not keep
size_t layer_h_bytes(const moe_shape* s, int n) {
  return round256(static_cast<size_t>(n) * (s->K + s->S) * s->f * 4);
}
size_t layer_ys_bytes(const moe_shape* s, int n) {
  return round256(static_cast<size_t>(n) * s->K * s->d * 4);
}
size_t layer_ysh_bytes(const moe_shape* s, int n) {
  return round256(static_cast<size_t>(n) * s->S * s->d * 4);
}

moe_status check_weights(const moe_shape* s, const moe_weights* w) {
  if (w == nullptr) return MOE_ERR_ARG;
  const void* need[3] = {w->w_gate, w->w_up, w->w_down};
  for (const void* p : need)
    if (p == nullptr || !aligned(p, 16)) return MOE_ERR_ARG;
  if (s->w_dtype == MOE_FP8_E4M3) {
    const void* sc[3] = {w->s_gate, w->s_up, w->s_down};
    for (const void* p : sc)
      if (p == nullptr || !aligned(p, 4)) return MOE_ERR_ARG;
  }
  if (s->S > 0) {
    const void* sh[3] = {w->sh_gate, w->sh_up, w->sh_down};
    for (const void* p : sh)
      if (p == nullptr || !aligned(p, 16)) return MOE_ERR_ARG;
    if (s->w_dtype == MOE_FP8_E4M3) {
      const void* ss[3] = {w->sh_s_gate, w->sh_s_up, w->sh_s_down};
      for (const void* p : ss)
        if (p == nullptr || !aligned(p, 4)) return MOE_ERR_ARG;
    }
  }
  return MOE_OK;
}

moe_status check_ffn_common(const moe_shape* s, const moe_weights* w, const void* x, int n,
                            float* y_slots, float* y_shared, const void* ws, size_t ws_bytes) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (n < 1 || n > kMaxN) return MOE_ERR_ARG;
  st = check_weights(s, w);
  if (st != MOE_OK) return st;
  if (x == nullptr || !aligned(x, 16) || y_slots == nullptr || !aligned(y_slots, 4))
    return MOE_ERR_ARG;
  if (s->S > 0 && (y_shared == nullptr || !aligned(y_shared, 4))) return MOE_ERR_ARG;
  if (ws == nullptr || !aligned(ws, 256)) return MOE_ERR_WORKSPACE;
  if (ws_bytes < kHOffset + h_bytes(s, n)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

moe::FfnParams make_params(const moe_shape* s, const moe_weights* w, const void* x, int n,
                           float* y_slots, float* y_shared, uint64_t* bytes, void* ws) {
  moe::FfnParams p{};
  p.w[0] = static_cast<const uint8_t*>(w->w_gate);
  p.w[1] = static_cast<const uint8_t*>(w->w_up);
  p.w[2] = static_cast<const uint8_t*>(w->w_down);
  p.s[0] = w->s_gate;
  p.s[1] = w->s_up;
  p.s[2] = w->s_down;
  p.shw[0] = static_cast<const uint8_t*>(w->sh_gate);
  p.shw[1] = static_cast<const uint8_t*>(w->sh_up);
  p.shw[2] = static_cast<const uint8_t*>(w->sh_down);
  p.shs[0] = w->sh_s_gate;
  p.shs[1] = w->sh_s_up;
  p.shs[2] = w->sh_s_down;
  p.x = static_cast<const uint8_t*>(x);
  p.err = static_cast<uint32_t*>(ws);
  p.zeros = static_cast<const uint8_t*>(ws) + moe::kZeroOffset;
  p.H = static_cast<uint8_t*>(ws) + kHOffset;
  p.y_slots = y_slots;
  p.y_shared = y_shared;
  p.bytes = bytes;
  p.expert_bytes = expert_bytes(s);
  p.n = n;
  p.K = s->K;
  p.S = s->S;
  p.E = s->E;
  p.d = s->d;
  p.f = s->f;
  p.ucap = n * s->K < s->E ? n * s->K : s->E;
  return p;
}

int wt_of(int w_dtype) {
  return w_dtype == MOE_F32 ? moe::WT_F32 : (w_dtype == MOE_BF16 ? moe::WT_BF16 : moe::WT_FP8);
}


// workspace bytes the one-launch pass needs: control block and flags, H in
// f32, and the slot outputs the caller does not keep
size_t layer_ws_need(const moe_shape* shape, int n, const float* y_slots, const float* y_shared) {
  return kHOffset + layer_h_bytes(shape, n) +
         (y_slots == nullptr ? layer_ys_bytes(shape, n) : 0) +
         (y_shared == nullptr ? layer_ysh_bytes(shape, n) : 0);
}

// argument checks of the one-launch pass shared by its fixed-mode and
// automatic-mode entry points, everything but the workspace
moe_status layer_args_check(const moe_shape* shape, const moe_weights* w, const float* logits,
                            const void* x, int n, int mode, void* out, int out_dtype,
                            const float* y_slots, const float* y_shared, const uint64_t* bytes) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (n < 1 || n > kMaxN) return MOE_ERR_ARG;
  if (mode != MOE_MODE_DEDUP && mode != MOE_MODE_PERSLOT) return MOE_ERR_ARG;
  st = check_weights(shape, w);
  if (st != MOE_OK) return st;
  if (logits == nullptr || !aligned(logits, 4)) return MOE_ERR_ARG;
  if (x == nullptr || !aligned(x, 16) || out == nullptr || !aligned(out, 16)) return MOE_ERR_ARG;
  if (out_dtype != MOE_F32 && out_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if ((y_slots != nullptr && !aligned(y_slots, 16)) ||
      (y_shared != nullptr && !aligned(y_shared, 16)))
    return MOE_ERR_ARG;
  if (bytes != nullptr && !aligned(bytes, 8)) return MOE_ERR_ARG;
  return MOE_OK;
}

moe_status moe_verify_layer_check(const moe_shape* shape, const moe_weights* w,
                                  const float* logits, const void* x, int n, int mode, void* out,
                                  int out_dtype, const float* y_slots, const float* y_shared,
                                  const uint64_t* bytes, const void* ws, size_t ws_bytes) {
  moe_status st = layer_args_check(shape, w, logits, x, n, mode, out, out_dtype, y_slots,
                                   y_shared, bytes);
  if (st != MOE_OK) return st;
  if (ws == nullptr || !aligned(ws, 256)) return MOE_ERR_WORKSPACE;
  if (ws_bytes < layer_ws_need(shape, n, y_slots, y_shared)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// the optional routing and union outputs of the fixed-mode pass: 4-byte
// aligned, the five union arrays all or none
moe_status layer_outputs_check(const int32_t* ids, const float* gates, const int32_t* U,
                               const int32_t* union_ids, const int32_t* offsets,
                               const int32_t* perm, const int32_t* slot_rank, int* given) {
  if ((ids != nullptr && !aligned(ids, 4)) || (gates != nullptr && !aligned(gates, 4)))
    return MOE_ERR_ARG;
  const void* uni[5] = {U, union_ids, offsets, perm, slot_rank};
  *given = 0;
  for (const void* p : uni) {
    if (p != nullptr && !aligned(p, 4)) return MOE_ERR_ARG;
    *given += p != nullptr;
  }
  if (*given != 0 && *given != 5) return MOE_ERR_ARG;
  return MOE_OK;
}

// launch parameters of the one-launch pass (arguments already checked)
moe::LayerParams layer_params(const moe_shape* shape, const moe_weights* w, const float* logits,
                              const void* x, int n, int mode, void* out, int out_dtype,
                              float* y_slots, float* y_shared, uint64_t* bytes, void* ws) {
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint8_t* next = base + kHOffset + layer_h_bytes(shape, n);
  if (y_slots == nullptr) {
    y_slots = reinterpret_cast<float*>(next);
    next += layer_ys_bytes(shape, n);
  }
  if (y_shared == nullptr) y_shared = reinterpret_cast<float*>(next);
  moe::LayerParams lp{};
  lp.f = make_params(shape, w, x, n, y_slots, y_shared, bytes, ws);
  lp.f.mode = mode;
  lp.logits = logits;
  lp.out = out;
  lp.out_bf16 = out_dtype == MOE_BF16;
  lp.epoch = reinterpret_cast<unsigned*>(base + moe::kEpochOffset);
  lp.spin = reinterpret_cast<const unsigned*>(base + moe::kSpinOffset);
  lp.up_flags = reinterpret_cast<unsigned*>(base + moe::kFlagsOffset);
  lp.down_flags = lp.up_flags + moe::kMaxGrid;
  return lp;
}

// the one-launch pass of moe_verify_layer / moe_verify_layer_budget (budget
// 0: none)
moe_status verify_layer_impl(const moe_shape* shape, const moe_weights* w, const float* logits,
                             const void* x, int n, int mode, int budget, int renorm, void* out,
                             int out_dtype, int32_t* ids, float* gates, int32_t* U,
                             int32_t* union_ids, int32_t* offsets, int32_t* perm,
                             int32_t* slot_rank, float* y_slots, float* y_shared, uint64_t* bytes,
                             void* ws, size_t ws_bytes, moe_stream_t stream) {
  if (mode != MOE_MODE_DEDUP && mode != MOE_MODE_PERSLOT) return MOE_ERR_ARG;
  moe_status st = moe_verify_layer_check(shape, w, logits, x, n, mode, out, out_dtype, y_slots,
                                         y_shared, bytes, ws, ws_bytes);
  if (st != MOE_OK) return st;
  int given = 0;
  st = layer_outputs_check(ids, gates, U, union_ids, offsets, perm, slot_rank, &given);
  if (st != MOE_OK) return st;
  moe::LayerParams lp = layer_params(
      shape, w, logits, x, n, mode == MOE_MODE_DEDUP ? moe::MODE_DEDUP : moe::MODE_PERSLOT, out,
      out_dtype, y_slots, y_shared, bytes, ws);
  lp.ids = ids;
  lp.gates = gates;
  lp.budget = budget;
  lp.renorm = renorm;
  if (mode == MOE_MODE_DEDUP && given == 5) {
    lp.U = U;
    lp.union_ids = union_ids;
    lp.offsets = offsets;
    lp.perm = perm;
    lp.slot_rank = slot_rank;
  }
  return hip_status(moe::launch_layer(lp, wt_of(shape->w_dtype), static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------- allocation-free variant

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// This device's scratch address, set up on the first call on the device
// (with the device current): the symbol's address is looked up once and
// the control block and flags are cleared with a fill kernel on `stream`,
// ahead of the call that follows on the same stream (device globals start
// zero-filled; the clear states the requirement).  Under stream capture
// the clear becomes the graph's first node.
moe_status scratch_of_current_device(hipStream_t stream, void** out) {
  int dev = 0;
  moe_status st = hip_status(hipGetDevice(&dev));
  if (st != MOE_OK) return st;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    st = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (st != MOE_OK) return st;
    if (p == nullptr || !aligned(p, 256)) return MOE_ERR_WORKSPACE;
    st = hip_status(moe::launch_fill_zero(p, kHOffset, stream));
    if (st != MOE_OK) return st;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

// the scratch address of the current device if a call has set it up there
void* scratch_if_set_up() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  return g_scratch[dev];
}
}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(int32_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported dtype or shape";
    case MOE_ERR_WORKSPACE: return "workspace too small or misaligned";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_BAD_IDS: return "expert id outside [0, E)";
    case MOE_ERR_TIMEOUT: return "bounded device wait gave up";
    case MOE_ERR_BAD_TREE: return "draft tree or probabilities out of range";
    case MOE_ERR_TOO_LARGE: return "pass needs more scratch than the static array holds";
    default: return "unknown status";
  }
}

moe_status moe_route_topk(const float* logits, int32_t n, int32_t E, int32_t K, int32_t* ids,
                          float* gates, moe_stream_t stream) {
  if (n < 1 || n > kMaxN || K < 1 || K > kMaxK || E < K || E > kMaxE) return MOE_ERR_ARG;
  if (logits == nullptr || ids == nullptr || gates == nullptr) return MOE_ERR_ARG;
  if (!aligned(logits, 4) || !aligned(ids, 4) || !aligned(gates, 4)) return MOE_ERR_ARG;
  return hip_status(moe::launch_route_topk(logits, n, E, K, ids, gates, static_cast<hipStream_t>(stream)));
}

moe_status moe_build_union(const int32_t* ids, int32_t n, int32_t K, int32_t E, int32_t* U,
                           int32_t* union_ids, int32_t* offsets, int32_t* perm,
                           int32_t* slot_rank, moe_stream_t stream) {
  if (n < 1 || n > kMaxN || K < 1 || K > kMaxK || E < K || E > kMaxE) return MOE_ERR_ARG;
  const void* ptrs[6] = {ids, U, union_ids, offsets, perm, slot_rank};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned(p, 4)) return MOE_ERR_ARG;
  return hip_status(moe::launch_build_union(ids, n, K, E, U, union_ids, offsets, perm, slot_rank,
                                 static_cast<hipStream_t>(stream)));
}

moe_status moe_route_union(const float* logits, int32_t n, int32_t E, int32_t K, int32_t* ids,
                           float* gates, int32_t* U, int32_t* union_ids, int32_t* offsets,
                           int32_t* perm, int32_t* slot_rank, moe_stream_t stream) {
  if (n < 1 || n > kMaxN || K < 1 || K > kMaxK || E < K || E > kMaxE) return MOE_ERR_ARG;
  const void* ptrs[8] = {logits, ids, gates, U, union_ids, offsets, perm, slot_rank};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned(p, 4)) return MOE_ERR_ARG;
  return hip_status(moe::launch_route_union(logits, n, E, K, ids, gates, U, union_ids, offsets, perm,
                                 slot_rank, static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_ffn_dedup(const moe_shape* shape, const moe_weights* w, const void* x,
                                int32_t n, const int32_t* U, const int32_t* union_ids,
                                const int32_t* offsets, const int32_t* perm, float* y_slots,
                                float* y_shared, uint64_t* bytes, void* ws, size_t ws_bytes,
                                moe_stream_t stream) {
  moe_status st = check_ffn_common(shape, w, x, n, y_slots, y_shared, ws, ws_bytes);
  if (st != MOE_OK) return st;
  const void* ptrs[4] = {U, union_ids, offsets, perm};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned(p, 4)) return MOE_ERR_ARG;
  if (bytes != nullptr && !aligned(bytes, 8)) return MOE_ERR_ARG;
  moe::FfnParams p = make_params(shape, w, x, n, y_slots, y_shared, bytes, ws);
  p.mode = moe::MODE_DEDUP;
  p.U = U;
  p.union_ids = union_ids;
  p.offsets = offsets;
  p.perm = perm;
  return hip_status(moe::launch_expert_ffn(p, wt_of(shape->w_dtype), static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_ffn_perslot(const moe_shape* shape, const moe_weights* w, const void* x,
                                  int32_t n, const int32_t* ids, float* y_slots, float* y_shared,
                                  uint64_t* bytes, void* ws, size_t ws_bytes,
                                  moe_stream_t stream) {
  moe_status st = check_ffn_common(shape, w, x, n, y_slots, y_shared, ws, ws_bytes);
  if (st != MOE_OK) return st;
  if (ids == nullptr || !aligned(ids, 4)) return MOE_ERR_ARG;
  if (bytes != nullptr && !aligned(bytes, 8)) return MOE_ERR_ARG;
  moe::FfnParams p = make_params(shape, w, x, n, y_slots, y_shared, bytes, ws);
  p.mode = moe::MODE_PERSLOT;
  p.ids = ids;
  return hip_status(moe::launch_expert_ffn(p, wt_of(shape->w_dtype), static_cast<hipStream_t>(stream)));
}

moe_status moe_combine(const float* y_slots, const float* gates, const float* y_shared,
                       int32_t n, int32_t K, int32_t S, int32_t d, void* out, int32_t out_dtype,
                       moe_stream_t stream) {
  if (n < 1 || n > kMaxN || K < 1 || K > kMaxK || S < 0 || S > kMaxS || d < 1 || d > kMaxDim)
    return MOE_ERR_ARG;
  if (y_slots == nullptr || gates == nullptr || out == nullptr) return MOE_ERR_ARG;
  if (S > 0 && y_shared == nullptr) return MOE_ERR_ARG;
  if (out_dtype != MOE_F32 && out_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (d % 4 != 0) return MOE_ERR_UNSUPPORTED;  // four columns per lane
  if (!aligned(y_slots, 16) || !aligned(gates, 4) || !aligned(out, 16)) return MOE_ERR_ARG;
  if (S > 0 && !aligned(y_shared, 16)) return MOE_ERR_ARG;
  return hip_status(moe::launch_combine(y_slots, gates, y_shared, n, K, S, d, out, out_dtype == MOE_BF16,
                             static_cast<hipStream_t>(stream)));
}

size_t moe_workspace_size(const moe_shape* shape, int32_t n_max, int32_t mode) {
  if (check_shape(shape) != MOE_OK || n_max < 1 || n_max > kMaxN) return 0;
  if (mode != MOE_MODE_DEDUP && mode != MOE_MODE_PERSLOT) return 0;
  // the largest need of any entry point: the one-launch pass keeping its
  // slot outputs in the workspace
  return kHOffset + layer_h_bytes(shape, n_max) + layer_ys_bytes(shape, n_max) +
         layer_ysh_bytes(shape, n_max);
}

moe_status moe_verify_layer(const moe_shape* shape, const moe_weights* w, const float* logits,
                            const void* x, int32_t n, int32_t mode, void* out, int32_t out_dtype,
                            int32_t* ids, float* gates, int32_t* U, int32_t* union_ids,
                            int32_t* offsets, int32_t* perm, int32_t* slot_rank, float* y_slots,
                            float* y_shared, uint64_t* bytes, void* ws, size_t ws_bytes,
                            moe_stream_t stream) {
  return verify_layer_impl(shape, w, logits, x, n, mode, 0, 0, out, out_dtype, ids, gates, U,
                           union_ids, offsets, perm, slot_rank, y_slots, y_shared, bytes, ws,
                           ws_bytes, stream);
}

moe_status moe_verify_layer_noalloc(const moe_shape* shape, const moe_weights* w,
                                    const float* logits, const void* x, int32_t n, int32_t mode,
                                    void* out, int32_t out_dtype, int32_t* ids, float* gates,
                                    int32_t* U, int32_t* union_ids, int32_t* offsets,
                                    int32_t* perm, int32_t* slot_rank, float* y_slots,
                                    float* y_shared, uint64_t* bytes, moe_stream_t stream) {
  // every argument is checked before the scratch is touched
  moe_status st = layer_args_check(shape, w, logits, x, n, mode, out, out_dtype, y_slots,
                                   y_shared, bytes);
  if (st != MOE_OK) return st;
  int given = 0;
  st = layer_outputs_check(ids, gates, U, union_ids, offsets, perm, slot_rank, &given);
  if (st != MOE_OK) return st;
  if (layer_ws_need(shape, n, y_slots, y_shared) > kScratchBytes) return MOE_ERR_TOO_LARGE;
  void* ws = nullptr;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  st = scratch_of_current_device(s, &ws);
  if (st != MOE_OK) return st;
  return verify_layer_impl(shape, w, logits, x, n, mode, 0, 0, out, out_dtype, ids, gates, U,
                           union_ids, offsets, perm, slot_rank, y_slots, y_shared, bytes, ws,
                           kScratchBytes, stream);
}

moe_status moe_verify_layer_budget(const moe_shape* shape, const moe_weights* w,
                                   const float* logits, const void* x, int32_t n, int32_t C,
                                   int32_t renorm, void* out, int32_t out_dtype, int32_t* ids,
                                   float* gates, int32_t* U, int32_t* union_ids, int32_t* offsets,
                                   int32_t* perm, int32_t* slot_rank, float* y_slots,
                                   float* y_shared, uint64_t* bytes, void* ws, size_t ws_bytes,
                                   moe_stream_t stream) {
  if (C < 1 || (renorm != 0 && renorm != 1)) return MOE_ERR_ARG;
  return verify_layer_impl(shape, w, logits, x, n, MOE_MODE_DEDUP, C, renorm, out, out_dtype,
                           ids, gates, U, union_ids, offsets, perm, slot_rank, y_slots, y_shared,
                           bytes, ws, ws_bytes, stream);
}

moe_status moe_expert_budget(const float* gates, int32_t n, int32_t K, int32_t E, int32_t C,
                             int32_t renorm, int32_t* U, int32_t* union_ids, int32_t* offsets,
                             int32_t* perm, int32_t* slot_rank, float* gates_out,
                             moe_stream_t stream) {
  if (n < 1 || n > kMaxN || K < 1 || K > kMaxK || E < K || E > kMaxE) return MOE_ERR_ARG;
  if (C < 1 || (renorm != 0 && renorm != 1)) return MOE_ERR_ARG;
  const void* ptrs[7] = {gates, U, union_ids, offsets, perm, slot_rank, gates_out};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned(p, 4)) return MOE_ERR_ARG;
  return hip_status(moe::launch_expert_budget(gates, n, K, E, C, renorm, U, union_ids, offsets,
                                              perm, slot_rank, gates_out,
                                              static_cast<hipStream_t>(stream)));
}

moe_status moe_verify_layer_auto(const moe_shape* shape, const moe_weights* w,
                                 const float* logits, const void* x, int32_t n, float r,
                                 void* out, int32_t out_dtype, int32_t* mode_out,
                                 uint64_t* bytes, void* ws, size_t ws_bytes,
                                 moe_stream_t stream) {
  if (!(r >= 0.0f) || r > 1e30f) return MOE_ERR_ARG;  // rejects NaN and infinities
  if (mode_out != nullptr && !aligned(mode_out, 4)) return MOE_ERR_ARG;
  // validate and lay out exactly as the fixed-mode call (deduplicating shape
  // of the arguments; the workspace need is the same for both modes)
  moe_status st = moe_verify_layer_check(shape, w, logits, x, n, MOE_MODE_DEDUP, out, out_dtype,
                                         nullptr, nullptr, bytes, ws, ws_bytes);
  if (st != MOE_OK) return st;
  moe::LayerParams lp = layer_params(shape, w, logits, x, n, moe::MODE_AUTO, out, out_dtype,
                                     nullptr, nullptr, bytes, ws);
  lp.r_auto = r;
  lp.mode_out = mode_out;
  return hip_status(moe::launch_layer(lp, wt_of(shape->w_dtype), static_cast<hipStream_t>(stream)));
}

moe_status moe_evict_select(const int32_t* parent, const float* q, const float* cost, int32_t N,
                            int32_t* order, double* scores, double* expected, int32_t* k_best,
                            void* ws, size_t ws_bytes, moe_stream_t stream) {
  if (N < 1 || N > kMaxTreeNodes) return MOE_ERR_ARG;
  const void* need4[5] = {parent, q, cost, order, k_best};
  for (const void* p : need4)
    if (p == nullptr || !aligned(p, 4)) return MOE_ERR_ARG;
  if ((scores != nullptr && !aligned(scores, 8)) || (expected != nullptr && !aligned(expected, 8)))
    return MOE_ERR_ARG;
  if (ws == nullptr || !aligned(ws, 256) || ws_bytes < kCtrlBytes) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_evict(parent, q, cost, N, order, scores, expected, k_best,
                                      static_cast<uint32_t*>(ws), static_cast<hipStream_t>(stream)));
}

moe_status moe_ecospec_select(const int32_t* parent, const float* q, const uint64_t* pred,
                              const uint64_t* buffer0, int32_t N, int32_t W, int32_t gamma,
                              double eps, int32_t* selected, uint64_t* buffer_out, void* ws,
                              size_t ws_bytes, moe_stream_t stream) {
  if (N < 1 || N > kMaxTreeNodes || W < 1 || W > kMaxSetWords || gamma < 1 || gamma > N)
    return MOE_ERR_ARG;
  if (static_cast<long long>(N) * W > kMaxTreeSetWords) return MOE_ERR_UNSUPPORTED;
  if (!(eps > 0.0) || eps > 1e300) return MOE_ERR_ARG;
  const void* need4[3] = {parent, q, selected};
  for (const void* p : need4)
    if (p == nullptr || !aligned(p, 4)) return MOE_ERR_ARG;
  if (pred == nullptr || !aligned(pred, 8)) return MOE_ERR_ARG;
  if ((buffer0 != nullptr && !aligned(buffer0, 8)) ||
      (buffer_out != nullptr && !aligned(buffer_out, 8)))
    return MOE_ERR_ARG;
  if (ws == nullptr || !aligned(ws, 256) || ws_bytes < kCtrlBytes) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_ecospec(parent, q, pred, buffer0, N, W, gamma, eps, selected,
                                        buffer_out, static_cast<uint32_t*>(ws),
                                        static_cast<hipStream_t>(stream)));
}

moe_status moe_bellman_policy(const double* q, const double* cost, int32_t N, int32_t L,
                              double* dp, int32_t* k_best, void* ws, size_t ws_bytes,
                              moe_stream_t stream) {
  if (N < 1 || N > kMaxSequence || L < 1 || L > kMaxDraftLength) return MOE_ERR_ARG;
  const void* need8[3] = {q, cost, dp};
  for (const void* p : need8)
    if (p == nullptr || !aligned(p, 8)) return MOE_ERR_ARG;
  if (k_best == nullptr || !aligned(k_best, 4)) return MOE_ERR_ARG;
  if (ws == nullptr || !aligned(ws, 256) || ws_bytes < kCtrlBytes) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_bellman(q, cost, N, L, dp, k_best, static_cast<uint32_t*>(ws),
                                        static_cast<hipStream_t>(stream)));
}

moe_status moe_pack_weights(const moe_shape* shape, int32_t count, const void* src_gate,
                            const void* src_up, const void* src_down, const float* src_s_gate,
                            const float* src_s_up, const float* src_s_down, void* dst_gate,
                            void* dst_up, void* dst_down, float* dst_s_gate, float* dst_s_up,
                            float* dst_s_down, moe_stream_t stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (count < 1 || count > kMaxE) return MOE_ERR_ARG;
  const int es = elem_bytes(shape->w_dtype);
  const void* src[3] = {src_gate, src_up, src_down};
  void* dst[3] = {dst_gate, dst_up, dst_down};
  for (int m = 0; m < 3; ++m) {
    if (src[m] == nullptr || dst[m] == nullptr || src[m] == dst[m]) return MOE_ERR_ARG;
    if (!aligned(src[m], es) || !aligned(dst[m], es)) return MOE_ERR_ARG;
  }
  const bool fp8 = shape->w_dtype == MOE_FP8_E4M3;
  const float* ssrc[3] = {src_s_gate, src_s_up, src_s_down};
  float* sdst[3] = {dst_s_gate, dst_s_up, dst_s_down};
  if (fp8)
    for (int m = 0; m < 3; ++m)
      if (ssrc[m] == nullptr || sdst[m] == nullptr || ssrc[m] == sdst[m] || !aligned(ssrc[m], 4) ||
          !aligned(sdst[m], 4))
        return MOE_ERR_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int d = shape->d, f = shape->f;
  // gate, up: [count][d][f] -> [count][f][d]; down: [count][f][d] -> [count][d][f]
  const int rows[3] = {d, d, f}, cols[3] = {f, f, d};
  for (int m = 0; m < 3; ++m) {
    st = hip_status(moe::launch_transpose(src[m], dst[m], count, rows[m], cols[m], es, s));
    if (st != MOE_OK) return st;
    if (fp8) {
      st = hip_status(moe::launch_transpose(ssrc[m], sdst[m], count, rows[m] / 128, cols[m] / 128,
                                            4, s));
      if (st != MOE_OK) return st;
    }
  }
  return MOE_OK;
}

moe_status moe_workspace_init(void* ws, size_t ws_bytes, moe_stream_t stream) {
  if (ws == nullptr || !aligned(ws, 256) || ws_bytes < kCtrlBytes) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_fill_zero(ws, ws_bytes, static_cast<hipStream_t>(stream)));
}

moe_status moe_byte_counts(const moe_shape* shape, int32_t n, int32_t U, uint64_t* union_bytes,
                           uint64_t* requested_bytes) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (n < 1 || n > kMaxN) return MOE_ERR_ARG;
  const int cap = n * shape->K < shape->E ? n * shape->K : shape->E;
  if (U < shape->K || U > cap) return MOE_ERR_ARG;
  const uint64_t b = expert_bytes(shape);
  if (union_bytes) *union_bytes = static_cast<uint64_t>(U + shape->S) * b;
  if (requested_bytes) *requested_bytes = static_cast<uint64_t>(n) * (shape->K + shape->S) * b;
  return MOE_OK;
}

int32_t moe_last_hip_error(void) { return static_cast<int32_t>(g_last_hip); }

const char* moe_hip_error_string(void) { return hipGetErrorString(g_last_hip); }

moe_status moe_get_error(void* ws, moe_stream_t stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (ws == nullptr) {
    // the static scratch of moe_verify_layer_noalloc on the current device
    ws = scratch_if_set_up();
    if (ws == nullptr) return hip_status(hipStreamSynchronize(s));  // no call ran there
  }
  if (!aligned(ws, 256)) return MOE_ERR_WORKSPACE;
  moe_status st = hip_status(hipStreamSynchronize(s));
  if (st != MOE_OK) return st;
  uint32_t word = 0;
  st = hip_status(hipMemcpy(&word, ws, sizeof(word), hipMemcpyDeviceToHost));
  if (st != MOE_OK) return st;
  if (word == 0) return MOE_OK;
  const uint32_t zero = 0;
  st = hip_status(hipMemcpy(ws, &zero, sizeof(zero), hipMemcpyHostToDevice));
  if (st != MOE_OK) return st;
  if (word & moe::ERRBIT_BAD_IDS) return MOE_ERR_BAD_IDS;
  if (word & moe::ERRBIT_BAD_TREE) return MOE_ERR_BAD_TREE;
  return MOE_ERR_TIMEOUT;
}

moe_status moe_unit_partition(const int32_t* counts, int32_t ng, int32_t tile, int32_t up,
                              int32_t upg, int32_t grid, int64_t* first_unit, int32_t* owner_lo,
                              int32_t* owner_hi) {
  if (counts == nullptr || first_unit == nullptr || ng < 1 || ng > moe::kCostGroups ||
      upg < 1 || upg > 16384 || grid < 1 || grid > moe::kMaxGrid ||
      (tile != 0 && tile != 8 && tile != 16 && tile != 32) || (owner_lo == nullptr) != (owner_hi == nullptr))
    return MOE_ERR_ARG;
  for (int g = 0; g < ng; ++g)
    if (counts[g] < 0 || counts[g] > 32) return MOE_ERR_ARG;
  const long long nu = static_cast<long long>(ng) * upg;
  std::vector<int> cpre(static_cast<size_t>(ng) + 1, 0);
  long long ctot = nu;
  if (tile > 0) {
    for (int g = 0; g < ng; ++g) cpre[g + 1] = cpre[g] + moe::unit_cost(counts[g], tile, up != 0) * upg;
    ctot = cpre[ng];
  }
  for (int c = 0; c <= grid; ++c)
    first_unit[c] = tile > 0 ? moe::weighted_first_unit(cpre.data(), ng, upg, ctot, grid, c, nu)
                             : moe::div_small(nu * c, grid);
  if (owner_lo != nullptr)
    for (int g = 0; g < ng; ++g)
      moe::group_owners(tile > 0 ? cpre.data() : nullptr, ctot, nu, grid, upg, g, owner_lo[g],
                        owner_hi[g]);
  return MOE_OK;
}

moe_status moe_decode_fp8(const uint8_t* codes, float* out, int64_t count, moe_stream_t stream) {
  if (count < 0 || (count > 0 && (codes == nullptr || out == nullptr))) return MOE_ERR_ARG;
  if (out != nullptr && !aligned(out, 4)) return MOE_ERR_ARG;
  return hip_status(moe::launch_decode_fp8(codes, out, count, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
