// Internal declarations of the MoE verify-pass library (gfx950 / CDNA4).
// Device helpers shared by the kernels and the launch functions the C ABI
// layer calls.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBlock = 256;  // 4 waves
// The streaming kernels (expert FFN, one-launch pass) run one workgroup per
// CU of twelve wavefronts (three per SIMD, at most 168 VGPRs) that share the
// CU's work through an LDS counter.
constexpr int kStreamWaves = 12;
// Their block size as a constant: device code that reads blockDim.x gets it
// through a global load, and the wait for that load (loads complete in
// order) would first drain every weight load in flight.
constexpr int kStreamThreads = kStreamWaves * kWave;
constexpr int kMaxStreamWaves = 16;  // routing scratch is sized for up to this many

enum { WT_F32 = 0, WT_BF16 = 1, WT_FP8 = 2 };
enum { MODE_DEDUP = 0, MODE_PERSLOT = 1, MODE_AUTO = 2 };  // AUTO: the one-launch pass decides
enum : uint32_t { ERRBIT_BAD_IDS = 1u, ERRBIT_TIMEOUT = 2u, ERRBIT_BAD_TREE = 4u };

// Workspace: [0, kCtrlBytes) control words (error word first, the epoch of
// the one-launch pass at kEpochOffset; bytes [kZeroOffset, kZeroOffset + 16)
// are never written and stay zero), then the hand-over flags of the
// one-launch pass (two arrays of kMaxGrid words), then the intermediate
// activations H [n*(K+S)][f] (token storage type for the two-kernel FFN, f32
// for the one-launch pass), then, for the one-launch pass, y_slots and
// y_shared when the caller keeps none.
constexpr size_t kCtrlBytes = 256;
constexpr size_t kEpochOffset = 64;
constexpr size_t kZeroOffset = 128;
// a nonzero word here replaces kSpinLimit for the one-launch pass (tests
// lower it to make a bounded wait give up; zero after moe_workspace_init)
constexpr size_t kSpinOffset = 192;
constexpr int kMaxGrid = 4096;
constexpr size_t kFlagsOffset = kCtrlBytes;
constexpr size_t kHOffset = kFlagsOffset + 2 * kMaxGrid * 4;
// bounded waits: polls of about a microsecond each before a time-out
constexpr int kSpinLimit = 1 << 21;

// ----------------------------------------------------------------- loads
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
__device__ __forceinline__ bf16x2 as_bf16x2(unsigned v) {
  return __builtin_bit_cast(bf16x2, v);
}

// Two E4M3FN codes (bytes 0,1 of the dword when hi == false, bytes 2,3
// otherwise) -> two bf16 values, exactly (every E4M3FN value is a bf16 value).
template <bool hi>
__device__ __forceinline__ bf16x2 fp8x2_to_bf16x2(unsigned w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, hi);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<unsigned>(b) << 16);
}

// Round-to-nearest-even f32 -> bf16 bits (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  unsigned u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// ---------------------------------------------------- FFN launch parameters
struct FfnParams {
  const uint8_t* w[3];    // routed gate [E][f][d], up [E][f][d], down [E][d][f]
  const float* s[3];      // fp8 block scales of the same three matrices
  const uint8_t* shw[3];  // shared experts, same layouts with S for E
  const float* shs[3];
  const uint8_t* x;       // [n][d] tokens
  uint8_t* H;             // [n*(K+S)][f] intermediate activations
  float* y_slots;         // [n][K][d]
  float* y_shared;        // [n][S][d]
  const int32_t* U;       // dedup: union size (device)
  const int32_t* union_ids;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* ids;     // per-slot: [n][K]
  uint32_t* err;          // error word (workspace)
  const uint8_t* zeros;   // 16 zero bytes inside the workspace control block
  uint64_t* bytes;        // [2] or null
  unsigned long long expert_bytes;
  int n, K, S, E, d, f;
  int ucap;               // dedup: upper bound of U = min(n*K, E)
  int mode;
  int lds_slots;          // token slots in LDS (set by the launcher)
  long long lds_bytes;    // dynamic LDS of the launch (set by the launcher)
};

// One MoE layer of a verify pass in one launch (fused.hip).
struct LayerParams {
  FfnParams f;            // weights, tokens, H (f32), slot outputs, shape, mode
  const float* logits;    // [n][E]
  int32_t* ids;           // optional [n][K]
  float* gates;           // optional [n][K]
  int32_t* U;             // optional (dedup): union size and arrays
  int32_t* union_ids;
  int32_t* offsets;
  int32_t* perm;
  int32_t* slot_rank;
  void* out;              // [n][d]
  int out_bf16;
  float r_auto;           // MODE_AUTO: deduplicate iff (U+S) < r_auto * n*(K+S)
  int32_t* mode_out;      // optional: the mode a MODE_AUTO pass ran
  unsigned* epoch;        // call counter of the workspace
  const unsigned* spin;   // polls of a bounded wait (0: kSpinLimit)
  unsigned* up_flags;     // [kMaxGrid] UP range done (tag of the call)
  unsigned* down_flags;   // [kMaxGrid] DOWN range done
  int budget;             // dedup: keep at most this many routed experts (0: no budget)
  int renorm;             // budget: renormalise the kept gates of a token that lost a slot
};

// Tile shapes of the dot-product FFN phases (rows per wave R, load steps per
// chunk SPC for UP and DOWN), the measured best on MI355X.
constexpr int kRowsUp = 1, kStepsUp = 4;
constexpr int kRowsDown = 4, kStepsDown = 2;

// token tile: a group serves at most n tokens (a token names an expert once),
// so the tile is the next power of two of n (up to 32); f32 weights take at
// most 8 and larger groups take several tiles
inline int token_tile(int mode, int n) {
  if (mode == MODE_PERSLOT) return 1;
  return n >= 17 ? 32 : (n >= 9 ? 16 : (n >= 5 ? 8 : (n >= 3 ? 4 : (n == 2 ? 2 : 1))));
}

// resident workgroups of a kernel of `block` threads on the current device
int resident_blocks(const void* fn, size_t smem, int block);
// CUs a launch on stream s may occupy (its CU mask), 0 if unknown
int stream_cus(hipStream_t s);
// dynamic LDS a launch of fn may take on the current device (the device's
// per-workgroup LDS less fn's static LDS); 0 if the query fails
size_t lds_budget(const void* fn);

hipError_t launch_route_topk(const float* logits, int n, int E, int K, int32_t* ids,
                             float* gates, hipStream_t s);
hipError_t launch_build_union(const int32_t* ids, int n, int K, int E, int32_t* U,
                              int32_t* union_ids, int32_t* offsets, int32_t* perm,
                              int32_t* slot_rank, hipStream_t s);
hipError_t launch_route_union(const float* logits, int n, int E, int K, int32_t* ids,
                              float* gates, int32_t* U, int32_t* union_ids, int32_t* offsets,
                              int32_t* perm, int32_t* slot_rank, hipStream_t s);
hipError_t launch_expert_budget(const float* gates, int n, int K, int E, int C, int renorm,
                                int32_t* U, int32_t* union_ids, int32_t* offsets, int32_t* perm,
                                int32_t* slot_rank, float* gates_out, hipStream_t s);
hipError_t launch_expert_ffn(const FfnParams& p, int w_dtype, hipStream_t s);
hipError_t launch_layer(const LayerParams& lp, int w_dtype, hipStream_t s);
hipError_t launch_combine(const float* y_slots, const float* gates, const float* y_shared,
                          int n, int K, int S, int d, void* out, int out_bf16, hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
// [count][R][C] -> [count][C][R] of 1-, 2- or 4-byte elements
hipError_t launch_transpose(const void* src, void* dst, int count, int R, int C, int elem,
                            hipStream_t s);
hipError_t launch_ecospec(const int32_t* parent, const float* q, const uint64_t* pred,
                          const uint64_t* buffer0, int N, int W, int gamma, double eps,
                          int32_t* selected, uint64_t* buffer_out, uint32_t* err, hipStream_t s);
hipError_t launch_evict(const int32_t* parent, const float* q, const float* cost, int N,
                        int32_t* order, double* scores, double* expected, int32_t* k_best,
                        uint32_t* err, hipStream_t s);
hipError_t launch_bellman(const double* q, const double* cost, int N, int L, double* dp,
                          int32_t* k_best, uint32_t* err, hipStream_t s);
hipError_t launch_decode_fp8(const uint8_t* codes, float* out, long long count, hipStream_t s);

}  // namespace moe
