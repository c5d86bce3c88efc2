// Expert FFN of a verify pass as two kernels, deduplicating and per-slot
// (gfx950).  The deduplicating mode streams each union expert once and
// applies it to every slot routed to it; the per-slot mode reads an expert
// once per token-slot ("Speculative Decoding for Mixture-of-Experts Models:
// Expert Bytes, Kernel Bandwidth and the Best Draft Length", abstract;
// Table 5 and Table 6 name the engines' kernels of each kind).
//
// Both modes run the same two kernels over "groups": a group is one expert
// with the list of token rows it serves (dedup: a union expert and its slots,
// or a shared expert and all n tokens; per-slot: one slot, or one
// (token, shared expert) pair).  Kernel 1 (up) computes the f intermediate
// activations of every token of a group; kernel 2 (down) the d outputs.  The
// streaming core is in stream.h.
#include <map>
#include <mutex>

#include "stream.h"

namespace moe {

// one workgroup of NW wavefronts per CU (NW / 4 per SIMD)
template <int WT, int TC, int R, int NMAT, int SPC, int NW>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(NW / 4)))
void ffn_stream_kernel(FfnParams p) {
  static_assert(NW == kStreamWaves, "the streaming core runs kStreamThreads threads");
  constexpr bool UP = NMAT == 2;
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
  __shared__ int tok_h[2 * TC];
  __shared__ float* tok_y[2 * TC];
  __shared__ Meta mt;
  __shared__ int claim;
  __shared__ RangeTab rt;
  const int rows = UP ? p.f : p.d;
  const int upg = units_per_group(rows, R);

  if (!UP && blockIdx.x == 0 && threadIdx.x == 0 && p.bytes != nullptr) {
    const unsigned long long req =
        static_cast<unsigned long long>(p.n) * (p.K + p.S) * p.expert_bytes;
    unsigned long long got = req;
    if (p.mode == MODE_DEDUP) {
      const int U0 = *p.U;
      got = U0 < 0 ? 0ull : static_cast<unsigned long long>(U0 + p.S) * p.expert_bytes;
    }
    p.bytes[0] = got;
    p.bytes[1] = req;
  }

  int U = 0, NG;
  if (p.mode == MODE_DEDUP) {
    U = uni(*p.U);
    if (U < 0) {
      if (UP && blockIdx.x == 0 && threadIdx.x == 0) atomicOr(p.err, ERRBIT_BAD_IDS);
      return;
    }
    NG = U + p.S;
  } else {
    NG = p.n * (p.K + p.S);
  }
  const long long NU = static_cast<long long>(NG) * upg;
  const long long lo = NU * blockIdx.x / gridDim.x;
  const long long hi = NU * (blockIdx.x + 1) / gridDim.x;

  load_meta(p, mt);
  __syncthreads();
  if (!UP && p.mode == MODE_DEDUP) zero_unrouted_rows(p, mt, U);
  if (lo >= hi) return;
  run_range<WT, TC, R, NMAT, SPC, false>(p, mt, U, lo, hi, xs, tok_h, tok_y, rt, &claim, Sync{});
}

// ------------------------------------------------------------------ launch
struct OccKey {
  const void* fn;
  size_t smem;
  int block;
  int dev;
  bool operator<(const OccKey& o) const {
    if (fn != o.fn) return fn < o.fn;
    if (smem != o.smem) return smem < o.smem;
    if (block != o.block) return block < o.block;
    return dev < o.dev;
  }
};

size_t lds_budget(const void* fn) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, size_t> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> g(mu);
  const auto key = std::make_pair(fn, dev);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int lim = 0;
  hipFuncAttributes fa;
  if (hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
      hipFuncGetAttributes(&fa, fn) != hipSuccess || static_cast<size_t>(lim) <= fa.sharedSizeBytes)
    return 0;
  const size_t b = static_cast<size_t>(lim) - fa.sharedSizeBytes;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(b)) !=
      hipSuccess)
    return 0;
  cache[key] = b;
  return b;
}

// resident workgroups of a kernel on the whole device (cached per process)
int resident_blocks(const void* fn, size_t smem, int block) {
  static std::mutex mu;
  static std::map<OccKey, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> g(mu);
  const OccKey key{fn, smem, block, dev};
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, block, smem) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  const int total = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
  cache[key] = total;
  return total;
}

// CUs a launch on stream s may occupy: the population of the stream's CU
// mask (a stream created with one, or a process-wide mask), at most the
// device's CU count; the device's CU count when the query is refused
int stream_cus(hipStream_t s) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  uint32_t mask[32] = {};
  if (hipExtStreamGetCUMask(s, 32, mask) != hipSuccess) {
    (void)hipGetLastError();  // the refusal must not surface as the launch's error
    return cus;
  }
  int n = 0;
  for (int i = 0; i < cus && i < 32 * 32; ++i) n += static_cast<int>((mask[i / 32] >> (i % 32)) & 1u);
  return n > 0 ? n : cus;
}

template <int WT, int TC, int R, int NMAT, int SPC>
static hipError_t launch_phase(const FfnParams& p, hipStream_t s) {
  using C = StreamCfg<WT, TC, R, NMAT, SPC>;
  constexpr bool UP = NMAT == 2;
  constexpr int NW = kStreamWaves;
  constexpr int kStreamBlock = NW * kWave;
  const int rows = UP ? p.f : p.d;
  const int Kdim = UP ? p.d : p.f;
  const int Kpad = (Kdim + C::CH - 1) / C::CH * C::CH;
  const void* fn = reinterpret_cast<const void*>(&ffn_stream_kernel<WT, TC, R, NMAT, SPC, NW>);
  // One workgroup per CU: the launch takes all the LDS a workgroup may have.
  // A second token slot lets ranges that cross a group boundary take the
  // slot fast path; the matrix-core kernels stage whole ranges instead.
  const size_t slot = static_cast<size_t>(TC) * Kpad * C::T::XB;
  const size_t smem = lds_budget(fn);
  if (slot > smem) return hipErrorInvalidConfiguration;
  FfnParams q = p;
  q.lds_slots = 2 * slot <= smem ? 2 : 1;
  q.lds_bytes = static_cast<long long>(smem);
  const int upg = units_per_group(rows, R);
  const int groups_max = p.mode == MODE_DEDUP ? p.ucap + p.S : p.n * (p.K + p.S);
  const long long units_max = static_cast<long long>(groups_max) * upg;
  long long grid = resident_blocks(fn, smem, kStreamBlock);
  if (grid <= 0) return hipErrorInvalidConfiguration;
  if (grid > units_max) grid = units_max;
  hipLaunchKernelGGL((ffn_stream_kernel<WT, TC, R, NMAT, SPC, NW>), dim3(static_cast<unsigned>(grid)),
                     dim3(kStreamBlock), smem, s, q);
  return hipGetLastError();
}

template <int WT, int TC>
static hipError_t launch_pair(const FfnParams& p, hipStream_t s) {
  // up: R rows of W_gate and W_up per wave; down: R rows of W_down per wave
  using Tl = Tiles<WT, TC>;
  hipError_t e = launch_phase<WT, Tl::TCU, Tl::RU, 2, Tl::SPCU>(p, s);
  if (e != hipSuccess) return e;
  return launch_phase<WT, TC, Tl::RD, 1, Tl::SPCD>(p, s);
}

template <int WT>
static hipError_t launch_typed(const FfnParams& p, hipStream_t s) {
  switch (token_tile(p.mode, p.n)) {
    case 1: return launch_pair<WT, 1>(p, s);
    case 2: return launch_pair<WT, 2>(p, s);
    case 4: return launch_pair<WT, 4>(p, s);
    case 8: return launch_pair<WT, 8>(p, s);
    default:
      // f32 weights (dot products) stop at 8 tokens; larger groups take tiles
      if constexpr (WT == WT_F32) return launch_pair<WT, 8>(p, s);
      else return token_tile(p.mode, p.n) == 16 ? launch_pair<WT, 16>(p, s)
                                                : launch_pair<WT, 32>(p, s);
  }
}

hipError_t launch_expert_ffn(const FfnParams& p, int w_dtype, hipStream_t s) {
  switch (w_dtype) {
    case WT_F32: return launch_typed<WT_F32>(p, s);
    case WT_BF16: return launch_typed<WT_BF16>(p, s);
    case WT_FP8: return launch_typed<WT_FP8>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
