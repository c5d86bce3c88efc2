// One launch for one MoE layer of a verify pass (gfx950): route, union,
// expert FFN (deduplicating or per-slot) and combine.
//
// The pass is the expert operation of a speculative-decoding verification:
// top-K routing of every drafted token ("Making Every Verified Token Count:
// Adaptive Verification for MoE Speculative Decoding", Sec. 2.2, Eq. (4)),
// the union of the routed experts ("Less Experts, Faster Decoding", Sec. 3,
// Eq. (1)), the SwiGLU experts streamed once per union expert or once per
// token-slot ("Speculative Decoding for Mixture-of-Experts Models: Expert
// Bytes, Kernel Bandwidth and the Best Draft Length", abstract), and the
// gate-weighted combine (adaptive-verification page, Sec. 2.2).
//
// Why one launch: at draft sizes of 1-8 tokens the expert bytes of a pass
// take 15-70 us to stream, and every kernel boundary costs a drain, a launch
// and a ramp of a few microseconds.  Here every workgroup routes the pass
// itself (n*E logits from L2) and builds the union in LDS, so no kernel has
// to publish it; workgroup b then streams UP range b and DOWN range b of the
// balanced unit split, and the first workgroups combine.
//
// Exchange between workgroups (they run on all eight XCDs, whose L2 caches
// are not coherent with one another):
//   - H (f32) and the slot outputs are written with device-scope stores and
//     read with device-scope loads (stream.h), never through a cache-wide
//     writeback or invalidate;
//   - a workgroup publishes a finished range once its stores completed
//     (vmcnt(0) in every wave, then a barrier) by storing the call's tag in
//     its UP or DOWN flag; a DOWN group waits for the UP flags of the
//     workgroups that own its units, the combine for every DOWN flag;
//   - the tag is the workspace epoch + 1, read at the start; workgroup 0
//     advances the epoch after it has seen every DOWN flag (so every
//     workgroup has read it), which retires all flags of the call at once.
//     There are no read-modify-write atomics on shared words: contended
//     device-scope atomics serialise at the memory side.
// The grid is the kernel's resident capacity on the CUs the launch stream may
// use (its CU mask), so every workgroup runs at once while no other kernel
// holds CUs; each wait is bounded besides and records a time-out in the
// error word instead of hanging.
#include <algorithm>
#include <map>
#include <mutex>

#include "route.h"
#include "stream.h"

namespace moe {

// routing scratch, overlaid on the dynamic LDS before the stream uses it:
// the union builder's tables, the top-K scratch of each wavefront, then the
// pass's logits [n][E]
struct RouteLds {
  UnionLds ul;
  int slot_rank[kMaxSlots];
};
constexpr size_t kRouteTopkOffset = (sizeof(RouteLds) + 15) / 16 * 16;
constexpr size_t kRouteLogitsOffset = kRouteTopkOffset + kMaxStreamWaves * sizeof(TopkLds);
static_assert(sizeof(BudgetLds) <= kMaxStreamWaves * sizeof(TopkLds),
              "the budget tables reuse the top-K scratch");

// DOWN range [lo, hi) with the tile shapes of token tile TC
template <int WT, int TC>
__device__ __forceinline__ void run_down(const FfnParams& p, const Meta& mt, int U, long long lo,
                                         long long hi, uint8_t* xs, int* tok_h, float** tok_y,
                                         RangeTab& rt, int* claim, const Sync& sy) {
  using Tl = Tiles<WT, TC>;
  run_range<WT, TC, Tl::RD, 1, Tl::SPCD, true>(p, mt, U, lo, hi, xs, tok_h, tok_y, rt, claim, sy);
}

// UP range b, then DOWN range b, with the tile shapes of token tile TC (the
// two-kernel FFN's shapes for the same tile, so both run the same arithmetic;
// a unit's sums do not depend on the tile that holds its tokens, so a pass
// whose groups all fit a smaller DOWN tile runs that one, which keeps more
// weight bytes in flight)
template <int WT, int TC>
__device__ __forceinline__ void run_phases(const LayerParams& lp, const Meta& mt, int U, int NG,
                                           uint8_t* xs, int* tok_h, float** tok_y, RangeTab& rt,
                                           int* claim, int* cpre, int* cpre_d, unsigned tag,
                                           int limit) {
  using Tl = Tiles<WT, TC>;
  const FfnParams& p = lp.f;
  const int upg_u = units_per_group(p.f, Tl::RU);
  const int upg_d = units_per_group(p.d, Tl::RD);
  const long long NUu = static_cast<long long>(NG) * upg_u;
  const long long NUd = static_cast<long long>(NG) * upg_d;
  const int G = gridDim.x, b = blockIdx.x;
  Sync sy{lp.up_flags, tag, NUu, G, upg_u, p.err, limit, nullptr, 0};
  // a deduplicating pass of more tokens than the small tiles hold splits the
  // units by cost (stream.h, phase_costs); otherwise by count
  const bool weighted = TC >= 16 && mt.mode == MODE_DEDUP && NG <= kCostGroups;
  long long ctot_d = 0;
  int maxcnt = TC;
  if (weighted) {
    sy.ctot = phase_costs<Tl::TCU, true>(p, mt, U, NG, upg_u, cpre);
    sy.cpre = cpre;
    ctot_d = phase_costs<TC, false>(p, mt, U, NG, upg_d, cpre_d, cpre_d + kCostGroups + 1);
    maxcnt = cpre_d[kCostGroups + 1];
  }
  {
    long long lo = div_small(NUu * b, G), hi = div_small(NUu * (b + 1), G);
    if (sy.cpre != nullptr) {
      lo = weighted_first_unit(cpre, NG, upg_u, sy.ctot, G, b, NUu);
      hi = weighted_first_unit(cpre, NG, upg_u, sy.ctot, G, b + 1, NUu);
    }
    if (lo < hi)
      run_range<WT, Tl::TCU, Tl::RU, 2, Tl::SPCU, true>(p, mt, U, lo, hi, xs, tok_h, tok_y, rt,
                                                         claim, sy);
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_store(lp.up_flags + b, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  {
    long long lo = div_small(NUd * b, G), hi = div_small(NUd * (b + 1), G);
    if (weighted) {
      lo = weighted_first_unit(cpre_d, NG, upg_d, ctot_d, G, b, NUd);
      hi = weighted_first_unit(cpre_d, NG, upg_d, ctot_d, G, b + 1, NUd);
    }
    if (lo < hi) {
      static_assert(Tiles<WT, 8>::RD == Tl::RD && Tiles<WT, 16>::RD == Tl::RD,
                    "DOWN tiles of one pass share the unit size");
      if (TC >= 16 && maxcnt <= 8) {
        run_down<WT, (TC >= 16 ? 8 : TC)>(p, mt, U, lo, hi, xs, tok_h, tok_y, rt, claim, sy);
      } else if (TC >= 32 && maxcnt <= 16) {
        run_down<WT, (TC >= 32 ? 16 : TC)>(p, mt, U, lo, hi, xs, tok_h, tok_y, rt, claim, sy);
      } else {
        run_down<WT, TC>(p, mt, U, lo, hi, xs, tok_h, tok_y, rt, claim, sy);
      }
    }
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_store(lp.down_flags + b, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// one workgroup of NW wavefronts per CU (NW / 4 per SIMD).  AUTO: the mode is
// chosen per pass on the device; a per-slot pass then runs the per-slot tile
// (one token), so it reproduces moe_expert_ffn_perslot bit for bit.
template <int WT, int TC, int NW, bool AUTO>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(NW / 4)))
void layer_kernel(LayerParams lp) {
  constexpr int kWaves = NW, kStreamBlock = NW * kWave;
  static_assert(NW == kStreamWaves, "the streaming core runs kStreamThreads threads");
  constexpr int TCM = TC;
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
  __shared__ int tok_h[2 * TCM];
  __shared__ float* tok_y[2 * TCM];
  __shared__ Meta mt;
  __shared__ int ids_l[kMaxSlots];
  __shared__ float gates_l[kMaxSlots];
  __shared__ int U_l;
  __shared__ uint8_t drop_l[kMaxSlots / 8];  // expert budget: bit k of token t = slot dropped
  __shared__ int claim;  // next unit of the running phase (stream.h)
  __shared__ int cpre[kCostGroups + 1];    // weighted UP partition (stream.h)
  __shared__ int cpre_d[kCostGroups + 2];  // weighted DOWN partition, then the largest group
  __shared__ RangeTab rt;
  const FfnParams& p = lp.f;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = p.n, K = p.K, E = p.E, S = p.S, nk = n * K;

  // ---- route every token and build the union, in every workgroup; the
  // logits are copied to LDS first (one round trip to memory for all tokens)
  RouteLds& rl = *reinterpret_cast<RouteLds*>(xs);
  float* lg = reinterpret_cast<float*>(xs + kRouteLogitsOffset);
  // the call's tag (workspace epoch + 1) travels with the logits: it is final
  // before the launch (the previous call advanced it before it ended); every
  // wavefront loads it, so no wavefront's logits wait behind it
  __shared__ unsigned tag_l;
  __shared__ int limit_l;
  const unsigned tag_v = coh_load_u32(lp.epoch);  // one request per wavefront
  const unsigned spin_v = *lp.spin;
  {
    // touch every 64-byte line of the argument block now, so the scalar
    // loads of the streaming set-up hit the scalar cache instead of each
    // waiting about a microsecond on its first line
    const unsigned* kw = reinterpret_cast<const unsigned*>(&lp);
#pragma unroll
    for (int i = 0; i < static_cast<int>(sizeof(LayerParams) / 4); i += 16) {
      const unsigned v = kw[i];
      asm volatile("" ::"s"(v));
    }
  }
  {
    // eight loads per lane in flight at once (clamped in bounds), then the stores
    constexpr int kPer = 8;
    const int words = n * E;
    for (int base = 0; base < words; base += kStreamBlock * kPer) {
      float v[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) v[i] = lp.logits[min(base + i * kStreamBlock + tid, words - 1)];
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (base + i * kStreamBlock + tid < words) lg[base + i * kStreamBlock + tid] = v[i];
    }
  }
  if (tid == 0) {
    tag_l = tag_v + 1u;
    limit_l = spin_v != 0u && spin_v <= static_cast<unsigned>(kSpinLimit) ? static_cast<int>(spin_v)
                                                                           : kSpinLimit;
  }
  __syncthreads();
  TopkLds* tk = reinterpret_cast<TopkLds*>(xs + kRouteTopkOffset);
  // wavefronts per token: up to 64 experts a few tokens share their rank
  // counts among the idle wavefronts; more experts take K rounds of a
  // wavefront maximum per token (route_token), which needs no team
  const int team = E <= kWave && n <= kWaves / 2 ? kWaves / n : 1;
  if (team > 1) {
    // few tokens: the idle wavefronts share the rank counts
    const int t = wave / team, q = wave - t * team;
    if (t < n) route_team_count(lg + t * E, E, lane, q, team, tk[wave]);
    __syncthreads();
    if (t < n && q == 0) {
      int id;
      float g;
      route_team_select(lg + t * E, E, K, lane, tk + wave, team, id, g);
      if (lane < K) {
        ids_l[t * K + lane] = id;
        gates_l[t * K + lane] = g;
      }
    }
  } else {
    for (int t = wave; t < n; t += kWaves) {
      int id;
      float g;
      route_token(lg + t * E, E, K, lane, tk[wave], id, g);
      if (lane < K) {
        ids_l[t * K + lane] = id;
        gates_l[t * K + lane] = g;
      }
    }
  }
  __syncthreads();
  int U = 0;
  int mode = p.mode;
  if (mode != MODE_PERSLOT) {
    if (n == 1)  // one token: its top-K ids are distinct
      build_union_one_token(ids_l, K, E, &U_l, mt.b, mt.a, mt.c, rl.slot_rank);
    else
      build_union_256(ids_l, n, K, E, &U_l, mt.b, mt.a, mt.c, rl.slot_rank, rl.ul);
    __syncthreads();
    U = uni(U_l);
  }
  // expert budget (deduplicating mode): the union keeps the lp.budget experts
  // of largest gate mass; the top-K scratch is dead and holds its tables
  const bool budgeted = mode == MODE_DEDUP && lp.budget > 0 && U > lp.budget;  // uniform
  if (budgeted)
    U = uni(apply_budget(U, lp.budget, lp.renorm, n, K, p.ucap, mt.b, mt.a, mt.c, rl.slot_rank,
                         gates_l, *reinterpret_cast<BudgetLds*>(xs + kRouteTopkOffset)));
  if (tid < n) {
    unsigned m = 0;
    if (budgeted)
      for (int k = 0; k < K; ++k) m |= (rl.slot_rank[tid * K + k] < 0 ? 1u : 0u) << k;
    drop_l[tid] = static_cast<uint8_t>(m);
  }
  if (mode == MODE_AUTO) {
    // the expert-bytes page's Eq. (7): deduplicate iff its byte share
    // (U+S)/(n(K+S)) is below the measured bandwidth ratio r (every
    // workgroup decides alike: it saw the same U)
    mode = static_cast<float>(U + S) < lp.r_auto * static_cast<float>(n * (K + S)) ? MODE_DEDUP
                                                                                    : MODE_PERSLOT;
  }
  if (mode == MODE_PERSLOT)
    for (int i = tid; i < nk; i += kStreamBlock) mt.a[i] = ids_l[i];
  if (tid == 0) mt.mode = mode;
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int i = tid; i < nk; i += kStreamBlock) {
      if (lp.ids != nullptr) lp.ids[i] = ids_l[i];
      if (lp.gates != nullptr) lp.gates[i] = gates_l[i];
    }
    if (mode == MODE_DEDUP && lp.U != nullptr) {
      const int cap = p.ucap;
      for (int i = tid; i < nk; i += kStreamBlock) {
        lp.perm[i] = mt.c[i];
        lp.slot_rank[i] = rl.slot_rank[i];
      }
      for (int i = tid; i < cap; i += kStreamBlock) lp.union_ids[i] = mt.b[i];
      for (int i = tid; i <= cap; i += kStreamBlock) lp.offsets[i] = mt.a[i];
      if (tid == 0) *lp.U = U;
    }
    if (tid == 0 && p.bytes != nullptr) {
      const unsigned long long req =
          static_cast<unsigned long long>(n) * (K + S) * p.expert_bytes;
      p.bytes[0] = mode == MODE_DEDUP ? static_cast<unsigned long long>(U + S) * p.expert_bytes
                                        : req;
      p.bytes[1] = req;
    }
    if (tid == 0 && lp.mode_out != nullptr) *lp.mode_out = mode;
  }
  __syncthreads();  // the routing scratch in xs is dead from here

  // ---- UP range b, then DOWN range b
  const unsigned tag = tag_l;
  const int limit = limit_l;
  const int NG = mode == MODE_DEDUP ? U + S : n * (K + S);
  const int G = gridDim.x, b = blockIdx.x;
  if (AUTO && TC > 1 && mode == MODE_PERSLOT)
    run_phases<WT, 1>(lp, mt, U, NG, xs, tok_h, tok_y, rt, &claim, cpre, cpre_d, tag, limit);
  else
    run_phases<WT, TC>(lp, mt, U, NG, xs, tok_h, tok_y, rt, &claim, cpre, cpre_d, tag, limit);

  // ---- combine: one lane per (token, 4 columns), first workgroups only
  const int quads = p.d / 4;
  const int tasks = n * quads;
  if (b * kStreamBlock >= tasks) return;
  wait_flags(lp.down_flags, 0, G - 1, tag, p.err, limit);
  if (b == 0 && tid == 0)  // every workgroup has read the epoch: retire this call's flags
    __hip_atomic_store(lp.epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned ys_size = static_cast<unsigned>(static_cast<size_t>(nk) * p.d * 4);
  const unsigned sh_size = static_cast<unsigned>(static_cast<size_t>(n) * S * p.d * 4);
  for (int task = b * kStreamBlock + tid; task < tasks; task += G * kStreamBlock) {
    const int t = task / quads;
    const int c = (task - t * quads) * 4;
    // every load is issued unconditionally, so all are in flight at once:
    // slots k >= K read the next token's rows or, past the end of the
    // buffer, zeros (the buffer range check), and are not summed
    u32x4 yv[8], sv[4];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      yv[k] = coh_ld16(p.y_slots,
                       static_cast<unsigned>(((static_cast<size_t>(t) * K + k) * p.d + c) * 4),
                       ys_size);
    if (S > 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        sv[q] = coh_ld16(p.y_shared,
                         static_cast<unsigned>(((static_cast<size_t>(t) * S + q) * p.d + c) * 4),
                         sh_size);
    }
    // the order of moe_combine: k ascending, then the shared experts; a slot
    // an expert budget dropped adds nothing and gets a zero output row
    const unsigned dm = drop_l[t];
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k < K && ((dm >> k) & 1u) != 0u)
        st16(reinterpret_cast<uint8_t*>(p.y_slots) +
                 ((static_cast<size_t>(t) * K + k) * p.d + c) * 4,
             u32x4{0u, 0u, 0u, 0u});
      if (k < K && ((dm >> k) & 1u) == 0u) {
        const float g = gates_l[t * K + k];
        acc[0] = fmaf(g, __uint_as_float(yv[k].x), acc[0]);
        acc[1] = fmaf(g, __uint_as_float(yv[k].y), acc[1]);
        acc[2] = fmaf(g, __uint_as_float(yv[k].z), acc[2]);
        acc[3] = fmaf(g, __uint_as_float(yv[k].w), acc[3]);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q < S) {
        acc[0] += __uint_as_float(sv[q].x);
        acc[1] += __uint_as_float(sv[q].y);
        acc[2] += __uint_as_float(sv[q].z);
        acc[3] += __uint_as_float(sv[q].w);
      }
    }
    const size_t o = static_cast<size_t>(t) * p.d + c;
    if (lp.out_bf16) {
      uint2 pk;
      pk.x = f32_to_bf16_bits(acc[0]) | (static_cast<unsigned>(f32_to_bf16_bits(acc[1])) << 16);
      pk.y = f32_to_bf16_bits(acc[2]) | (static_cast<unsigned>(f32_to_bf16_bits(acc[3])) << 16);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(lp.out) + o) = pk;
    } else {
      f32x4 r;
      r.x = acc[0];
      r.y = acc[1];
      r.z = acc[2];
      r.w = acc[3];
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(lp.out) + o) = r;
    }
  }
}

// ------------------------------------------------------------------ launch
// LDS bytes of one token slot (the larger of the UP and DOWN phases) of tile TC
template <int WT, int TC>
static size_t slot_bytes(const FfnParams& p) {
  using Tl = Tiles<WT, TC>;
  using CU = StreamCfg<WT, Tl::TCU, Tl::RU, 2, Tl::SPCU>;
  using CD = StreamCfg<WT, TC, Tl::RD, 1, Tl::SPCD>;
  const size_t su = static_cast<size_t>(Tl::TCU) * ((p.d + CU::CH - 1) / CU::CH * CU::CH) * CU::T::XB;
  const size_t sd = static_cast<size_t>(TC) * ((p.f + CD::CH - 1) / CD::CH * CD::CH) * CD::T::XB;
  return su > sd ? su : sd;
}

template <int WT, int TC, bool AUTO>
static hipError_t launch_layer_t(const LayerParams& lp0, hipStream_t s) {
  constexpr int NW = kStreamWaves;
  constexpr int kStreamBlock = NW * kWave;
  const FfnParams& p = lp0.f;
  // the coherent buffer loads (coh_ld16) take 32-bit byte offsets: the
  // combine reads y_slots up to slot row n*K + 7 and y_shared up to row
  // n*S + 3, the DOWN staging H up to row n*(K+S) (+16 bytes); all must stay
  // below 2^31 (the num_records of H's resource)
  const unsigned long long kOffLimit = 0x7fffffffull;
  if ((static_cast<unsigned long long>(p.n) * p.K + 8) * p.d * 4 > kOffLimit ||
      (static_cast<unsigned long long>(p.n) * p.S + 4) * p.d * 4 > kOffLimit ||
      static_cast<unsigned long long>(p.n) * (p.K + p.S) * p.f * 4 + 32 > kOffLimit)
    return hipErrorInvalidValue;
  const void* fn = reinterpret_cast<const void*>(&layer_kernel<WT, TC, NW, AUTO>);
  size_t slot = slot_bytes<WT, TC>(p);
  if (AUTO) slot = std::max(slot, slot_bytes<WT, 1>(p));
  // one workgroup per CU: the launch takes all the LDS a workgroup may have
  const size_t floor_bytes = kRouteLogitsOffset + static_cast<size_t>(p.n) * p.E * 4;
  const size_t smem = lds_budget(fn);
  if (slot > smem || floor_bytes > smem) return hipErrorInvalidConfiguration;
  LayerParams lp = lp0;
  lp.f.lds_slots = 2 * slot <= smem ? 2 : 1;
  lp.f.lds_bytes = static_cast<long long>(smem);
  int grid = resident_blocks(fn, smem, kStreamBlock);
  if (grid <= 0) return hipErrorInvalidConfiguration;
  // the workgroups wait for one another, so the grid must fit the CUs this
  // stream may use: a stream restricted by a CU mask gets a smaller grid
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      cus > 0) {
    const int avail = stream_cus(s);
    if (avail > 0 && avail < cus) grid = grid / cus * avail;
  }
  if (grid <= 0) return hipErrorInvalidConfiguration;
  if (grid > kMaxGrid) grid = kMaxGrid;
  hipLaunchKernelGGL((layer_kernel<WT, TC, NW, AUTO>), dim3(grid), dim3(kStreamBlock), smem, s, lp);
  return hipGetLastError();
}

template <int WT, int TC>
static hipError_t launch_layer_tc(const LayerParams& lp, hipStream_t s) {
  return lp.f.mode == MODE_AUTO ? launch_layer_t<WT, TC, true>(lp, s)
                                : launch_layer_t<WT, TC, false>(lp, s);
}

template <int WT>
static hipError_t launch_layer_w(const LayerParams& lp, hipStream_t s) {
  switch (token_tile(lp.f.mode, lp.f.n)) {
    case 1: return launch_layer_tc<WT, 1>(lp, s);
    case 2: return launch_layer_tc<WT, 2>(lp, s);
    case 4: return launch_layer_tc<WT, 4>(lp, s);
    case 8: return launch_layer_tc<WT, 8>(lp, s);
    default:
      // f32 weights (dot products) stop at 8 tokens; larger groups take tiles
      if constexpr (WT == WT_F32) return launch_layer_tc<WT, 8>(lp, s);
      else return token_tile(lp.f.mode, lp.f.n) == 16 ? launch_layer_tc<WT, 16>(lp, s)
                                                      : launch_layer_tc<WT, 32>(lp, s);
  }
}

hipError_t launch_layer(const LayerParams& lp, int w_dtype, hipStream_t s) {
  switch (w_dtype) {
    case WT_F32: return launch_layer_w<WT_F32>(lp, s);
    case WT_BF16: return launch_layer_w<WT_BF16>(lp, s);
    case WT_FP8: return launch_layer_w<WT_FP8>(lp, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
