// Streaming core of the expert FFN kernels (gfx950): weight traits, dot
// products, the group walk, chunk loads and multiplies, token staging, unit
// epilogues and the per-range streaming loop.  Included by the two-kernel
// FFN (ffn.hip) and the one-launch layer pass (fused.hip).
//
// For every (expert, slot) pair: a = x W_gate, v = x W_up, h = silu(a) * v,
// y = h W_down ("Speculative Decoding for Mixture-of-Experts Models: Expert
// Bytes, Kernel Bandwidth and the Best Draft Length", abstract).  Work is a
// batched matrix-vector product with at most a handful of tokens per weight
// row, so it is bound by HBM bandwidth, not by matrix throughput.  Each
// wavefront owns R weight rows (stored one row per output, so the reduction
// runs along contiguous memory) and streams them with 16-byte loads, 64 lanes
// covering 1 KiB of a row per step; the group's tokens sit in LDS as bf16
// (f32 for f32 weights) and are reused by every row of the workgroup.
// Products use v_dot2_f32_bf16 (two bf16 MACs, fp32 accumulate); fp8 codes
// are widened to bf16 pairs exactly with v_cvt_scalef32_pk_bf16_fp8 and the
// 128x128 block scale is applied once per 16 codes.  Partial sums are
// combined across the wavefront by recursive halving (each shuffle stage
// halves the values per lane), so a wave reduces R*T values with about R*T
// shuffles instead of 6*R*T.
#pragma once

#include "common.h"
#include "partition.h"

namespace moe {

// ------------------------------------------------- coherent exchange
// Data handed between workgroups of one launch crosses XCDs, whose L2 caches
// are not coherent with each other.  Stores and loads with the device-scope
// bit (sc1) write through to, and read from, the coherent level, so only the
// exchanged words pay for coherence (no cache-wide writeback or invalidate).
__device__ __forceinline__ void coh_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned coh_load_u32(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes at base + off with a device-scope buffer load (bytes at or beyond
// `size` read as zero).  The raw buffer load takes a 32-bit byte offset and,
// with swizzling off and stride 0, returns zero for offset >= num_records
// without touching memory; the launcher checks that every offset the pass
// computes fits 31 bits.  The auxiliary operand of gfx940-family buffer
// instructions holds sc0 (bit 0), nt (bit 1), swz (bit 3) and sc1 (bit 4):
// bit 3 is not a cache policy but turns on swizzled addressing, under which
// the range check applies to the record index (0 for a raw load) rather than
// the byte offset, so an out-of-range offset would be dereferenced.
constexpr int kAuxSc1 = 16;  // cache-policy operand: sc1
constexpr int kAuxPolicyBits = 0x1 | 0x2 | 0x10;  // sc0, nt, sc1
static_assert((kAuxSc1 & ~kAuxPolicyBits) == 0, "aux operand: cache-policy bits only (no swz)");
__device__ __forceinline__ u32x4 coh_ld16(const void* base, unsigned off, unsigned size) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(base), static_cast<short>(0), static_cast<int>(size), 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, kAuxSc1);
}
// every store this wavefront issued has completed (is visible device-wide
// for sc1 stores) before anything after this point
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// f32 H words at byte offset off -> one 16-byte LDS vector of the staged type
template <int XB>
__device__ __forceinline__ u32x4 coh_h_to_staged(const uint8_t* H, size_t off) {
  const unsigned o = static_cast<unsigned>(off);
  if (XB == 4) return coh_ld16(H, o, 0x7fffffffu);
  const u32x4 a = coh_ld16(H, o, 0x7fffffffu), b = coh_ld16(H, o + 16, 0x7fffffffu);
  u32x4 r;
  r.x = f32_to_bf16_bits(__uint_as_float(a.x)) | (static_cast<unsigned>(f32_to_bf16_bits(__uint_as_float(a.y))) << 16);
  r.y = f32_to_bf16_bits(__uint_as_float(a.z)) | (static_cast<unsigned>(f32_to_bf16_bits(__uint_as_float(a.w))) << 16);
  r.z = f32_to_bf16_bits(__uint_as_float(b.x)) | (static_cast<unsigned>(f32_to_bf16_bits(__uint_as_float(b.y))) << 16);
  r.w = f32_to_bf16_bits(__uint_as_float(b.z)) | (static_cast<unsigned>(f32_to_bf16_bits(__uint_as_float(b.w))) << 16);
  return r;
}

// Hand-over inside one launch: workgroup c publishes the end of its UP range
// by storing the call's tag in up_flags[c].  The tag is one more than the
// epoch word the launch read at its start, so flags of earlier calls never
// match and nothing has to be reset.
struct Sync {
  const unsigned* up_flags;
  unsigned tag;
  long long nu_up;  // UP units of the pass
  int grid;         // workgroups (UP range c = [nu_up*c/grid, nu_up*(c+1)/grid))
  int upg_up;       // UP units per group
  uint32_t* err;
  int limit;        // polls before a wait gives up
  const int* cpre;  // weighted UP partition (phase_costs), or nullptr
  long long ctot;   // its total cost
};

// every lane polls its share of the flags until they hold the tag (bounded:
// a wait that gives up after `limit` polls records a time-out in the error
// word and goes on)
__device__ __forceinline__ void wait_flags(const unsigned* flags, int c_lo, int c_hi, unsigned tag,
                                           uint32_t* err, int limit) {
  for (int c = c_lo + static_cast<int>(threadIdx.x); c <= c_hi; c += kStreamThreads) {
    int spins = 0;
    while (coh_load_u32(flags + c) != tag) {
      if (++spins > limit) {
        atomicOr(err, ERRBIT_TIMEOUT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

// DOWN of group g may start once the workgroups owning g's UP units are done
__device__ __forceinline__ void wait_group_ready(const Sync& sy, int g) {
  int c_lo, c_hi;
  group_owners(sy.cpre, sy.ctot, sy.nu_up, sy.grid, sy.upg_up, g, c_lo, c_hi);
  wait_flags(sy.up_flags, c_lo, c_hi, sy.tag, sy.err, sy.limit);
}

template <int WT>
struct WTraits;
// VEC: weight elements per 16-byte load; SPC: load steps per staged chunk;
// EB: bytes per weight element; XB: bytes per staged token element.
template <>
struct WTraits<WT_F32> {
  static constexpr int VEC = 4, SPC = 4, EB = 4, XB = 4;
};
template <>
struct WTraits<WT_BF16> {
  static constexpr int VEC = 8, SPC = 4, EB = 2, XB = 2;
};
template <>
struct WTraits<WT_FP8> {
  static constexpr int VEC = 16, SPC = 2, EB = 1, XB = 2;
};

// ------------------------------------------------------------ dot products
// acc += <16 bytes of weights, VEC token elements in LDS>
template <int WT>
struct Dot;

template <>
struct Dot<WT_F32> {
  struct W {
    u32x4 v;
  };
  static __device__ __forceinline__ W prep(u32x4 v) { return W{v}; }
  static __device__ __forceinline__ float run(const W& w, const uint8_t* xs, float acc, float) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(xs);
    acc = fmaf(__uint_as_float(w.v.x), x.x, acc);
    acc = fmaf(__uint_as_float(w.v.y), x.y, acc);
    acc = fmaf(__uint_as_float(w.v.z), x.z, acc);
    acc = fmaf(__uint_as_float(w.v.w), x.w, acc);
    return acc;
  }
};

template <>
struct Dot<WT_BF16> {
  struct W {
    u32x4 v;
  };
  static __device__ __forceinline__ W prep(u32x4 v) { return W{v}; }
  static __device__ __forceinline__ float run(const W& w, const uint8_t* xs, float acc, float) {
    const u32x4 x = ld16(xs);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.v.x), as_bf16x2(x.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.v.y), as_bf16x2(x.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.v.z), as_bf16x2(x.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w.v.w), as_bf16x2(x.w), acc, false);
    return acc;
  }
};

template <>
struct Dot<WT_FP8> {
  struct W {
    bf16x2 p[8];
  };
  static __device__ __forceinline__ W prep(u32x4 v) {
    W w;
    w.p[0] = fp8x2_to_bf16x2<false>(v.x);
    w.p[1] = fp8x2_to_bf16x2<true>(v.x);
    w.p[2] = fp8x2_to_bf16x2<false>(v.y);
    w.p[3] = fp8x2_to_bf16x2<true>(v.y);
    w.p[4] = fp8x2_to_bf16x2<false>(v.z);
    w.p[5] = fp8x2_to_bf16x2<true>(v.z);
    w.p[6] = fp8x2_to_bf16x2<false>(v.w);
    w.p[7] = fp8x2_to_bf16x2<true>(v.w);
    return w;
  }
  // the 16 codes of one load lie in one 128-wide block: one scale
  static __device__ __forceinline__ float run(const W& w, const uint8_t* xs, float acc,
                                              float scale) {
    const u32x4 x0 = ld16(xs), x1 = ld16(xs + 16);
    float t = 0.0f;
    t = __builtin_amdgcn_fdot2_f32_bf16(w.p[0], as_bf16x2(x0.x), t, false);
    t = __builtin_amdgcn_fdot2_f32_bf16(w.p[1], as_bf16x2(x0.y), t, false);
    t = __builtin_amdgcn_fdot2_f32_bf16(w.p[2], as_bf16x2(x0.z), t, false);
    t = __builtin_amdgcn_fdot2_f32_bf16(w.p[3], as_bf16x2(x0.w), t, false);
    t = __builtin_amdgcn_fdot2_f32_bf16(w.p[4], as_bf16x2(x1.x), t, false);
    t = __builtin_amdgcn_fdot2_f32_bf16(w.p[5], as_bf16x2(x1.y), t, false);
    t = __builtin_amdgcn_fdot2_f32_bf16(w.p[6], as_bf16x2(x1.z), t, false);
    t = __builtin_amdgcn_fdot2_f32_bf16(w.p[7], as_bf16x2(x1.w), t, false);
    return fmaf(scale, t, acc);
  }
};

// --------------------------------------------------- wavefront reduction
// Recursive halving: N partial sums per lane -> every lane holds the total
// of value index (lane >> (6 - log2 N)).
template <int N>
struct Halve {
  static __device__ __forceinline__ void run(float* v, int lane, int o) {
    const bool upper = (lane & o) != 0;
#pragma unroll
    for (int k = 0; k < N / 2; ++k) {
      const float send = upper ? v[k] : v[k + N / 2];
      const float keep = upper ? v[k + N / 2] : v[k];
      v[k] = keep + __shfl_xor(send, o);
    }
    Halve<N / 2>::run(v, lane, o >> 1);
  }
};
template <>
struct Halve<1> {
  static __device__ __forceinline__ void run(float* v, int, int o) {
    for (; o >= 1; o >>= 1) v[0] += __shfl_xor(v[0], o);
  }
};

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

// ------------------------------------------------------------------ groups
struct Group {
  int e;       // expert index (routed or shared)
  int shared;  // 1 for a shared expert
  int cnt;     // tokens served
  int first;   // dedup routed: offset into perm; per-slot: slot or shared pair index
  int s_idx;   // shared expert index (dedup) or (token * S + s) pair (per-slot)
};

// ------------------------------------------------------ routing metadata
// The union arrays (dedup) or the slot ids (per-slot) are copied to LDS once
// per workgroup before the stream starts: loads issued later would complete
// in order behind the weight prefetch, so reading them from global memory in
// the loop would drain the prefetch every time.
constexpr int kMaxSlots = 256;  // n*K <= 32*8
struct Meta {
  int a[kMaxSlots + 1];  // dedup: offsets[0..cap]; per-slot: ids[0..nK)
  int b[kMaxSlots];      // dedup: union_ids[0..cap)
  int c[kMaxSlots];      // dedup: perm[0..nK)
  int mode;              // MODE_DEDUP or MODE_PERSLOT: how a, b, c are read
};

__device__ __forceinline__ void load_meta(const FfnParams& p, Meta& m) {
  const int nk = p.n * p.K;
  if (threadIdx.x == 0) m.mode = p.mode;
  if (p.mode == MODE_DEDUP) {
    for (int i = threadIdx.x; i <= p.ucap; i += kStreamThreads) m.a[i] = p.offsets[i];
    for (int i = threadIdx.x; i < p.ucap; i += kStreamThreads) m.b[i] = p.union_ids[i];
    for (int i = threadIdx.x; i < nk; i += kStreamThreads) m.c[i] = p.perm[i];
  } else {
    for (int i = threadIdx.x; i < nk; i += kStreamThreads) m.a[i] = p.ids[i];
  }
}

// Deduplicating mode: the slots after offsets[U] in perm (dropped by an
// expert budget) belong to no group; their output rows are zero.  Spread over
// the whole grid; nothing to do for a plain union (offsets[U] = n*K).
__device__ __forceinline__ void zero_unrouted_rows(const FfnParams& p, const Meta& mt, int U) {
  const int nk = p.n * p.K, first = mt.a[U];
  const long long total = static_cast<long long>(nk - first) * p.d;
  for (long long i = static_cast<long long>(blockIdx.x) * kStreamThreads + threadIdx.x; i < total;
       i += static_cast<long long>(gridDim.x) * kStreamThreads) {
    const long long r = i / p.d;
    p.y_slots[static_cast<size_t>(mt.c[first + r]) * p.d + (i - r * p.d)] = 0.0f;
  }
}

// Weighted partition of the one-launch pass.  A unit of a group of many
// tokens can cost more than its bytes:
//   - UP: a group of more tokens than the UP tile takes the general path,
//     which streams the group's rows once per token tile, at about 2.3 times
//     a one-tile unit's time for two tiles (measured on 32-node draft trees);
//     one-tile units cost the same whatever their tokens (two 4-token groups
//     of matrix-core work hide under the loads);
//   - DOWN: every four tokens of the tile add matrix-core and scaling work
//     per weight byte, about a fifth of a one-token unit's time each.
// For a deduplicating pass of more tokens than the small tiles hold, a unit
// of group g costs w_g (UP: 8 for one tile, 9 per tile beyond; DOWN:
// 3 + ceil(tokens / 4)), and workgroup c owns the units u with
// floor(P(u) * G / ctot) = c, P(u) the cost of the units before u: equal
// shares of the work, not of the bytes.  cpre[g] = cost of the units of
// groups before g (g = 0..NG), built by wavefront 0; returns ctot.
static_assert(kCostGroups >= kMaxSlots + 4, "cost tables hold U + S groups");
// (and *maxcnt = the largest group's token count, when maxcnt is set)
template <int TCP, bool UP>
__device__ __forceinline__ long long phase_costs(const FfnParams& p, const Meta& mt, int U, int NG,
                                                 int upg, int* cpre, int* maxcnt = nullptr) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int carry = 0, mc = 0;
    if (lane == 0) cpre[0] = 0;
    for (int base = 0; base < NG; base += kWave) {
      const int g = base + lane;
      int w = 0;
      if (g < NG) {
        const int cnt = g < U ? mt.a[g + 1] - mt.a[g] : p.n;
        mc = cnt > mc ? cnt : mc;
        w = unit_cost(cnt, TCP, UP) * upg;
      }
      // inclusive scan across the wavefront
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(w, o);
        if (lane >= o) w += v;
      }
      if (g < NG) cpre[g + 1] = carry + w;
      carry += __shfl(w, kWave - 1);
    }
    if (maxcnt != nullptr) {
#pragma unroll
      for (int o = kWave / 2; o > 0; o >>= 1) {
        const int v = __shfl_xor(mc, o);
        mc = v > mc ? v : mc;
      }
      if (lane == 0) *maxcnt = mc;
    }
  }
  __syncthreads();
  return cpre[NG];
}

// token j of a group: its row in x, its row in H and its output row
__device__ __forceinline__ void token_of(const FfnParams& p, const Meta& mt, const Group& G, int j,
                                         int& xrow, int& hrow, float*& yrow) {
  const int nk = p.n * p.K;
  if (mt.mode == MODE_DEDUP) {
    if (!G.shared) {
      const int slot = mt.c[G.first + j];
      xrow = slot / p.K;
      hrow = G.first + j;
      yrow = p.y_slots + static_cast<size_t>(slot) * p.d;
    } else {
      xrow = j;
      hrow = nk + G.s_idx * p.n + j;
      yrow = p.y_shared + (static_cast<size_t>(j) * p.S + G.s_idx) * p.d;
    }
  } else {
    if (!G.shared) {
      xrow = G.first / p.K;
      hrow = G.first;
      yrow = p.y_slots + static_cast<size_t>(G.first) * p.d;
    } else {
      xrow = G.s_idx / p.S;
      hrow = nk + G.s_idx;
      yrow = p.y_shared + static_cast<size_t>(G.s_idx) * p.d;
    }
  }
}

// a value every lane holds the same, kept in a scalar register
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// ------------------------------------------------------------ the walk
// One phase (up: gate/up rows, or down rows) is a list of units: (group g,
// block of R rows), groups in order, row blocks in order.  Workgroup b owns
// the contiguous unit range [b*NU/G, (b+1)*NU/G), so every workgroup streams
// the same bytes to within one unit of R rows (a unit per wavefront, not per
// workgroup: coarser units left workgroups with one or two of them, and the
// ones with two set the phase's time); passes with groups of many tokens
// split by cost instead (phase_costs).  On the general path, inside a group
// segment of the range the wavefronts take consecutive units, one unit each
// per step; the walk goes chunk by chunk (K split in chunks of SPC load
// steps): for each group segment, for each token tile of that group, for
// each step, for each chunk.  The walk is the same for every lane of the
// workgroup.

// units (blocks of R rows) of one group
__host__ __device__ constexpr int units_per_group(int rows, int R) { return (rows + R - 1) / R; }

struct Walk {
  int g, tile, s, kc, done;
  int ntile, ua, ub, nsteps;  // the segment's units [ua, ub) of group g, in steps of four
  int valid;                  // expert id in range
  Group G;
};

// group g of a phase: dedup 0..U-1 routed union experts, then the S shared;
// per-slot 0..n*K-1 slots, then the n*S (token, shared expert) pairs
__device__ __forceinline__ void group_at(const FfnParams& p, const Meta& mt, int U, int g,
                                         Group& G) {
  if (uni(mt.mode) == MODE_DEDUP) {
    if (g < U) {
      G.e = mt.b[g];
      G.shared = 0;
      G.first = mt.a[g];
      G.cnt = mt.a[g + 1] - G.first;
      G.s_idx = 0;
    } else {
      G.e = g - U;
      G.shared = 1;
      G.first = 0;
      G.cnt = p.n;
      G.s_idx = g - U;
    }
    return;
  }
  const int nk = p.n * p.K;
  if (g < nk) {
    G.e = mt.a[g];
    G.shared = 0;
    G.first = g;
    G.cnt = 1;
    G.s_idx = 0;
  } else {
    const int q = g - nk;
    G.e = q % p.S;
    G.shared = 1;
    G.first = q;
    G.cnt = 1;
    G.s_idx = q;
  }
}


template <int TC>
__device__ __forceinline__ void walk_group(const FfnParams& p, const Meta& mt, int U, Walk& w,
                                           int g, long long lo, long long hi, int upg) {
  // every field is the same in all lanes: keep the walk in scalar registers
  w.g = uni(g);
  group_at(p, mt, U, w.g, w.G);
  w.G.e = uni(w.G.e);
  w.G.shared = uni(w.G.shared);
  w.G.cnt = uni(w.G.cnt);
  w.G.first = uni(w.G.first);
  w.G.s_idx = uni(w.G.s_idx);
  w.valid = w.G.shared || (w.G.e >= 0 && w.G.e < p.E);
  w.ntile = (w.G.cnt + TC - 1) / TC;
  w.tile = 0;
  const long long glo = static_cast<long long>(g) * upg;
  w.ua = uni(static_cast<int>((lo > glo ? lo : glo) - glo));
  w.ub = uni(static_cast<int>((hi < glo + upg ? hi : glo + upg) - glo));
  const int nw = kStreamWaves;
  w.nsteps = (w.ub - w.ua + nw - 1) / nw;
  w.s = 0;
  w.kc = 0;
}

template <int TC>
__device__ __forceinline__ void walk_next(const FfnParams& p, const Meta& mt, int U, Walk& w,
                                          int nchunks, long long lo, long long hi, int upg) {
  if (++w.kc < nchunks) return;
  w.kc = 0;
  if (++w.s < w.nsteps) return;
  if (++w.tile < w.ntile) {
    w.s = 0;
    return;
  }
  if (static_cast<long long>(w.g + 1) * upg >= hi) {
    w.done = 1;
    return;
  }
  walk_group<TC>(p, mt, U, w, w.g + 1, lo, hi, upg);
}

// the unit a wavefront streams in step s of a segment [ua, ub): its first
// row r0 (relative to the group) and its valid rows rv (0 beyond the segment)
template <int R>
__device__ __forceinline__ void wave_unit(int ua, int ub, int s, int wave, int rows, int& r0,
                                          int& rv) {
  const int unit = ua + s * kStreamWaves + wave;
  r0 = unit * R;
  rv = unit < ub ? min(R, rows - r0) : 0;
}

// ------------------------------------------------------- streaming kernel
// UP (NMAT = 2): rows j of W_gate and W_up (Kdim = d) -> H[token][j] = silu(a) * v.
// DOWN (NMAT = 1): rows c of W_down (Kdim = f, tokens read from H) -> y[slot][c].
// Each wave owns R rows of the current unit; the weights of the next chunk
// are in flight while the current chunk is multiplied (two register buffers).
// Matrix cores for tiles of four or more tokens (bf16 and fp8 weights): the
// dot-product path spends about 8*TC VALU operations per 16 weight bytes,
// which at eight tokens approaches the memory time; one 4x4x4 MFMA block
// product covers four rows, four tokens and four K elements per lane.
constexpr bool use_mfma(int WT, int TC, int R) { return WT != WT_F32 && TC >= 4 && R == 4; }

// Tile shapes shared by the two-kernel FFN and the one-launch pass (both must
// run the same arithmetic): rows per wavefront R and load steps per chunk SPC
// of the UP and DOWN phases, and the UP token tile: at most 16 tokens (the
// gate and up accumulators of 32 would not fit 168 VGPRs), 8 for fp8 (d =
// 7168: 112 KB of LDS).  The matrix-core path takes four rows and keeps the
// bytes per chunk of the dot-product path.
template <int WT, int TC>
struct Tiles {
  static constexpr int TCU = (WT == WT_FP8 && TC > 8) ? 8 : (TC > 16 ? 16 : TC);
  static constexpr int RU0 = WT == WT_FP8 ? 4 : kRowsUp;
  static constexpr int SPCU0 = WT == WT_FP8 ? 1 : kStepsUp;
  static constexpr int RD0 = kRowsDown;
  // fp8 DOWN: two load steps per chunk, the UP phase's bytes in flight per
  // wavefront (one step left the DOWN phase ~18% below the UP phase's
  // bandwidth); the 32-token tile keeps one (its accumulators need the room)
  static constexpr int SPCD0 = WT == WT_FP8 ? (TC >= 32 ? 1 : 2) : kStepsDown;
  static constexpr bool MFU = use_mfma(WT, TCU, 4), MFD = use_mfma(WT, TC, 4);
  static constexpr int RU = MFU ? 4 : RU0;
  static constexpr int SPCU = MFU ? SPCU0 * RU0 : SPCU0;
  static constexpr int RD = MFD ? 4 : RD0;
  static constexpr int SPCD = MFD ? SPCD0 * RD0 : SPCD0;
};

template <int WT, int TC, int R, int NMAT, int SPC>
struct StreamCfg {
  using T = WTraits<WT>;
  // MF: the products run on the matrix cores (4x4x4 bf16 blocks, see
  // mul_chunk_mf); one load per matrix and step then covers the R = 4 rows.
  static constexpr bool MF = use_mfma(WT, TC, R);
  static constexpr int LR = MF ? 1 : R;                            // loads per matrix and step
  static constexpr int STEP = MF ? kWave * T::VEC / 4 : kWave * T::VEC;  // elements of a row per step
  static constexpr int CH = SPC * STEP;        // elements per chunk
  static constexpr int V = NMAT * R * TC;      // partial sums per lane (dot products)
  static constexpr int NACC = MF ? NMAT * TC : V;  // accumulators per lane
  static constexpr int SH = 6 - ilog2(V);
  static_assert(MF || ((V & (V - 1)) == 0 && V <= 64), "values per lane must be a power of two <= 64");
  static_assert(MF || NMAT == 1 || V >= 2, "gate/up pairing needs two values");
  static_assert(!MF || (R == 4 && TC % 4 == 0), "matrix-core path: four rows, tokens in fours");
};

// matrix MI's base pointer (0 gate, 1 up, 2 down), routed or shared; the
// fields are read with constant indices so the argument block stays in
// scalar registers (a selected address would force a copy to scratch)
template <int MI>
__device__ __forceinline__ const uint8_t* wptr(const FfnParams& p, int shared) {
  const uint8_t* a = p.w[MI];
  const uint8_t* b = p.shw[MI];
  return shared ? b : a;
}
template <int MI>
__device__ __forceinline__ const float* sptr(const FfnParams& p, int shared) {
  const float* a = p.s[MI];
  const float* b = p.shs[MI];
  return shared ? b : a;
}

template <int WT, int TC, int R, int NMAT, int SPC>
__device__ __forceinline__ void load_chunk(
    const FfnParams& p, const Group& G, int r0, int rv, int kc, int rows, int Kdim, int lane,
    u32x4 (&buf)[NMAT][SPC][StreamCfg<WT, TC, R, NMAT, SPC>::LR], float (&sc)[NMAT][SPC]) {
  using C = StreamCfg<WT, TC, R, NMAT, SPC>;
  using T = typename C::T;
  if constexpr (C::MF) {
    // lane 4b + i reads row r0 + i at K offset b * VEC of the step: a load
    // covers four rows of STEP elements (16 lanes per row, contiguous), the
    // A operand layout of the 4x4x4 block products
    const int i = lane & 3, b = lane >> 2;
    const size_t row_bytes = static_cast<size_t>(Kdim) * T::EB;
    const size_t mat = static_cast<size_t>(rows) * row_bytes;
    const int kb = Kdim / 128;
    const int e = rv > 0 ? G.e : 0;
    const bool rok = i < rv;
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      const uint8_t* base = (NMAT == 1 ? wptr<2>(p, G.shared)
                                       : (m == 0 ? wptr<0>(p, G.shared) : wptr<1>(p, G.shared))) +
                            static_cast<size_t>(e) * mat +
                            static_cast<size_t>(rok ? r0 + i : 0) * row_bytes;
      const float* sbase = nullptr;
      if (WT == WT_FP8)
        sbase = (NMAT == 1 ? sptr<2>(p, G.shared)
                           : (m == 0 ? sptr<0>(p, G.shared) : sptr<1>(p, G.shared))) +
                (static_cast<size_t>(e) * (rows / 128) + (rv > 0 ? r0 / 128 : 0)) * kb;
#pragma unroll
      for (int s = 0; s < SPC; ++s) {
        const int k = kc * C::CH + s * C::STEP + b * T::VEC;
        const bool ok = rok && k < Kdim;
        const uint8_t* a = ok ? base + static_cast<size_t>(k) * T::EB : p.zeros;
        buf[m][s][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a));
        if (WT == WT_FP8)
          sc[m][s] = *(ok ? sbase + (k >> 7) : reinterpret_cast<const float*>(p.zeros));
      }
    }
    return;
  }
  // Every lane issues every load, outside any branch, and nothing inspects the
  // loaded value before the multiply, so the next chunk stays in flight while
  // the current one is used.  Masked lanes read 16 zero bytes of the
  // workspace's control block instead of weights.  rv = 0 masks the whole
  // unit (beyond the range, or an expert id out of range).
  const size_t row_bytes = static_cast<size_t>(Kdim) * T::EB;
  const size_t mat = static_cast<size_t>(rows) * row_bytes;
  const int kb = Kdim / 128;
  const int e = rv > 0 ? G.e : 0;
#pragma unroll
  for (int m = 0; m < NMAT; ++m) {
    const uint8_t* base = (NMAT == 1 ? wptr<2>(p, G.shared)
                                     : (m == 0 ? wptr<0>(p, G.shared) : wptr<1>(p, G.shared))) +
                          static_cast<size_t>(e) * mat + static_cast<size_t>(r0) * row_bytes;
    const float* sbase = nullptr;
    if (WT == WT_FP8)
      sbase = (NMAT == 1 ? sptr<2>(p, G.shared)
                         : (m == 0 ? sptr<0>(p, G.shared) : sptr<1>(p, G.shared))) +
              (static_cast<size_t>(e) * (rows / 128) + (rv > 0 ? r0 / 128 : 0)) * kb;
#pragma unroll
    for (int s = 0; s < SPC; ++s) {
      const int k = kc * C::CH + s * C::STEP + lane * T::VEC;
      const bool kin = k < Kdim;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const bool ok = kin && r < rv;
        const uint8_t* a = ok ? base + static_cast<size_t>(r) * row_bytes +
                                    static_cast<size_t>(k) * T::EB
                              : p.zeros;
        // streamed once: non-temporal, so the weights do not evict tokens,
        // H and routing data from the caches (measured: +13% bandwidth)
        buf[m][s][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a));
      }
      if (WT == WT_FP8) {
        const bool ok = kin && rv > 0;
        sc[m][s] = *(ok ? sbase + (k >> 7) : reinterpret_cast<const float*>(p.zeros));
      }
    }
  }
}

// Matrix-core chunk loads from a unit's precomputed bases: wrow[m] = the
// unit's first row of matrix m, sblk[m] = the scales of its 128-row block
// (the per-chunk address math then stays 32-bit)
template <int WT, int TC, int R, int NMAT, int SPC>
__device__ __forceinline__ void load_chunk_mf(const uint8_t* const (&wrow)[NMAT],
                                              const float* const (&sblk)[NMAT], unsigned row_bytes,
                                              int rv, int kc, int Kdim, int lane,
                                              const uint8_t* zeros, u32x4 (&buf)[NMAT][SPC][1],
                                              float (&sc)[NMAT][SPC]) {
  using C = StreamCfg<WT, TC, R, NMAT, SPC>;
  using T = typename C::T;
  const int i = lane & 3, b = lane >> 2;
  const bool rok = i < rv;
  const unsigned roff = static_cast<unsigned>(i) * row_bytes;
#pragma unroll
  for (int m = 0; m < NMAT; ++m) {
#pragma unroll
    for (int s = 0; s < SPC; ++s) {
      const int k = kc * C::CH + s * C::STEP + b * T::VEC;
      const bool ok = rok && k < Kdim;
      const uint8_t* a = ok ? wrow[m] + (roff + static_cast<unsigned>(k) * T::EB) : zeros;
      buf[m][s][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a));
      if (WT == WT_FP8)
        sc[m][s] = *(ok ? sblk[m] + (k >> 7) : reinterpret_cast<const float*>(zeros));
    }
  }
}

template <int WT, int TC, int R, int NMAT, int SPC, int NT>
__device__ __forceinline__ void mul_chunk_nt(int kc, int Kpad, int lane, const uint8_t* xs,
                                             const u32x4 (&buf)[NMAT][SPC][StreamCfg<WT, TC, R, NMAT, SPC>::LR],
                                             const float (&sc)[NMAT][SPC], float* acc) {
  using C = StreamCfg<WT, TC, R, NMAT, SPC>;
  using T = typename C::T;
#pragma unroll
  for (int s = 0; s < SPC; ++s) {
    const int k = kc * C::CH + s * C::STEP + lane * T::VEC;
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const typename Dot<WT>::W wt = Dot<WT>::prep(buf[m][s][r]);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          float& a = acc[(m * R + r) * TC + tt];
          a = Dot<WT>::run(wt, xs + (static_cast<size_t>(tt) * Kpad + k) * T::XB, a,
                           WT == WT_FP8 ? sc[m][s] : 0.0f);
        }
      }
    }
  }
}

// tokens of (group, tile) -> LDS [TC][Kpad], zero beyond Kdim and beyond the
// tile; the H row and output row of every token go to LDS too, so the
// epilogue issues no global loads
template <int WT, int TC, bool FROM_H, bool COH>
__device__ __forceinline__ void stage_tokens(const FfnParams& p, const Meta& mt, const Walk& w,
                                             int Kdim, int Kpad, uint8_t* xs, int* tok_h,
                                             float** tok_y) {
  using T = WTraits<WT>;
  constexpr int EPV = 16 / T::XB;  // elements per 16-byte vector
  const int vpt = Kpad / EPV;
  const int nt = min(TC, w.G.cnt - w.tile * TC);
  if (threadIdx.x < TC) {
    int xrow = 0, hrow = 0;
    float* yrow = nullptr;
    if (static_cast<int>(threadIdx.x) < nt) token_of(p, mt, w.G, w.tile * TC + threadIdx.x, xrow, hrow, yrow);
    tok_h[threadIdx.x] = hrow;
    tok_y[threadIdx.x] = yrow;
  }
  // vector v of the slot: token v / vpt, elements from (v % vpt) * EPV
  auto fetch = [&](int v) {
    const int tt = v / vpt;
    const int k = (v - tt * vpt) * EPV;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (tt < nt && k < Kdim) {
      int xrow, hrow;
      float* yrow;
      token_of(p, mt, w.G, w.tile * TC + tt, xrow, hrow, yrow);
      if (FROM_H && COH) {
        // H holds f32 written by other workgroups: read it coherently and
        // round to the staged type here
        const size_t off = (static_cast<size_t>(hrow) * Kdim + k) * 4;
        val = coh_h_to_staged<T::XB>(p.H, off);
      } else {
        const uint8_t* src = FROM_H ? p.H + static_cast<size_t>(hrow) * Kdim * T::XB
                                    : p.x + static_cast<size_t>(xrow) * Kdim * T::XB;
        val = ld16(src + static_cast<size_t>(k) * T::XB);
      }
    }
    return val;
  };
  const int nv = TC * vpt, step = kStreamThreads;
  int v = threadIdx.x;
  for (; v + step < nv; v += 2 * step) {  // two loads in flight before the stores
    const u32x4 a = fetch(v), b = fetch(v + step);
    st16(xs + static_cast<size_t>(v) * 16, a);
    st16(xs + static_cast<size_t>(v + step) * 16, b);
  }
  if (v < nv) st16(xs + static_cast<size_t>(v) * 16, fetch(v));
}

// End of a unit whose tile holds at most NT of its TC tokens (the partial
// sums of tokens NT..TC-1 are zero): the NMAT*R*NT sums of the lane are
// compacted and reduced across the wavefront; the gate value of (row, token)
// ends in lane l and the up value in lane l ^ 32.
template <int WT, int TC, int R, int NMAT, int SPC, bool COH, int NT>
__device__ __forceinline__ void finish_unit(const FfnParams& p, int nt, int r0, int rv, int rows,
                                            int lane, const int* tok_h, float* const* tok_y,
                                            float* acc, float* yb = nullptr, int ystride = 0) {
  constexpr int V = NMAT * R * NT;
  constexpr int SH = 6 - ilog2(V);
  static_assert(NT <= TC && (V & (V - 1)) == 0 && V <= 64 && (NMAT == 1 || V >= 2),
                "values per lane must be a power of two <= 64");
  float v[V];
#pragma unroll
  for (int mr = 0; mr < NMAT * R; ++mr)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      v[mr * NT + tt] = acc[mr * TC + tt];
      acc[mr * TC + tt] = 0.0f;
    }
  Halve<V>::run(v, lane, 32);
  if (NMAT == 2) {
    const float u = __shfl_xor(v[0], 32);  // the up value pairs with this gate value
    if (lane < 32 && (lane & ((1 << SH) - 1)) == 0) {
      const int idx = lane >> SH;
      const int r = idx / NT, tt = idx - (idx / NT) * NT;
      if (r < rv && tt < nt) {
        const float a = v[0];
        const float h = a / (1.0f + expf(-a)) * u;
        const size_t off = static_cast<size_t>(tok_h[tt]) * rows + r0 + r;
        if (yb != nullptr) {
          yb[tt * ystride + r0 + r] = h;
        } else if (COH) {
          coh_store(reinterpret_cast<float*>(p.H) + off, h);
        } else if (WTraits<WT>::XB == 4) {
          reinterpret_cast<float*>(p.H)[off] = h;
        } else {
          reinterpret_cast<uint16_t*>(p.H)[off] = f32_to_bf16_bits(h);
        }
      }
    }
  } else {
    if ((lane & ((1 << SH) - 1)) == 0) {
      const int idx = lane >> SH;
      const int r = idx / NT, tt = idx - (idx / NT) * NT;
      if (r < rv && tt < nt) {
        if (yb != nullptr) {
          yb[tt * ystride + r0 + r] = v[0];
        } else if (COH) {
          coh_store(tok_y[tt] + r0 + r, v[0]);
        } else {
          tok_y[tt][r0 + r] = v[0];
        }
      }
    }
  }
}

// ------------------------------------------------- matrix-core products
// v_mfma_f32_4x4x4_16b_bf16 computes 16 independent 4x4x4 block products:
// lane 4b + q holds row q of block b's A (4 K elements), column q of its B
// (token q, the same 4 K elements) and column q of its D (row i in register
// i; layout checked on the device with one-hot operands).  Here block b
// of step s is K range [s*STEP + b*VEC, +VEC) of the four rows: every block
// sums part of the same dot products, and the 16 partial blocks are added
// across lanes once per unit (finish_unit_mf).  Token group g (tokens 4g..4g+3)
// has its own D; the tokens come from LDS as bf16.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4 as_s16x4(unsigned lo, unsigned hi) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  u32x2 v;
  v.x = lo;
  v.y = hi;
  return __builtin_bit_cast(s16x4, v);
}
__device__ __forceinline__ f32x4 mfma4(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, b, c, 0, 0, 0);
}

// Token rows of the B operand: lane 4b + q of token group g reads the staged
// row at byte offset boff[g] (token 4g + q of the unit's group); only the
// first tga groups hold tokens (tga is the same in every lane).
template <int WT, int TC, int R, int NMAT, int SPC>
__device__ __forceinline__ void mul_chunk_mf(int kc, int lane, const uint8_t* xs,
                                             const int (&boff)[TC / 4], int tga,
                                             const u32x4 (&buf)[NMAT][SPC][1],
                                             const float (&sc)[NMAT][SPC], float* acc) {
  using C = StreamCfg<WT, TC, R, NMAT, SPC>;
  using T = typename C::T;
  constexpr int TG = TC / 4;
  const int b = lane >> 2;
#pragma unroll
  for (int s = 0; s < SPC; ++s) {
    const int k = kc * C::CH + s * C::STEP + b * T::VEC;
#pragma unroll
    for (int g = 0; g < TG; ++g) {
      if (g > 0 && g >= tga) break;  // uniform: the unit's tokens end here
      // token 4g + q, elements [k, k + VEC): 16 bytes per 8 elements
      u32x4 xf[T::VEC / 8];
#pragma unroll
      for (int h = 0; h < T::VEC / 8; ++h) xf[h] = ld16(xs + boff[g] + (k + 8 * h) * 2);
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        const u32x4 w = buf[m][s][0];
        float* d4 = acc + (m * TG + g) * 4;
        if constexpr (WT == WT_BF16) {
          f32x4 d = {d4[0], d4[1], d4[2], d4[3]};
          d = mfma4(as_s16x4(w.x, w.y), as_s16x4(xf[0].x, xf[0].y), d);
          d = mfma4(as_s16x4(w.z, w.w), as_s16x4(xf[0].z, xf[0].w), d);
#pragma unroll
          for (int r = 0; r < 4; ++r) d4[r] = d[r];
        } else {
          // 16 E4M3FN codes -> bf16 exactly; the block scale of the lane's K
          // range multiplies the block products of this step
          const unsigned wd[4] = {w.x, w.y, w.z, w.w};
          f32x4 t = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const s16x4 a = as_s16x4(__builtin_bit_cast(unsigned, fp8x2_to_bf16x2<false>(wd[h])),
                                     __builtin_bit_cast(unsigned, fp8x2_to_bf16x2<true>(wd[h])));
            const u32x4 xv = xf[h >> 1];
            t = mfma4(a, (h & 1) ? as_s16x4(xv.z, xv.w) : as_s16x4(xv.x, xv.y), t);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) d4[r] = fmaf(sc[m][s], t[r], d4[r]);
        }
      }
    }
  }
}

// End of a matrix-core unit: add the 16 block products of every (matrix,
// token group) across lanes (bits 5 and 4 by halving, then bits 3 and 2), so
// lane l with bits 2 and 3 clear holds row 2*bit5 + bit4, token l & 3; the
// gate and up sums of one (row, token) land in the same lane.  Token t of the
// unit's group (t < nt) writes H row hrows[t] (UP) or output row yrows[t]
// (DOWN); with an LDS output buffer yb, row r of token t goes to
// yb[t * ystride + r] instead.  BUF: yb is always given, and no global store
// is compiled in (the one-launch streaming loop).
template <int WT, int TC, int R, int NMAT, int SPC, bool COH, bool BUF = false>
__device__ __forceinline__ void finish_unit_mf(const FfnParams& p, int nt, int tga, int r0, int rv,
                                               int rows, int lane, const int* hrows,
                                               float* const* yrows, float* acc,
                                               float* yb = nullptr, int ystride = 0) {
  constexpr int TG = TC / 4;
  const bool h5 = (lane & 32) != 0, h4 = (lane & 16) != 0;
  float res[NMAT][TG];
#pragma unroll
  for (int g = 0; g < TG; ++g) {
    if (g > 0 && g >= tga) break;
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      float* d = acc + (m * TG + g) * 4;
      float k0 = h5 ? d[2] : d[0], k1 = h5 ? d[3] : d[1];
      const float s0 = h5 ? d[0] : d[2], s1 = h5 ? d[1] : d[3];
      k0 += __shfl_xor(s0, 32);
      k1 += __shfl_xor(s1, 32);
      float v = h4 ? k1 : k0;
      v += __shfl_xor(h4 ? k0 : k1, 16);
      v += __shfl_xor(v, 8);
      v += __shfl_xor(v, 4);
      res[m][g] = v;
#pragma unroll
      for (int r = 0; r < 4; ++r) d[r] = 0.0f;
    }
  }
  if ((lane & 12) != 0) return;
  const int r = (h5 ? 2 : 0) + (h4 ? 1 : 0), q = lane & 3;
  if (r >= rv) return;
#pragma unroll
  for (int g = 0; g < TG; ++g) {
    if (g > 0 && g >= tga) break;
    const int tt = 4 * g + q;
    if (tt >= nt) continue;
    if (NMAT == 2) {
      const float a = res[0][g];
      const float h = a / (1.0f + expf(-a)) * res[NMAT - 1][g];
      const size_t off = static_cast<size_t>(hrows[tt]) * rows + r0 + r;
      if (BUF || yb != nullptr) {
        yb[tt * ystride + r0 + r] = h;
      } else if (COH) {
        coh_store(reinterpret_cast<float*>(p.H) + off, h);
      } else {
        reinterpret_cast<uint16_t*>(p.H)[off] = f32_to_bf16_bits(h);
      }
    } else {
      if (BUF || yb != nullptr) {
        yb[tt * ystride + r0 + r] = res[0][g];
      } else if (COH) {
        coh_store(yrows[tt] + r0 + r, res[0][g]);
      } else {
        yrows[tt][r0 + r] = res[0][g];
      }
    }
  }
}

// Multiply one chunk, and end the unit after its last chunk: on the matrix
// cores for token tiles of four or more (bf16, fp8), else as dot products.
template <int WT, int TC, int R, int NMAT, int SPC, bool COH>
__device__ __forceinline__ void mul_finish(int nt, bool last, int kc, int Kpad, int lane,
                                           const uint8_t* xs,
                                           const u32x4 (&buf)[NMAT][SPC][StreamCfg<WT, TC, R, NMAT, SPC>::LR],
                                           const float (&sc)[NMAT][SPC], float* acc,
                                           const FfnParams& p, int r0, int rv, int rows,
                                           const int* tok_h, float* const* tok_y,
                                           float* yb = nullptr, int ys = 0) {
  if constexpr (StreamCfg<WT, TC, R, NMAT, SPC>::MF) {
    // tokens staged as one tile [TC][Kpad]: token 4g + q in row 4g + q
    int boff[TC / 4];
#pragma unroll
    for (int g = 0; g < TC / 4; ++g) boff[g] = (4 * g + (lane & 3)) * Kpad * 2;
    mul_chunk_mf<WT, TC, R, NMAT, SPC>(kc, lane, xs, boff, TC / 4, buf, sc, acc);
    if (last)
      finish_unit_mf<WT, TC, R, NMAT, SPC, COH>(p, nt, TC / 4, r0, rv, rows, lane, tok_h, tok_y,
                                                acc, yb, ys);
  } else {
    mul_chunk_nt<WT, TC, R, NMAT, SPC, TC>(kc, Kpad, lane, xs, buf, sc, acc);
    if (last)
      finish_unit<WT, TC, R, NMAT, SPC, COH, TC>(p, nt, r0, rv, rows, lane, tok_h, tok_y, acc, yb,
                                                 ys);
  }
}

// ------------------------------------------------ matrix-core range table
// The matrix-core kernels stage the tokens of a whole range once, packed
// group after group: the token vectors of each group (UP, rows of x) or its
// H rows (DOWN).  A unit of group j then multiplies only that group's rows
// of the table (ceil(cnt/4) token groups), so a group of up to TC tokens
// streams its expert once and the range needs no restaging between groups.
constexpr int kRangeGroups = 8;  // groups one range may touch on this path
struct RangeTab {
  int ustart[kRangeGroups + 1];  // first unit of group j, relative to the range
  int cnt[kRangeGroups];         // tokens of group j
  int ylo[kRangeGroups];         // DOWN output buffer: first row of group j in the range,
  int ylen[kRangeGroups];        //   its rows in the range,
  int yoff[kRangeGroups];        //   and its first float in the buffer
  int row0[kRangeGroups];        // first row of group j in the staged table
  int xrow[kRangeGroups][32];    // row of x of token t of group j
  int hrow[kRangeGroups][32];    // H row of token t of group j
  float* yrow[kRangeGroups][32]; // output row of token t of group j
};

// Streams units [lo, hi) on the matrix cores from a range table; false (and
// nothing done) when the range does not fit it: more than kRangeGroups
// groups, a group of more than TC tokens, or a table larger than the LDS.
template <int WT, int TC, int R, int NMAT, int SPC, bool COH>
__device__ __forceinline__ bool run_range_mf(const FfnParams& p, const Meta& mt, int U, long long lo,
                                             long long hi, uint8_t* xs, RangeTab& rt, int* claim,
                                             const Sync& sy) {
  using C = StreamCfg<WT, TC, R, NMAT, SPC>;
  static_assert(C::MF, "matrix-core tiles only");
  constexpr bool UP = NMAT == 2;
  constexpr int TG = TC / 4;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rows = UP ? p.f : p.d;
  const int Kdim = UP ? p.d : p.f;
  const int nchunks = (Kdim + C::CH - 1) / C::CH;
  const int Kpad = nchunks * C::CH;
  const int upg = units_per_group(rows, R);
  // unit indices fit 31 bits (the launcher bounds n, K, S and f)
  const int g0 = uni(static_cast<int>(static_cast<unsigned>(lo) / static_cast<unsigned>(upg)));
  const int ng = uni(static_cast<int>(static_cast<unsigned>(hi - 1) / static_cast<unsigned>(upg))) -
                 g0 + 1;
  if (ng > kRangeGroups) return false;
  int tot = 0, big = 0;
  for (int j = 0; j < ng; ++j) {
    Group G;
    group_at(p, mt, U, g0 + j, G);
    const int c = uni(G.cnt);
    tot += c;
    big |= c > TC;
  }
  // UP with more staged rows than tokens (groups sharing tokens): stage the
  // n token rows once and let each group index them
  const bool xtab = UP && tot > p.n;
  const int trows = xtab ? p.n : tot;
  if (big || static_cast<long long>(trows) * Kpad * 2 > p.lds_bytes) return false;

  // rows of group j inside the range: [ylo, ylo + ylen)
  auto out_rows = [&](int j, int& ylo, int& ylen) {
    const long long gs = static_cast<long long>(g0 + j) * upg;
    const int ulo = static_cast<int>((gs > lo ? gs : lo) - gs);
    const int uhi = static_cast<int>((hi < gs + upg ? hi : gs + upg) - gs);
    ylo = ulo * R;
    ylen = min(rows, uhi * R) - ylo;
  };
  // One-launch pass: the unit outputs (H rows, or slot output rows) collect
  // in LDS after the table and go out with device-scope stores at the end of
  // the range, so the streaming loop holds no global store.  A store there
  // would hold back the weight loads issued after it until memory
  // acknowledged it (loads and stores complete in order), and the compiler,
  // which counts stores and loads on one counter, would wait for every load
  // in flight before each multiply (the prefetch drained every step).  A
  // range without room for the buffer takes the dot-product path.
  float* ybuf = nullptr;
  if (COH) {
    const long long tb = (static_cast<long long>(trows) * Kpad * 2 + 15) / 16 * 16;
    long long yfl = 0;
    for (int j = 0; j < ng; ++j) {
      Group G;
      group_at(p, mt, U, g0 + j, G);
      int ylo, ylen;
      out_rows(j, ylo, ylen);
      yfl += static_cast<long long>(uni(G.cnt)) * ylen;
    }
    if (tb + yfl * 4 <= p.lds_bytes) ybuf = reinterpret_cast<float*>(xs + tb);
    if (ybuf == nullptr) return false;
  }

  const int nur = static_cast<int>(hi - lo);
  u32x4 b0[NMAT][SPC][1], b1[NMAT][SPC][1];
  float s0[NMAT][SPC], s1[NMAT][SPC];
  float acc[C::NACC];
#pragma unroll
  for (int i = 0; i < C::NACC; ++i) acc[i] = 0.0f;
  // (32-bit unit arithmetic: the 64-bit division routine in the loop holds
  // a wait for every load in flight on its slow path)
  auto unit_group = [&](int u, Group& G, int& r0, int& rv) {
    const unsigned gu = static_cast<unsigned>(lo) + static_cast<unsigned>(u < nur ? u : 0);
    const int g = static_cast<int>(gu / static_cast<unsigned>(upg));
    group_at(p, mt, U, g, G);
    G.e = uni(G.e);
    G.shared = uni(G.shared);
    r0 = static_cast<int>(gu - static_cast<unsigned>(g) * static_cast<unsigned>(upg)) * R;
    const int valid = G.shared || (G.e >= 0 && G.e < p.E);
    rv = (u < nur && valid) ? min(R, rows - r0) : 0;
  };
  auto first_chunk = [&]() {
    Group G;
    int r0, rv;
    unit_group(wave, G, r0, rv);
    load_chunk<WT, TC, R, NMAT, SPC>(p, G, r0, rv, 0, rows, Kdim, lane, b0, s0);
  };
  // DOWN: the first weight chunk goes out before the range table is built,
  // so the table is built while it is in flight (and while the UP owners of
  // the range's groups finish)
  if (!UP) first_chunk();

  // the range table (the LDS the previous phase used is free: its last
  // barrier has passed)
  // (lane j of wavefront 0 takes group j; the staged rows and the buffered
  // outputs of the groups before j are exclusive prefix sums across lanes)
  if (static_cast<int>(threadIdx.x) < kWave) {
    const int j = threadIdx.x;
    int c = 0, yl = 0;
    if (j < ng) {
      Group G;
      group_at(p, mt, U, g0 + j, G);
      const long long gs = static_cast<long long>(g0 + j) * upg;
      rt.ustart[j] = static_cast<int>((gs > lo ? gs : lo) - lo);
      rt.cnt[j] = G.cnt;
      int ylo, ylen;
      out_rows(j, ylo, ylen);
      rt.ylo[j] = ylo;
      rt.ylen[j] = ylen;
      c = G.cnt;
      yl = G.cnt * ylen;
      if (j == ng - 1) rt.ustart[ng] = static_cast<int>(hi - lo);
    }
    int r = c, yo = yl;  // inclusive sums over lanes 0..j (ng <= kRangeGroups = 8)
#pragma unroll
    for (int o = 1; o < kRangeGroups; o <<= 1) {
      const int a = __shfl_up(r, o), b = __shfl_up(yo, o);
      if (j >= o) {
        r += a;
        yo += b;
      }
    }
    if (j < ng) {
      rt.row0[j] = r - c;
      rt.yoff[j] = yo - yl;
    }
  }
  for (int i = threadIdx.x; i < ng * 32; i += kStreamThreads) {
    const int j = i >> 5, t = i & 31;
    Group G;
    group_at(p, mt, U, g0 + j, G);
    int xrow = 0, hrow = 0;
    float* yrow = nullptr;
    if (t < G.cnt) token_of(p, mt, G, t, xrow, hrow, yrow);
    rt.xrow[j][t] = xrow;
    rt.hrow[j][t] = hrow;
    rt.yrow[j][t] = yrow;
  }

  // the staged table: rows of x (UP, bf16: token rows when xtab, else each
  // group's tokens in turn) or each group's rows of H (DOWN: f32 coherent
  // loads rounded to bf16 in one launch, bf16 otherwise); zero beyond Kdim.
  // Two loads in flight per thread before their stores.
  auto stage = [&]() {
    const int vpt = Kpad / 8;
    auto fetch = [&](int v) {
      const int row = v / vpt;
      const int k = (v - row * vpt) * 8;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (k < Kdim) {
        if (xtab) return ld16(p.x + (static_cast<size_t>(row) * Kdim + k) * 2);
        int j = 0;
        while (j + 1 < ng && rt.row0[j + 1] <= row) ++j;
        if (UP) {
          const int xrow = rt.xrow[j][row - rt.row0[j]];
          val = ld16(p.x + (static_cast<size_t>(xrow) * Kdim + k) * 2);
        } else {
          const int hrow = rt.hrow[j][row - rt.row0[j]];
          if (COH) {
            val = coh_h_to_staged<2>(p.H, (static_cast<size_t>(hrow) * Kdim + k) * 4);
          } else {
            val = ld16(p.H + (static_cast<size_t>(hrow) * Kdim + k) * 2);
          }
        }
      }
      return val;
    };
    const int nv = trows * vpt, step = kStreamThreads;
    int v = threadIdx.x;
    for (; v + step < nv; v += 2 * step) {
      const u32x4 a = fetch(v), b = fetch(v + step);
      st16(xs + static_cast<size_t>(v) * 16, a);
      st16(xs + static_cast<size_t>(v + step) * 16, b);
    }
    if (v < nv) st16(xs + static_cast<size_t>(v) * 16, fetch(v));
  };
  if (UP) {
    // the table (written above) is read by the staging: publish it; the x
    // rows are loaded before the first weight chunk, so their LDS stores do
    // not wait behind it (loads complete in order)
    __syncthreads();
    stage();
    __builtin_amdgcn_sched_barrier(0);
    first_chunk();
    if (threadIdx.x == 0) {
      for (int j = 0; j < ng; ++j) {
        Group G;
        group_at(p, mt, U, g0 + j, G);
        if (!G.shared && (G.e < 0 || G.e >= p.E)) atomicOr(p.err, ERRBIT_BAD_IDS);
      }
    }
  } else {
    // DOWN: the first chunk (issued above) is in flight during the wait for
    // the UP flags
    if (COH)
      for (int j = 0; j < ng; ++j) wait_group_ready(sy, g0 + j);
    __syncthreads();
    stage();
  }
  if (threadIdx.x == 0) *claim = kStreamWaves;
  __syncthreads();

  // unit u: group j of the range, its rows, the B rows of its tokens and
  // where its outputs go in the LDS buffer
  auto unit_tab = [&](int u, int& j, int& r0, int& rv, int& nt, int& tga, int (&boff)[TG],
                      float*& yb, int& ys) {
    j = 0;
#pragma unroll
    for (int i = 1; i < kRangeGroups; ++i)
      if (i < ng && rt.ustart[i] <= u) j = i;
    j = uni(j);
    if (ybuf != nullptr) {
      yb = ybuf + rt.yoff[j] - rt.ylo[j];
      ys = rt.ylen[j];
    }
    const long long gu = lo + (u < nur ? u : 0);
    r0 = static_cast<int>(gu - static_cast<long long>(g0 + j) * upg) * R;
    rv = u < nur ? min(R, rows - r0) : 0;
    nt = uni(rt.cnt[j]);
    tga = (nt + 3) >> 2;
#pragma unroll
    for (int g = 0; g < TG; ++g) {
      const int t = max(min(4 * g + (lane & 3), nt - 1), 0);
      const int row = xtab ? rt.xrow[j][t] : rt.row0[j] + t;
      boff[g] = row * Kpad * 2;
    }
  };
  int u = wave, kc = 0;
  int j, r0, rv, nt, tga, boff[TG], ys = 0;
  float* yb = nullptr;
  unit_tab(u, j, r0, rv, nt, tga, boff, yb, ys);
  // the bases of the unit whose chunks are loaded next, recomputed when it
  // changes: the 64-bit address products stay out of the per-chunk code,
  // whose temporaries otherwise took registers of loads in flight (and the
  // compiler then waited for every load before reusing them)
  const size_t row_bytes = static_cast<size_t>(Kdim) * C::T::EB;
  const size_t mat = static_cast<size_t>(rows) * row_bytes;
  const int kb = Kdim / 128;
  int nb_u = -1, nb_rv = 0;
  const uint8_t* nb_w[NMAT];
  const float* nb_s[NMAT];
  auto unit_base = [&](int c) {
    Group G;
    int r0;
    unit_group(c, G, r0, nb_rv);
    const int e = nb_rv > 0 ? G.e : 0;
    const int rr = nb_rv > 0 ? r0 : 0;
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      nb_w[m] = (NMAT == 1 ? wptr<2>(p, G.shared)
                           : (m == 0 ? wptr<0>(p, G.shared) : wptr<1>(p, G.shared))) +
                static_cast<size_t>(e) * mat + static_cast<size_t>(rr) * row_bytes;
      if (WT == WT_FP8)
        nb_s[m] = (NMAT == 1 ? sptr<2>(p, G.shared)
                             : (m == 0 ? sptr<0>(p, G.shared) : sptr<1>(p, G.shared))) +
                  (static_cast<size_t>(e) * (rows / 128) + rr / 128) * kb;
      else
        nb_s[m] = nullptr;
    }
    nb_u = c;
  };
  auto half = [&](int un, int kn, u32x4 (&bl)[NMAT][SPC][1], float (&sl)[NMAT][SPC],
                  const u32x4 (&bm)[NMAT][SPC][1], const float (&sm)[NMAT][SPC]) {
    if (un != nb_u) unit_base(un);
    load_chunk_mf<WT, TC, R, NMAT, SPC>(nb_w, nb_s, static_cast<unsigned>(row_bytes), nb_rv, kn,
                                        Kdim, lane, p.zeros, bl, sl);
    mul_chunk_mf<WT, TC, R, NMAT, SPC>(kc, lane, xs, boff, tga, bm, sm, acc);
    if (kc == nchunks - 1)
      finish_unit_mf<WT, TC, R, NMAT, SPC, COH, COH>(p, nt, tga, r0, rv, rows, lane, rt.hrow[j],
                                                     rt.yrow[j], acc, yb, ys);
  };
  auto take = [&]() {
    int v = 0;
    if (lane == 0) v = atomicAdd(claim, 1);
    return uni(v);
  };
  int un = u, kn = kc + 1;
  if (kn == nchunks) {
    kn = 0;
    un = take();
  }
  while (true) {
    half(un, kn, b1, s1, b0, s0);
    if (un >= nur) break;
    if (kn == 0) unit_tab(un, j, r0, rv, nt, tga, boff, yb, ys);
    u = un;
    kc = kn;
    if (++kn == nchunks) {
      kn = 0;
      un = take();
    }
    half(un, kn, b0, s0, b1, s1);
    if (un >= nur) break;
    if (kn == 0) unit_tab(un, j, r0, rv, nt, tga, boff, yb, ys);
    u = un;
    kc = kn;
    if (++kn == nchunks) {
      kn = 0;
      un = take();
    }
  }
  if (ybuf != nullptr) {
    __syncthreads();  // every unit's outputs are in the buffer
    for (int jj = 0; jj < ng; ++jj) {
      const int c = rt.cnt[jj], len = rt.ylen[jj], y0 = rt.ylo[jj], off = rt.yoff[jj];
      for (int i = threadIdx.x; i < c * len; i += kStreamThreads) {
        const int t = i / len, r = i - t * len;
        float* dst = UP ? reinterpret_cast<float*>(p.H) + static_cast<size_t>(rt.hrow[jj][t]) * rows
                        : rt.yrow[jj][t];
        coh_store(dst + y0 + r, ybuf[off + i]);
      }
    }
  }
  return true;
}

// ------------------------------------------------------------ one range
// Streams units [lo, hi) of one phase on the dot-product paths (tiles of one
// or two tokens, and ranges the matrix-core range table does not take).
template <int WT, int TC, int R, int NMAT, int SPC, bool COH>
__device__ __forceinline__ void run_range_dot(const FfnParams& p, const Meta& mt, int U,
                                              long long lo, long long hi, uint8_t* xs, int* tok_h,
                                              float** tok_y, int* claim, const Sync& sy) {
  using C = StreamCfg<WT, TC, R, NMAT, SPC>;
  constexpr bool UP = NMAT == 2;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rows = UP ? p.f : p.d;
  const int Kdim = UP ? p.d : p.f;
  const int nchunks = (Kdim + C::CH - 1) / C::CH;
  const int Kpad = nchunks * C::CH;
  const int upg = units_per_group(rows, R);

  u32x4 b0[NMAT][SPC][C::LR], b1[NMAT][SPC][C::LR];
  float s0[NMAT][SPC], s1[NMAT][SPC];
  float acc[C::NACC];
#pragma unroll
  for (int i = 0; i < C::NACC; ++i) acc[i] = 0.0f;

  // Fast path: the range touches at most two groups, each within one token
  // tile, and LDS has two token slots: stage both up front, then stream with
  // no load other than the weights (a load that must be waited for would,
  // with in-order completion, drain the weight prefetch).
  const int g0 = uni(static_cast<int>(static_cast<unsigned>(lo) / static_cast<unsigned>(upg)));
  const int g1 = uni(static_cast<int>(static_cast<unsigned>(hi - 1) / static_cast<unsigned>(upg)));
  Group G0, G1;
  group_at(p, mt, U, g0, G0);
  group_at(p, mt, U, g1, G1);
  G0.e = uni(G0.e); G0.shared = uni(G0.shared); G0.cnt = uni(G0.cnt);
  G0.first = uni(G0.first); G0.s_idx = uni(G0.s_idx);
  G1.e = uni(G1.e); G1.shared = uni(G1.shared); G1.cnt = uni(G1.cnt);
  G1.first = uni(G1.first); G1.s_idx = uni(G1.s_idx);
  const bool fast = g1 - g0 <= 1 && G0.cnt <= TC && G1.cnt <= TC && (g1 == g0 || p.lds_slots >= 2);
  if (fast) {
    const int v0 = G0.shared || (G0.e >= 0 && G0.e < p.E);
    const int v1 = G1.shared || (G1.e >= 0 && G1.e < p.E);
    if (UP && threadIdx.x == 0 && (!v0 || !v1)) atomicOr(p.err, ERRBIT_BAD_IDS);
    const int nur = static_cast<int>(hi - lo);  // units of the range, in order
    const long long g1lo = static_cast<long long>(g0 + 1) * upg;  // first unit of g1
    const size_t slot_bytes = static_cast<size_t>(TC) * Kpad * C::T::XB;
    uint8_t* xs1 = xs + (g1 != g0 ? slot_bytes : 0);
    // one-launch pass, DOWN: the slot outputs collect in LDS after the token
    // slots and go out at the end of the range (as on the matrix-core path):
    // rows [ylo_s, ylo_s + ylen_s) of group g0 (s = 0) and g1 (s = 1).  (UP
    // writes H directly here: its units span several chunks, and the end of
    // an UP range is what the DOWN waits are for; measured slower buffered.)
    float* ybuf = nullptr;
    int ylo0 = 0, ylen0 = 0, ylo1 = 0, ylen1 = 0;
    if (COH && !UP) {
      auto rows_in = [&](long long gs, int& ylo, int& ylen) {
        const int ulo = static_cast<int>((gs > lo ? gs : lo) - gs);
        const int uhi = static_cast<int>((hi < gs + upg ? hi : gs + upg) - gs);
        ylo = ulo * R;
        ylen = min(rows, uhi * R) - ylo;
      };
      rows_in(g1lo - upg, ylo0, ylen0);
      if (g1 != g0) rows_in(g1lo, ylo1, ylen1);
      const long long base = ((g1 != g0 ? 2 : 1) * static_cast<long long>(slot_bytes) + 15) / 16 * 16;
      const long long need = base + 4LL * (static_cast<long long>(G0.cnt) * ylen0 +
                                           (g1 != g0 ? static_cast<long long>(G1.cnt) * ylen1 : 0));
      if (need <= p.lds_bytes) ybuf = reinterpret_cast<float*>(xs + base);
    }
    // Units are handed out dynamically: wavefront w starts with unit w and
    // then takes the next unclaimed unit from the workgroup's LDS counter, so
    // the wavefronts of the CU finish together however the hardware shares
    // the memory pipeline among them.  Unit u: its group (0: g0, 1: g1), its
    // first row r0 in that group and its valid rows rv (0 beyond the range).
    auto unit_info = [&](int u, int& sg, int& r0, int& rv) {
      const long long gu = lo + u;
      sg = gu >= g1lo;
      r0 = static_cast<int>(gu - (sg ? g1lo : g1lo - upg)) * R;
      rv = u < nur ? min(R, rows - r0) : 0;
    };
    auto take = [&]() {
      int v = 0;
      if (lane == 0) v = atomicAdd(claim, 1);
      return uni(v);
    };
    int u = wave, kc = 0;
    auto stage_both = [&]() {
      Walk w;
      w.G = G0;
      w.tile = 0;
      stage_tokens<WT, TC, !UP, COH>(p, mt, w, Kdim, Kpad, xs, tok_h, tok_y);
      if (g1 != g0) {
        w.G = G1;
        stage_tokens<WT, TC, !UP, COH>(p, mt, w, Kdim, Kpad, xs1, tok_h + TC, tok_y + TC);
      }
    };
    // UP: the token rows (cached) are loaded before the first weight chunk,
    // so their LDS stores do not wait behind it (loads complete in order)
    // and the chunk is in flight across the barrier; DOWN: the chunk is in
    // flight during the wait for the UP flags, H is staged after it
    if (UP) stage_both();
    __builtin_amdgcn_sched_barrier(0);  // keep the weight loads behind the staging loads
    {
      int sg, r0, rv;
      unit_info(u, sg, r0, rv);
      load_chunk<WT, TC, R, NMAT, SPC>(p, sg ? G1 : G0, r0, (sg ? v1 : v0) ? rv : 0, 0, rows,
                                       Kdim, lane, b0, s0);
    }
    if (COH && !UP) {
      wait_group_ready(sy, g0);
      if (g1 != g0) wait_group_ready(sy, g1);
    }
    if (!UP) stage_both();
    if (threadIdx.x == 0) *claim = kStreamWaves;
    __syncthreads();
    // One half-step prefetches chunk (un, kn) into one buffer and multiplies
    // chunk (u, kc) from the other.  The loop runs whole pairs of half-steps,
    // so on every path back to its head the only loads in flight are the
    // prefetch of the next chunk (a half-finished pair would leave a buffer
    // that the head overwrites in flight, and the compiler would wait for
    // every load there).
    auto half = [&](int uc, int kcc, int un, int kn, u32x4 (&bl)[NMAT][SPC][C::LR],
                    float (&sl)[NMAT][SPC], const u32x4 (&bm)[NMAT][SPC][C::LR],
                    const float (&sm)[NMAT][SPC]) {
      {
        int sg, r0, rv;
        unit_info(un, sg, r0, rv);
        load_chunk<WT, TC, R, NMAT, SPC>(p, sg ? G1 : G0, r0, (sg ? v1 : v0) ? rv : 0, kn, rows,
                                         Kdim, lane, bl, sl);
      }
      int sg, r0, rv;
      unit_info(uc, sg, r0, rv);
      float* yb = nullptr;
      if (ybuf != nullptr) yb = sg ? ybuf + G0.cnt * ylen0 - ylo1 : ybuf - ylo0;
      mul_finish<WT, TC, R, NMAT, SPC, COH>(sg ? G1.cnt : G0.cnt, kcc == nchunks - 1, kcc, Kpad,
                                            lane, sg ? xs1 : xs, bm, sm, acc, p, r0, rv, rows,
                                            tok_h + (sg ? TC : 0), tok_y + (sg ? TC : 0), yb,
                                            sg ? ylen1 : ylen0);
    };
    int un = u, kn = kc + 1;
    if (kn == nchunks) {
      kn = 0;
      un = take();
    }
    while (true) {
      half(u, kc, un, kn, b1, s1, b0, s0);
      if (un >= nur) break;
      u = un;
      kc = kn;
      if (++kn == nchunks) {
        kn = 0;
        un = take();
      }
      half(u, kc, un, kn, b0, s0, b1, s1);
      if (un >= nur) break;
      u = un;
      kc = kn;
      if (++kn == nchunks) {
        kn = 0;
        un = take();
      }
    }
    if (ybuf != nullptr) {
      __syncthreads();  // every unit's outputs are in the buffer
      for (int sg = 0; sg < (g1 != g0 ? 2 : 1); ++sg) {
        const int c = sg ? G1.cnt : G0.cnt, len = sg ? ylen1 : ylen0, y0 = sg ? ylo1 : ylo0;
        const float* src = ybuf + (sg ? G0.cnt * ylen0 : 0);
        for (int i = threadIdx.x; i < c * len; i += kStreamThreads) {
          const int t = i / len, r = i - t * len;
          float* dst = UP ? reinterpret_cast<float*>(p.H) +
                                static_cast<size_t>(tok_h[sg * TC + t]) * rows
                          : tok_y[sg * TC + t];
          coh_store(dst + y0 + r, src[i]);
        }
      }
    }
    return;
  }

  // General path: restage tokens at every (group, token tile) change.
  Walk cur;
  cur.done = 0;
  walk_group<TC>(p, mt, U, cur, g0, lo, hi, upg);
  if (UP && !cur.valid && threadIdx.x == 0) atomicOr(p.err, ERRBIT_BAD_IDS);

  int r0, rv;
  wave_unit<R>(cur.ua, cur.ub, cur.s, wave, rows, r0, rv);
  load_chunk<WT, TC, R, NMAT, SPC>(p, cur.G, r0, cur.valid ? rv : 0, cur.kc, rows, Kdim, lane, b0,
                                   s0);
  if (COH && !UP) wait_group_ready(sy, g0);
  stage_tokens<WT, TC, !UP, COH>(p, mt, cur, Kdim, Kpad, xs, tok_h, tok_y);
  __syncthreads();

  Walk nxt = cur;
  walk_next<TC>(p, mt, U, nxt, nchunks, lo, hi, upg);
  // two chunks per trip so the register buffers keep fixed names
  while (true) {
    int n0, nv;
    wave_unit<R>(nxt.ua, nxt.ub, nxt.s, wave, rows, n0, nv);
    load_chunk<WT, TC, R, NMAT, SPC>(p, nxt.G, n0, (nxt.valid && !nxt.done) ? nv : 0, nxt.kc, rows,
                                     Kdim, lane, b1, s1);
    wave_unit<R>(cur.ua, cur.ub, cur.s, wave, rows, r0, rv);
    mul_finish<WT, TC, R, NMAT, SPC, COH>(min(TC, cur.G.cnt - cur.tile * TC), cur.kc == nchunks - 1,
                                          cur.kc, Kpad, lane, xs, b0, s0, acc, p, r0, rv, rows,
                                          tok_h, tok_y);
    if (nxt.done) break;
    if (nxt.g != cur.g || nxt.tile != cur.tile) {
      if (UP && nxt.g != cur.g && !nxt.valid && threadIdx.x == 0) atomicOr(p.err, ERRBIT_BAD_IDS);
      __syncthreads();
      if (COH && !UP && nxt.g != cur.g) wait_group_ready(sy, nxt.g);
      stage_tokens<WT, TC, !UP, COH>(p, mt, nxt, Kdim, Kpad, xs, tok_h, tok_y);
      __syncthreads();
    }
    cur = nxt;
    walk_next<TC>(p, mt, U, nxt, nchunks, lo, hi, upg);

    wave_unit<R>(nxt.ua, nxt.ub, nxt.s, wave, rows, n0, nv);
    load_chunk<WT, TC, R, NMAT, SPC>(p, nxt.G, n0, (nxt.valid && !nxt.done) ? nv : 0, nxt.kc, rows,
                                     Kdim, lane, b0, s0);
    wave_unit<R>(cur.ua, cur.ub, cur.s, wave, rows, r0, rv);
    mul_finish<WT, TC, R, NMAT, SPC, COH>(min(TC, cur.G.cnt - cur.tile * TC), cur.kc == nchunks - 1,
                                          cur.kc, Kpad, lane, xs, b1, s1, acc, p, r0, rv, rows,
                                          tok_h, tok_y);
    if (nxt.done) break;
    if (nxt.g != cur.g || nxt.tile != cur.tile) {
      if (UP && nxt.g != cur.g && !nxt.valid && threadIdx.x == 0) atomicOr(p.err, ERRBIT_BAD_IDS);
      __syncthreads();
      if (COH && !UP && nxt.g != cur.g) wait_group_ready(sy, nxt.g);
      stage_tokens<WT, TC, !UP, COH>(p, mt, nxt, Kdim, Kpad, xs, tok_h, tok_y);
      __syncthreads();
    }
    cur = nxt;
    walk_next<TC>(p, mt, U, nxt, nchunks, lo, hi, upg);
  }
}

// Streams units [lo, hi) of one phase.  UP (NMAT = 2) reads W_gate and W_up
// rows against the tokens x; DOWN (NMAT = 1) reads W_down rows against H.
// COH: H and the outputs are exchanged between workgroups of one launch
// (H in f32 with coherent stores and loads, and each DOWN group waits for the
// flags of the workgroups that own its UP units); otherwise a kernel boundary
// separates them.
template <int WT, int TC, int R, int NMAT, int SPC, bool COH>
__device__ __forceinline__ void run_range(const FfnParams& p, const Meta& mt, int U, long long lo,
                                          long long hi, uint8_t* xs, int* tok_h, float** tok_y,
                                          RangeTab& rt, int* claim, const Sync& sy) {
  if constexpr (StreamCfg<WT, TC, R, NMAT, SPC>::MF) {
    if (run_range_mf<WT, TC, R, NMAT, SPC, COH>(p, mt, U, lo, hi, xs, rt, claim, sy)) return;
  }
  run_range_dot<WT, TC, R, NMAT, SPC, COH>(p, mt, U, lo, hi, xs, tok_h, tok_y, claim, sy);
}

}  // namespace moe
