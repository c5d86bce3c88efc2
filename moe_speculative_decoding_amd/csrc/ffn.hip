// Expert FFN of a verify pass, deduplicating and per-slot (gfx950).
//
// For every (expert, slot) pair: a = x W_gate, v = x W_up, h = silu(a) * v,
// y = h W_down.  The deduplicating mode streams each union expert once and
// applies it to every slot routed to it; the per-slot mode reads an expert
// once per token-slot ("Speculative Decoding for Mixture-of-Experts Models:
// Expert Bytes, Kernel Bandwidth and the Best Draft Length", abstract;
// Table 5 and Table 6 name the engines' kernels of each kind).
//
// Both modes run the same two kernels over "groups": a group is one expert
// with the list of token rows it serves (dedup: a union expert and its slots,
// or a shared expert and all n tokens; per-slot: one slot, or one
// (token, shared expert) pair).  Kernel 1 (up) computes the f intermediate
// activations of every token of a group; kernel 2 (down) the d outputs.
//
// The work is a batched matrix-vector product with at most a handful of
// tokens per weight row, so it is bound by HBM bandwidth, not by matrix
// throughput.  Each wavefront owns R weight rows (stored one row per output,
// so the reduction runs along contiguous memory) and streams them with
// 16-byte loads, 64 lanes covering 1 KiB of a row per step; the group's
// tokens sit in LDS as bf16 (f32 for f32 weights) and are reused by every row
// of the workgroup.  Products use v_dot2_f32_bf16 (two bf16 MACs, fp32
// accumulate); fp8 codes are widened to bf16 pairs exactly with
// v_cvt_scalef32_pk_bf16_fp8 and the 128x128 block scale is applied once per
// 16 codes.  Partial sums are combined across the wavefront by recursive
// halving (each shuffle stage halves the values per lane), so a wave reduces
// R*T values with about R*T shuffles instead of 6*R*T.
#include <map>
#include <mutex>

#include "common.h"

namespace moe {

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
};

__device__ __forceinline__ void load_meta(const FfnParams& p, Meta& m) {
  const int nk = p.n * p.K;
  if (p.mode == MODE_DEDUP) {
    for (int i = threadIdx.x; i <= p.ucap; i += kBlock) m.a[i] = p.offsets[i];
    for (int i = threadIdx.x; i < p.ucap; i += kBlock) m.b[i] = p.union_ids[i];
    for (int i = threadIdx.x; i < nk; i += kBlock) m.c[i] = p.perm[i];
  } else {
    for (int i = threadIdx.x; i < nk; i += kBlock) m.a[i] = p.ids[i];
  }
}

// token j of a group: its row in x, its row in H and its output row
__device__ __forceinline__ void token_of(const FfnParams& p, const Meta& mt, const Group& G, int j,
                                         int& xrow, int& hrow, float*& yrow) {
  const int nk = p.n * p.K;
  if (p.mode == MODE_DEDUP) {
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

// ------------------------------------------------------------ the walk
// One phase (up: gate/up rows, or down rows) is a list of units: (group g,
// row block of 4*R rows), groups in order, row blocks in order.  Workgroup b
// owns the contiguous unit range [b*NU/G, (b+1)*NU/G), so every workgroup
// streams the same number of bytes and all finish together.  It walks its
// range chunk by chunk (K split in chunks of SPC load steps): for each group
// segment, for each token tile of that group, for each unit, for each chunk.
// The walk is the same for every lane of the workgroup.
struct Walk {
  int g, tile, u, kc, done;
  int ntile, seg_lo, seg_hi;
  int valid;  // expert id in range
  Group G;
};

// group g of a phase: dedup 0..U-1 routed union experts, then the S shared;
// per-slot 0..n*K-1 slots, then the n*S (token, shared expert) pairs
__device__ __forceinline__ void group_at(const FfnParams& p, const Meta& mt, int U, int g,
                                         Group& G) {
  if (p.mode == MODE_DEDUP) {
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

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

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
  w.seg_lo = uni(static_cast<int>(lo > glo ? lo : glo));
  w.seg_hi = uni(static_cast<int>(hi < glo + upg ? hi : glo + upg));
  w.u = w.seg_lo;
  w.kc = 0;
}

template <int TC>
__device__ __forceinline__ void walk_next(const FfnParams& p, const Meta& mt, int U, Walk& w,
                                          int nchunks, long long lo, long long hi, int upg) {
  if (++w.kc < nchunks) return;
  w.kc = 0;
  if (++w.u < w.seg_hi) return;
  if (++w.tile < w.ntile) {
    w.u = w.seg_lo;
    return;
  }
  if (w.seg_hi >= hi) {
    w.done = 1;
    return;
  }
  walk_group<TC>(p, mt, U, w, w.g + 1, lo, hi, upg);
}

// ------------------------------------------------------- streaming kernel
// UP (NMAT = 2): rows j of W_gate and W_up (Kdim = d) -> H[token][j] = silu(a) * v.
// DOWN (NMAT = 1): rows c of W_down (Kdim = f, tokens read from H) -> y[slot][c].
// Each wave owns R rows of the current unit; the weights of the next chunk
// are in flight while the current chunk is multiplied (two register buffers).
template <int WT, int TC, int R, int NMAT, int SPC>
struct StreamCfg {
  using T = WTraits<WT>;
  static constexpr int STEP = kWave * T::VEC;  // elements per load step
  static constexpr int CH = SPC * STEP;        // elements per chunk
  static constexpr int V = NMAT * R * TC;      // partial sums per lane
  static constexpr int SH = 6 - ilog2(V);
  static_assert((V & (V - 1)) == 0 && V <= 64, "values per lane must be a power of two <= 64");
  static_assert(NMAT == 1 || V >= 2, "gate/up pairing needs two values");
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
__device__ __forceinline__ void load_chunk(const FfnParams& p, const Group& G, int live, int urel,
                                           int kc, int rows, int Kdim, int lane, int wave,
                                           u32x4 (&buf)[NMAT][SPC][R], float (&sc)[NMAT][SPC]) {
  using C = StreamCfg<WT, TC, R, NMAT, SPC>;
  using T = typename C::T;
  // Every lane issues every load, outside any branch, and nothing inspects the
  // loaded value before the multiply, so the next chunk stays in flight while
  // the current one is used.  Masked lanes read 16 zero bytes of the
  // workspace's control block instead of weights.
  const int r0 = urel * (kBlock / kWave) * R + wave * R;
  const int rv = live ? max(0, min(R, rows - r0)) : 0;
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

template <int WT, int TC, int R, int NMAT, int SPC, int NT>
__device__ __forceinline__ void mul_chunk_nt(int kc, int Kpad, int lane, const uint8_t* xs,
                                             const u32x4 (&buf)[NMAT][SPC][R],
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

// all TC staged tokens are multiplied: tokens beyond the tile's count are
// zero in LDS, and a branch on the count would cost the prefetch pipeline
template <int WT, int TC, int R, int NMAT, int SPC>
__device__ __forceinline__ void mul_chunk(int kc, int Kpad, int lane, const uint8_t* xs,
                                          const u32x4 (&buf)[NMAT][SPC][R],
                                          const float (&sc)[NMAT][SPC], float* acc) {
  mul_chunk_nt<WT, TC, R, NMAT, SPC, TC>(kc, Kpad, lane, xs, buf, sc, acc);
}

// tokens of (group, tile) -> LDS [TC][Kpad], zero beyond Kdim and beyond the
// tile; the H row and output row of every token go to LDS too, so the
// epilogue issues no global loads
template <int WT, int TC, bool FROM_H>
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
  for (int v = threadIdx.x; v < TC * vpt; v += kBlock) {
    const int tt = v / vpt;
    const int k = (v - tt * vpt) * EPV;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (tt < nt && k < Kdim) {
      int xrow, hrow;
      float* yrow;
      token_of(p, mt, w.G, w.tile * TC + tt, xrow, hrow, yrow);
      const uint8_t* src = FROM_H ? p.H + static_cast<size_t>(hrow) * Kdim * T::XB
                                  : p.x + static_cast<size_t>(xrow) * Kdim * T::XB;
      val = ld16(src + static_cast<size_t>(k) * T::XB);
    }
    st16(xs + static_cast<size_t>(v) * 16, val);
  }
}

template <int WT, int TC, int R, int NMAT, int SPC>
__device__ __forceinline__ void finish_unit(const FfnParams& p, int nt, int urel, int rows,
                                            int lane, int wave, const int* tok_h,
                                            float* const* tok_y, float* acc) {
  using C = StreamCfg<WT, TC, R, NMAT, SPC>;
  Halve<C::V>::run(acc, lane, 32);
  const int r0 = urel * (kBlock / kWave) * R + wave * R;
  const int rv = max(0, min(R, rows - r0));
  if (NMAT == 2) {
    const float v = __shfl_xor(acc[0], 32);  // the up value pairs with this gate value
    if (lane < 32 && (lane & ((1 << C::SH) - 1)) == 0) {
      const int idx = lane >> C::SH;
      const int r = idx / TC, tt = idx - (idx / TC) * TC;
      if (r < rv && tt < nt) {
        const float a = acc[0];
        const float h = a / (1.0f + expf(-a)) * v;
        const size_t off = static_cast<size_t>(tok_h[tt]) * rows + r0 + r;
        if (WTraits<WT>::XB == 4) {
          reinterpret_cast<float*>(p.H)[off] = h;
        } else {
          reinterpret_cast<uint16_t*>(p.H)[off] = f32_to_bf16_bits(h);
        }
      }
    }
  } else {
    if ((lane & ((1 << C::SH) - 1)) == 0) {
      const int idx = lane >> C::SH;
      const int r = idx / TC, tt = idx - (idx / TC) * TC;
      if (r < rv && tt < nt) tok_y[tt][r0 + r] = acc[0];
    }
  }
#pragma unroll
  for (int i = 0; i < C::V; ++i) acc[i] = 0.0f;
}

template <int WT, int TC, int R, int NMAT, int SPC>
__global__ __launch_bounds__(kBlock) void ffn_stream_kernel(FfnParams p) {
  using C = StreamCfg<WT, TC, R, NMAT, SPC>;
  constexpr bool UP = NMAT == 2;
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
  __shared__ int tok_h[2 * TC];
  __shared__ float* tok_y[2 * TC];
  __shared__ Meta mt;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rows = UP ? p.f : p.d;
  const int Kdim = UP ? p.d : p.f;
  const int nchunks = (Kdim + C::CH - 1) / C::CH;
  const int Kpad = nchunks * C::CH;
  const int upg = (rows + (kBlock / kWave) * R - 1) / ((kBlock / kWave) * R);

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
  if (lo >= hi) return;

  load_meta(p, mt);
  __syncthreads();

  u32x4 b0[NMAT][SPC][R], b1[NMAT][SPC][R];
  float s0[NMAT][SPC], s1[NMAT][SPC];
  float acc[C::V];
#pragma unroll
  for (int i = 0; i < C::V; ++i) acc[i] = 0.0f;

  // Fast path: the range touches at most two groups, each within one token
  // tile, and LDS has two token slots: stage both up front, then stream with
  // no load other than the weights (a load that must be waited for would,
  // with in-order completion, drain the weight prefetch).
  const int g0 = uni(static_cast<int>(lo / upg));
  const int g1 = uni(static_cast<int>((hi - 1) / upg));
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
    const int base0 = g0 * upg;
    const int nct = static_cast<int>(hi - lo) * nchunks;  // chunks of this range
    const size_t slot_bytes = static_cast<size_t>(TC) * Kpad * C::T::XB;
    uint8_t* xs1 = xs + (g1 != g0 ? slot_bytes : 0);
    load_chunk<WT, TC, R, NMAT, SPC>(p, G0, v0, static_cast<int>(lo) - base0, 0, rows, Kdim, lane,
                                     wave, b0, s0);
    {
      Walk w;
      w.G = G0;
      w.tile = 0;
      stage_tokens<WT, TC, !UP>(p, mt, w, Kdim, Kpad, xs, tok_h, tok_y);
      if (g1 != g0) {
        w.G = G1;
        stage_tokens<WT, TC, !UP>(p, mt, w, Kdim, Kpad, xs1, tok_h + TC, tok_y + TC);
      }
    }
    __syncthreads();
    // chunk c: unit lo + c / nchunks, K chunk c % nchunks.  One step
    // prefetches chunk cc + 1 into one buffer and multiplies chunk cc from
    // the other.  The loop runs whole pairs of steps, so on every path back
    // to its head the only loads in flight are the prefetch of the next
    // chunk (a half-finished pair would leave a buffer that the head
    // overwrites in flight, and the compiler would wait for every load there).
    auto step = [&](int cc, u32x4 (&bl)[NMAT][SPC][R], float (&sl)[NMAT][SPC],
                    const u32x4 (&bm)[NMAT][SPC][R], const float (&sm)[NMAT][SPC],
                    bool prefetch) {
      if (prefetch) {
        const int un = static_cast<int>(lo) + (cc + 1) / nchunks;  // unit of the next chunk
        const int kn = (cc + 1) - ((cc + 1) / nchunks) * nchunks;
        const int sn = un - base0 >= upg;  // next chunk in the second group
        load_chunk<WT, TC, R, NMAT, SPC>(p, sn ? G1 : G0, (cc + 1 < nct) && (sn ? v1 : v0),
                                         un - base0 - (sn ? upg : 0), kn, rows, Kdim, lane, wave,
                                         bl, sl);
#ifdef MOE_TUNE_SCHED
        __builtin_amdgcn_sched_barrier(0);
#endif
      }
      const int uc = static_cast<int>(lo) + cc / nchunks;
      const int kcc = cc - (cc / nchunks) * nchunks;
      const int sc_ = uc - base0 >= upg;
      mul_chunk<WT, TC, R, NMAT, SPC>(kcc, Kpad, lane, sc_ ? xs1 : xs, bm, sm, acc);
      if (kcc == nchunks - 1)
        finish_unit<WT, TC, R, NMAT, SPC>(p, sc_ ? G1.cnt : G0.cnt, uc - base0 - (sc_ ? upg : 0),
                                          rows, lane, wave, tok_h + (sc_ ? TC : 0),
                                          tok_y + (sc_ ? TC : 0), acc);
    };
    int c = 0;
    for (; c + 2 <= nct; c += 2) {
      step(c, b1, s1, b0, s0, true);
      step(c + 1, b0, s0, b1, s1, true);
    }
    if (c < nct) step(c, b1, s1, b0, s0, false);  // odd count: the last chunk is in b0
    return;
  }

  // General path: restage tokens at every (group, token tile) change.
  Walk cur;
  cur.done = 0;
  walk_group<TC>(p, mt, U, cur, g0, lo, hi, upg);
  if (UP && !cur.valid && threadIdx.x == 0) atomicOr(p.err, ERRBIT_BAD_IDS);

  load_chunk<WT, TC, R, NMAT, SPC>(p, cur.G, cur.valid, cur.u - cur.g * upg, cur.kc, rows, Kdim,
                                   lane, wave, b0, s0);
  stage_tokens<WT, TC, !UP>(p, mt, cur, Kdim, Kpad, xs, tok_h, tok_y);
  __syncthreads();

  Walk nxt = cur;
  walk_next<TC>(p, mt, U, nxt, nchunks, lo, hi, upg);
  // two chunks per trip so the register buffers keep fixed names
  while (true) {
    load_chunk<WT, TC, R, NMAT, SPC>(p, nxt.G, nxt.valid && !nxt.done, nxt.u - nxt.g * upg, nxt.kc,
                                     rows, Kdim, lane, wave, b1, s1);
    mul_chunk<WT, TC, R, NMAT, SPC>(cur.kc, Kpad, lane, xs, b0, s0, acc);
    if (cur.kc == nchunks - 1)
      finish_unit<WT, TC, R, NMAT, SPC>(p, min(TC, cur.G.cnt - cur.tile * TC), cur.u - cur.g * upg,
                                        rows, lane, wave, tok_h, tok_y, acc);
    if (nxt.done) break;
    if (nxt.g != cur.g || nxt.tile != cur.tile) {
      if (UP && nxt.g != cur.g && !nxt.valid && threadIdx.x == 0) atomicOr(p.err, ERRBIT_BAD_IDS);
      __syncthreads();
      stage_tokens<WT, TC, !UP>(p, mt, nxt, Kdim, Kpad, xs, tok_h, tok_y);
      __syncthreads();
    }
    cur = nxt;
    walk_next<TC>(p, mt, U, nxt, nchunks, lo, hi, upg);

    load_chunk<WT, TC, R, NMAT, SPC>(p, nxt.G, nxt.valid && !nxt.done, nxt.u - nxt.g * upg, nxt.kc,
                                     rows, Kdim, lane, wave, b0, s0);
    mul_chunk<WT, TC, R, NMAT, SPC>(cur.kc, Kpad, lane, xs, b1, s1, acc);
    if (cur.kc == nchunks - 1)
      finish_unit<WT, TC, R, NMAT, SPC>(p, min(TC, cur.G.cnt - cur.tile * TC), cur.u - cur.g * upg,
                                        rows, lane, wave, tok_h, tok_y, acc);
    if (nxt.done) break;
    if (nxt.g != cur.g || nxt.tile != cur.tile) {
      if (UP && nxt.g != cur.g && !nxt.valid && threadIdx.x == 0) atomicOr(p.err, ERRBIT_BAD_IDS);
      __syncthreads();
      stage_tokens<WT, TC, !UP>(p, mt, nxt, Kdim, Kpad, xs, tok_h, tok_y);
      __syncthreads();
    }
    cur = nxt;
    walk_next<TC>(p, mt, U, nxt, nchunks, lo, hi, upg);
  }
}

// ------------------------------------------------------------------ launch
struct OccKey {
  const void* fn;
  size_t smem;
  int dev;
  bool operator<(const OccKey& o) const {
    if (fn != o.fn) return fn < o.fn;
    if (smem != o.smem) return smem < o.smem;
    return dev < o.dev;
  }
};

// resident workgroups of a kernel on the whole device (cached per process)
static int resident_blocks(const void* fn, size_t smem) {
  static std::mutex mu;
  static std::map<OccKey, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> g(mu);
  const OccKey key{fn, smem, dev};
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kBlock, smem) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  const int total = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
  cache[key] = total;
  return total;
}

template <int WT, int TC, int R, int NMAT, int SPC>
static hipError_t launch_phase(const FfnParams& p, hipStream_t s) {
  using C = StreamCfg<WT, TC, R, NMAT, SPC>;
  constexpr bool UP = NMAT == 2;
  const int rows = UP ? p.f : p.d;
  const int Kdim = UP ? p.d : p.f;
  const int Kpad = (Kdim + C::CH - 1) / C::CH * C::CH;
  const void* fn = reinterpret_cast<const void*>(&ffn_stream_kernel<WT, TC, R, NMAT, SPC>);
  // A second token slot lets ranges that cross a group boundary take the
  // fast path; it is used only when it costs no resident workgroups.
  const size_t slot = static_cast<size_t>(TC) * Kpad * C::T::XB;
#ifndef MOE_TUNE_SLOTS
  const int slots =
      2 * slot <= 65536 && resident_blocks(fn, 2 * slot) >= resident_blocks(fn, slot) ? 2 : 1;
#else
  const int slots = MOE_TUNE_SLOTS;
#endif
  const size_t smem = slots * slot;
  FfnParams q = p;
  q.lds_slots = slots;
  const int upg = (rows + (kBlock / kWave) * R - 1) / ((kBlock / kWave) * R);
  const int groups_max = p.mode == MODE_DEDUP ? p.ucap + p.S : p.n * (p.K + p.S);
  const long long units_max = static_cast<long long>(groups_max) * upg;
  long long grid = resident_blocks(fn, smem);
  if (grid <= 0) return hipErrorInvalidConfiguration;
#ifdef MOE_TUNE_MAXBPC
  if (grid > 256LL * MOE_TUNE_MAXBPC) grid = 256LL * MOE_TUNE_MAXBPC;
#endif
  if (grid > units_max) grid = units_max;
  hipLaunchKernelGGL((ffn_stream_kernel<WT, TC, R, NMAT, SPC>), dim3(static_cast<unsigned>(grid)),
                     dim3(kBlock), smem, s, q);
  return hipGetLastError();
}

// Tile shape knobs (rows per wave R, load steps per chunk SPC) of the up and
// down kernels; the defaults are the measured best on MI355X.
#ifndef MOE_TUNE_RU
#define MOE_TUNE_RU 2
#endif
#ifndef MOE_TUNE_SPCU
#define MOE_TUNE_SPCU 2
#endif
#ifndef MOE_TUNE_RD
#define MOE_TUNE_RD 4
#endif
#ifndef MOE_TUNE_SPCD
#define MOE_TUNE_SPCD 2
#endif

template <int WT, int TC>
static hipError_t launch_pair(const FfnParams& p, hipStream_t s) {
  // up: R rows of W_gate and W_up per wave; down: R rows of W_down per wave.
  // fp8 (d = 7168): the up phase stages at most 4 tokens (56 KB of LDS)
  constexpr int RU = WT == WT_FP8 ? 4 : MOE_TUNE_RU;
  constexpr int SPCU = WT == WT_FP8 ? 1 : MOE_TUNE_SPCU;
  constexpr int RD = MOE_TUNE_RD;
  constexpr int SPCD = WT == WT_FP8 ? 1 : MOE_TUNE_SPCD;
  constexpr int TCU = (WT == WT_FP8 && TC > 4) ? 4 : TC;
  hipError_t e = launch_phase<WT, TCU, RU, 2, SPCU>(p, s);
  if (e != hipSuccess) return e;
  return launch_phase<WT, TC, RD, 1, SPCD>(p, s);
}

// token tile: a group serves at most n tokens (a token names an expert once),
// so the tile is the next power of two of min(n, 8); larger groups (shared
// experts of a long pass, trees) take several tiles
static int token_tile(const FfnParams& p) {
  if (p.mode == MODE_PERSLOT) return 1;
  const int n = p.n;
  return n >= 5 ? 8 : (n >= 3 ? 4 : (n == 2 ? 2 : 1));
}

template <int WT>
static hipError_t launch_typed(const FfnParams& p, hipStream_t s) {
  switch (token_tile(p)) {
    case 1: return launch_pair<WT, 1>(p, s);
    case 2: return launch_pair<WT, 2>(p, s);
    case 4: return launch_pair<WT, 4>(p, s);
    default: return launch_pair<WT, 8>(p, s);
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
