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

__device__ __forceinline__ bool group_of(const FfnParams& p, int g, Group& G, bool report) {
  if (p.mode == MODE_DEDUP) {
    if (g < p.ucap) {
      const int U = *p.U;
      if (U < 0) {
        if (report) atomicOr(p.err, ERRBIT_BAD_IDS);
        return false;
      }
      if (g >= U) return false;
      G.e = p.union_ids[g];
      G.shared = 0;
      G.first = p.offsets[g];
      G.cnt = p.offsets[g + 1] - G.first;
      G.s_idx = 0;
      return G.cnt > 0;
    }
    const int s = g - p.ucap;
    if (s >= p.S) return false;
    G.e = s;
    G.shared = 1;
    G.first = 0;
    G.cnt = p.n;
    G.s_idx = s;
    return true;
  }
  const int nk = p.n * p.K;
  if (g < nk) {
    G.e = p.ids[g];
    G.shared = 0;
    G.first = g;
    G.cnt = 1;
    G.s_idx = 0;
    return true;
  }
  const int q = g - nk;
  if (q >= p.n * p.S) return false;
  G.e = q % p.S;
  G.shared = 1;
  G.first = q;
  G.cnt = 1;
  G.s_idx = q;
  return true;
}

// token j of a group: its row in x, its row in H and its output row
__device__ __forceinline__ void token_of(const FfnParams& p, const Group& G, int j, int& xrow,
                                         int& hrow, float*& yrow) {
  const int nk = p.n * p.K;
  if (p.mode == MODE_DEDUP) {
    if (!G.shared) {
      const int slot = p.perm[G.first + j];
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

// ------------------------------------------------------------- main tile
// Wave-level product of R stored rows of NMAT matrices (each Kdim long) with
// up to TC token vectors staged chunk by chunk in LDS.  acc[(m*R + r)*TC + tt].
// All waves of the workgroup must call it together (it holds barriers).
template <int WT, int TC, int R, int NMAT, bool FROM_H>
__device__ __forceinline__ void rows_times_tokens(
    const FfnParams& p, const Group& G, int tile, int nt, const uint8_t* const (&Wrow)[NMAT],
    const float* const (&Srow)[NMAT], int rv, int Kdim, uint8_t* xs, float* acc) {
  using T = WTraits<WT>;
  constexpr int STEP = kWave * T::VEC;
  constexpr int KC = T::SPC * STEP;
  constexpr int VPT = KC * T::XB / 16;  // 16-byte vectors per staged token chunk
  const int lane = threadIdx.x & 63;
  const size_t row_bytes = static_cast<size_t>(Kdim) * T::EB;

#pragma unroll
  for (int i = 0; i < NMAT * R * TC; ++i) acc[i] = 0.0f;

  for (int kc = 0; kc < Kdim; kc += KC) {
    // weights of this chunk first, so their latency overlaps the staging
    u32x4 wv[NMAT][T::SPC][R];
    float sc[NMAT][T::SPC];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
#pragma unroll
      for (int s = 0; s < T::SPC; ++s) {
        const int k = kc + s * STEP + lane * T::VEC;
        const bool kin = k < Kdim;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          wv[m][s][r] = (kin && r < rv)
                            ? ld16(Wrow[m] + static_cast<size_t>(r) * row_bytes +
                                   static_cast<size_t>(k) * T::EB)
                            : u32x4{0u, 0u, 0u, 0u};
        }
        sc[m][s] = (WT == WT_FP8 && kin && rv > 0) ? Srow[m][k >> 7] : 0.0f;
      }
    }
    __syncthreads();  // everyone is done reading the previous chunk
    for (int v = threadIdx.x; v < TC * VPT; v += kBlock) {
      const int tt = v / VPT;
      const int c = v - tt * VPT;
      const int k = kc + c * (16 / T::XB);
      u32x4 val = {0u, 0u, 0u, 0u};
      if (tt < nt && k < Kdim) {
        int xrow, hrow;
        float* yrow;
        token_of(p, G, tile + tt, xrow, hrow, yrow);
        const uint8_t* src = FROM_H ? p.H + static_cast<size_t>(hrow) * Kdim * T::XB
                                    : p.x + static_cast<size_t>(xrow) * Kdim * T::XB;
        val = ld16(src + static_cast<size_t>(k) * T::XB);
      }
      st16(xs + static_cast<size_t>(tt) * KC * T::XB + c * 16, val);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < T::SPC; ++s) {
      const int kl = s * STEP + lane * T::VEC;  // element offset within the chunk
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const typename Dot<WT>::W w = Dot<WT>::prep(wv[m][s][r]);
#pragma unroll
          for (int tt = 0; tt < TC; ++tt) {
            if (tt < nt) {
              const uint8_t* xp = xs + (static_cast<size_t>(tt) * KC + kl) * T::XB;
              float& a = acc[(m * R + r) * TC + tt];
              a = Dot<WT>::run(w, xp, a, sc[m][s]);
            }
          }
        }
      }
    }
  }
}

// -------------------------------------------------------------- kernel 1
// grid.x: blocks of 4*R intermediate rows j; grid.y: groups.
template <int WT, int TC, int R>
__global__ __launch_bounds__(kBlock) void ffn_up_kernel(FfnParams p) {
  using T = WTraits<WT>;
  constexpr int KC = T::SPC * kWave * T::VEC;
  constexpr int V = 2 * R * TC;
  static_assert((V & (V - 1)) == 0 && V <= 64, "values per lane must be a power of two <= 64");
  __shared__ __attribute__((aligned(16))) uint8_t xs[TC * KC * T::XB];
  __shared__ float red[kBlock / kWave][V];

  Group G;
  if (!group_of(p, blockIdx.y, G, blockIdx.x == 0 && threadIdx.x == 0)) return;
  if (!G.shared && (G.e < 0 || G.e >= p.E)) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(p.err, ERRBIT_BAD_IDS);
    return;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rows = p.f, Kdim = p.d;
  const int r0 = (blockIdx.x * (kBlock / kWave) + wave) * R;
  const int rv = max(0, min(R, rows - r0));
  const size_t mat = static_cast<size_t>(rows) * Kdim * T::EB;
  const size_t row_bytes = static_cast<size_t>(Kdim) * T::EB;
  const uint8_t* w0 = G.shared ? p.shw[0] : p.w[0];
  const uint8_t* w1 = G.shared ? p.shw[1] : p.w[1];
  const uint8_t* const Wrow[2] = {
      w0 + static_cast<size_t>(G.e) * mat + static_cast<size_t>(r0) * row_bytes,
      w1 + static_cast<size_t>(G.e) * mat + static_cast<size_t>(r0) * row_bytes};
  const int kb = Kdim / 128;
  const size_t sexp = static_cast<size_t>(rows / 128) * kb;
  const size_t soff = static_cast<size_t>(G.e) * sexp + static_cast<size_t>(r0 / 128) * kb;
  const float* const Srow[2] = {
      WT == WT_FP8 ? (G.shared ? p.shs[0] : p.s[0]) + soff : nullptr,
      WT == WT_FP8 ? (G.shared ? p.shs[1] : p.s[1]) + soff : nullptr};

  for (int tile = 0; tile < G.cnt; tile += TC) {
    const int nt = min(TC, G.cnt - tile);
    float acc[V];
    rows_times_tokens<WT, TC, R, 2, false>(p, G, tile, nt, Wrow, Srow, rv, Kdim, xs, acc);
    Halve<V>::run(acc, lane, 32);
    constexpr int SH = 6 - ilog2(V);
    if ((lane & ((1 << SH) - 1)) == 0) red[wave][lane >> SH] = acc[0];
    __syncthreads();
    if (lane < R * TC) {
      const int r = lane / TC, tt = lane - (lane / TC) * TC;
      if (r < rv && tt < nt) {
        const float a = red[wave][(0 * R + r) * TC + tt];
        const float v = red[wave][(1 * R + r) * TC + tt];
        const float h = a / (1.0f + expf(-a)) * v;
        int xrow, hrow;
        float* yrow;
        token_of(p, G, tile + tt, xrow, hrow, yrow);
        const size_t off = static_cast<size_t>(hrow) * rows + r0 + r;
        if (T::XB == 4) {
          reinterpret_cast<float*>(p.H)[off] = h;
        } else {
          reinterpret_cast<uint16_t*>(p.H)[off] = f32_to_bf16_bits(h);
        }
      }
    }
    // the next tile's first barrier orders red[] reuse
  }
}

// -------------------------------------------------------------- kernel 2
// grid.x: blocks of 4*R output rows c; grid.y: groups.
template <int WT, int TC, int R>
__global__ __launch_bounds__(kBlock) void ffn_down_kernel(FfnParams p) {
  using T = WTraits<WT>;
  constexpr int KC = T::SPC * kWave * T::VEC;
  constexpr int V = R * TC;
  static_assert((V & (V - 1)) == 0 && V <= 64, "values per lane must be a power of two <= 64");
  __shared__ __attribute__((aligned(16))) uint8_t xs[TC * KC * T::XB];
  __shared__ float red[kBlock / kWave][V];

  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0 && p.bytes != nullptr) {
    const unsigned long long req =
        static_cast<unsigned long long>(p.n) * (p.K + p.S) * p.expert_bytes;
    unsigned long long got = req;
    if (p.mode == MODE_DEDUP) {
      const int U = *p.U;
      got = U < 0 ? 0ull : static_cast<unsigned long long>(U + p.S) * p.expert_bytes;
    }
    p.bytes[0] = got;
    p.bytes[1] = req;
  }

  Group G;
  if (!group_of(p, blockIdx.y, G, false)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rows = p.d, Kdim = p.f;
  const int r0 = (blockIdx.x * (kBlock / kWave) + wave) * R;
  const int rv = max(0, min(R, rows - r0));
  if (!G.shared && (G.e < 0 || G.e >= p.E)) {
    // per-slot slot with an invalid id: defined zero output
    int xrow, hrow;
    float* yrow;
    token_of(p, G, 0, xrow, hrow, yrow);
    if (lane < rv) yrow[r0 + lane] = 0.0f;
    return;
  }
  const size_t mat = static_cast<size_t>(rows) * Kdim * T::EB;
  const size_t row_bytes = static_cast<size_t>(Kdim) * T::EB;
  const uint8_t* w2 = G.shared ? p.shw[2] : p.w[2];
  const uint8_t* const Wrow[1] = {w2 + static_cast<size_t>(G.e) * mat +
                                  static_cast<size_t>(r0) * row_bytes};
  const int kb = Kdim / 128;
  const size_t sexp = static_cast<size_t>(rows / 128) * kb;
  const size_t soff = static_cast<size_t>(G.e) * sexp + static_cast<size_t>(r0 / 128) * kb;
  const float* const Srow[1] = {WT == WT_FP8 ? (G.shared ? p.shs[2] : p.s[2]) + soff : nullptr};

  for (int tile = 0; tile < G.cnt; tile += TC) {
    const int nt = min(TC, G.cnt - tile);
    float acc[V];
    rows_times_tokens<WT, TC, R, 1, true>(p, G, tile, nt, Wrow, Srow, rv, Kdim, xs, acc);
    Halve<V>::run(acc, lane, 32);
    constexpr int SH = 6 - ilog2(V);
    if ((lane & ((1 << SH) - 1)) == 0) red[wave][lane >> SH] = acc[0];
    __syncthreads();
    if (lane < R * TC) {
      const int r = lane / TC, tt = lane - (lane / TC) * TC;
      if (r < rv && tt < nt) {
        int xrow, hrow;
        float* yrow;
        token_of(p, G, tile + tt, xrow, hrow, yrow);
        yrow[r0 + r] = red[wave][r * TC + tt];
      }
    }
  }
}

// ------------------------------------------------------------------ launch
template <int WT, int TC>
static hipError_t launch_typed(const FfnParams& p, hipStream_t s) {
  constexpr int R_UP = 2, R_DOWN = 4;
  const int groups = p.mode == MODE_DEDUP ? p.ucap + p.S : p.n * (p.K + p.S);
  const int rows_up = (kBlock / kWave) * R_UP;
  const int rows_down = (kBlock / kWave) * R_DOWN;
  dim3 g1((p.f + rows_up - 1) / rows_up, groups);
  dim3 g2((p.d + rows_down - 1) / rows_down, groups);
  hipLaunchKernelGGL((ffn_up_kernel<WT, TC, R_UP>), g1, dim3(kBlock), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((ffn_down_kernel<WT, TC, R_DOWN>), g2, dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_expert_ffn(const FfnParams& p, int w_dtype, hipStream_t s) {
  const bool dedup = p.mode == MODE_DEDUP;
  switch (w_dtype) {
    case WT_F32:
      return dedup ? launch_typed<WT_F32, 8>(p, s) : launch_typed<WT_F32, 1>(p, s);
    case WT_BF16:
      return dedup ? launch_typed<WT_BF16, 8>(p, s) : launch_typed<WT_BF16, 1>(p, s);
    case WT_FP8:
      return dedup ? launch_typed<WT_FP8, 8>(p, s) : launch_typed<WT_FP8, 1>(p, s);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace moe
