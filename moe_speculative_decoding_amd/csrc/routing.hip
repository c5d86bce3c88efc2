// Router top-K and expert union for one verify pass (gfx950).
//
// Top-K: "Making Every Verified Token Count: Adaptive Verification for MoE
// Speculative Decoding", Sec. 2.2, Eq. (4) — the indices of the K largest
// router scores, normalised (softmax over the K here).
// Union: "Less Experts, Faster Decoding", Sec. 3, Eq. (1), and the same page
// family's Eq. (5) / (A2): the distinct experts of all verified tokens; the
// slot permutation sorts rows by expert as the MLX-LM deduplicating engine
// does (expert-bytes page, Table 6).
//
// Both are integer-exact: top-K compares 64-bit keys built from the fp32
// bit pattern (no float arithmetic decides a selection), and the union uses
// an LDS histogram per wavefront, ballot scans and a ballot-based match of
// equal ids, so every output is deterministic.
#include "common.h"

namespace moe {

// ------------------------------------------------------------------ top-K
// Key order = (logit descending, id ascending); NaN below every number,
// -0.0 equal to +0.0.  The 32-bit key orders the values: every number maps
// above 1, NaN maps to 1 and 0 marks an entry that is absent (beyond E) or
// already taken; equal keys are split by the id afterwards.
__device__ __forceinline__ unsigned topk_key(float v) {
  unsigned b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0u;                     // -0.0 -> +0.0
  if ((b & 0x7fffffffu) > 0x7f800000u) return 1u;  // NaN
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);  // -inf -> 0x007fffff
}

// Cross-lane moves inside rows of 16 lanes (DPP): no LDS round trip.
template <int CTRL>
__device__ __forceinline__ unsigned dpp(unsigned v) {
  return static_cast<unsigned>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// maximum over the wavefront, returned in a scalar register
__device__ __forceinline__ unsigned wave_max_u32(unsigned v) {
  v = max(v, dpp<kDppQuadXor1>(v));
  v = max(v, dpp<kDppQuadXor2>(v));
  v = max(v, dpp<kDppHalfMirror>(v));  // max over 8 lanes
  v = max(v, dpp<kDppMirror>(v));      // max over the row of 16
  const unsigned a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const unsigned c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

// inclusive prefix sum over the wavefront: Hillis-Steele inside each row of
// 16 lanes, then the row totals added in from scalar registers
__device__ __forceinline__ int wave_inclusive_sum(int v, int lane) {
  unsigned u = static_cast<unsigned>(v);
  u += dpp<0x111>(u);  // row_shr:1 (lanes shifted in from outside the row read 0)
  u += dpp<0x112>(u);  // row_shr:2
  u += dpp<0x114>(u);  // row_shr:4
  u += dpp<0x118>(u);  // row_shr:8
  const unsigned r0 = __builtin_amdgcn_readlane(u, 15);
  const unsigned r1 = __builtin_amdgcn_readlane(u, 31);
  const unsigned r2 = __builtin_amdgcn_readlane(u, 47);
  u += (lane >= 16 ? r0 : 0u) + (lane >= 32 ? r1 : 0u) + (lane >= 48 ? r2 : 0u);
  return static_cast<int>(u);
}

// One wavefront routes one token; lane l holds the logits of experts
// l, l+64, l+128, l+192 (E <= 256).  Lane k (< K) ends with the k-th selected
// id and its gate.  Each of the K rounds takes the wavefront maximum of the
// lanes' best remaining keys, then the lowest id holding it (id = l + 64 j,
// so the lowest j first, then the lowest lane).
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int K, int lane,
                                            int& my_id, float& my_gate) {
  float val[4];
  unsigned key[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + kWave * j;
    val[j] = (e < E) ? row[e] : 0.0f;
    key[j] = (e < E) ? topk_key(val[j]) : 0u;
  }
  int sel_id[8];
  float sel_l[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    sel_id[k] = 0;
    sel_l[k] = 0.0f;
    if (k < K) {
      unsigned best = 0u;
      int bj = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (key[j] > best) {  // strict: the lowest j keeps a tie
          best = key[j];
          bj = j;
        }
      }
      const unsigned M = wave_max_u32(best);
      int e = 0;
      const bool hit = best == M;
#pragma unroll
      for (int j = 3; j >= 0; --j) {  // the lowest j with a hit wins
        const unsigned long long m = __ballot(hit && bj == j);
        if (m != 0ull) e = j * kWave + static_cast<int>(__builtin_ctzll(m));
      }
      e = __builtin_amdgcn_readfirstlane(e);
      const int ej = e >> 6, el = e & 63;
      const float lv = ej == 0 ? val[0] : (ej == 1 ? val[1] : (ej == 2 ? val[2] : val[3]));
      sel_l[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), el));
      sel_id[k] = e;
      if (lane == el) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (j == ej) key[j] = 0u;
      }
    }
  }
  // softmax over the selected logits; the first selection holds the maximum
  const float top = sel_l[0];
  float sum = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (k < K) sum += expf(sel_l[k] - top);
  my_id = 0;
  float l = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (lane == k) {
      my_id = sel_id[k];
      l = sel_l[k];
    }
  my_gate = expf(l - top) / sum;
}

__global__ __launch_bounds__(kBlock) void route_topk_kernel(const float* __restrict__ logits,
                                                            int n, int E, int K,
                                                            int32_t* __restrict__ ids,
                                                            float* __restrict__ gates) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kBlock / kWave) + wave;
  if (t >= n) return;  // wave-uniform
  int id;
  float g;
  route_token(logits + static_cast<size_t>(t) * E, E, K, lane, id, g);
  if (lane < K) {
    ids[static_cast<size_t>(t) * K + lane] = id;
    gates[static_cast<size_t>(t) * K + lane] = g;
  }
}

hipError_t launch_route_topk(const float* logits, int n, int E, int K, int32_t* ids,
                             float* gates, hipStream_t s) {
  const int per_block = kBlock / kWave;
  dim3 grid((n + per_block - 1) / per_block);
  hipLaunchKernelGGL(route_topk_kernel, grid, dim3(kBlock), 0, s, logits, n, E, K, ids, gates);
  return hipGetLastError();
}

// ------------------------------------------------------------------ union
// Lanes 0..255 of the workgroup: lane s owns slot s (n*K <= 256) and expert
// e = s (E <= 256).  `ids` may point to LDS or global memory.
struct UnionLds {
  int wcnt[4][256];  // per-wave histogram of ids
  int rank_of[256];  // expert -> union position
  int start_of[256]; // expert -> first position in perm
  int wtot_present[4];
  int wtot_count[4];
  int bad;
};

// Every thread of the workgroup calls this (it holds __syncthreads); threads
// 0..255 do the work.
__device__ __forceinline__ void build_union_256(const int32_t* ids, int n, int K, int E,
                                                int32_t* __restrict__ U_out,
                                                int32_t* __restrict__ union_ids,
                                                int32_t* __restrict__ offsets,
                                                int32_t* __restrict__ perm,
                                                int32_t* __restrict__ slot_rank, UnionLds& sh) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool mine = tid < 256;
  const int nk = n * K;
  const int cap = nk < E ? nk : E;
  for (int i = tid; i < 4 * 256; i += blockDim.x) (&sh.wcnt[0][0])[i] = 0;
  if (tid == 0) sh.bad = 0;
  __syncthreads();

  const bool act = tid < nk;  // nk <= 256
  const int id = act ? ids[tid] : 0;
  if (act) {
    if (id < 0 || id >= E) {
      atomicOr(&sh.bad, 1);
    } else {
      atomicAdd(&sh.wcnt[wave][id], 1);
    }
  }
  __syncthreads();
  if (sh.bad) {  // uniform
    if (tid == 0) *U_out = -1;
    return;
  }

  // exclusive scans over experts e = tid of "present" and of the slot count
  const int e = tid;
  int c = 0;
  if (e < E) c = sh.wcnt[0][e] + sh.wcnt[1][e] + sh.wcnt[2][e] + sh.wcnt[3][e];
  const int pres = (e < E && c > 0) ? 1 : 0;
  const unsigned long long pmask = __ballot(pres);
  const int pre_present = __popcll(pmask & ((1ull << lane) - 1ull));
  const int inc = wave_inclusive_sum(c, lane);
  if (mine && lane == kWave - 1) {
    sh.wtot_present[wave] = __popcll(pmask);
    sh.wtot_count[wave] = inc;
  }
  __syncthreads();
  int base_p = 0, base_c = 0, Utot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave) {
      base_p += sh.wtot_present[w];
      base_c += sh.wtot_count[w];
    }
    Utot += sh.wtot_present[w];
  }
  const int rank = base_p + pre_present;
  const int start = base_c + inc - c;
  if (mine) {
    sh.rank_of[e] = rank;
    sh.start_of[e] = start;
  }
  if (pres) {
    union_ids[rank] = e;
    offsets[rank] = start;
  }
  if (mine) {
    for (int i = Utot + tid; i < cap; i += 256) union_ids[i] = -1;
    for (int i = Utot + tid; i <= cap; i += 256) offsets[i] = nk;
  }
  if (tid == 0) *U_out = Utot;
  __syncthreads();

  // stable position of slot tid among the slots of its expert:
  // slots of earlier waves (histograms) + earlier lanes of this wave with the
  // same id (8 ballots over the id bits, ids < 256)
  unsigned long long same = __ballot(act);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int bit = (id >> b) & 1;
    const unsigned long long ones = __ballot(act && bit);
    same &= bit ? ones : ~ones;
  }
  if (act) {
    int before = 0;
    for (int w = 0; w < wave; ++w) before += sh.wcnt[w][id];
    const int pos = sh.start_of[id] + before + __popcll(same & ((1ull << lane) - 1ull));
    perm[pos] = tid;
    slot_rank[tid] = sh.rank_of[id];
  }
}

__global__ __launch_bounds__(kBlock) void build_union_kernel(
    const int32_t* __restrict__ ids, int n, int K, int E, int32_t* __restrict__ U_out,
    int32_t* __restrict__ union_ids, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ slot_rank) {
  __shared__ UnionLds sh;
  build_union_256(ids, n, K, E, U_out, union_ids, offsets, perm, slot_rank, sh);
}

// Route every token (one wavefront each, 16 wavefronts) into LDS, then build
// the union from LDS: one launch for both steps of the pass.
constexpr int kRouteUnionBlock = 1024;

__global__ __launch_bounds__(kRouteUnionBlock) void route_union_kernel(
    const float* __restrict__ logits, int n, int E, int K, int32_t* __restrict__ ids,
    float* __restrict__ gates, int32_t* __restrict__ U_out, int32_t* __restrict__ union_ids,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ slot_rank) {
  __shared__ int32_t ids_lds[256];
  __shared__ UnionLds sh;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int t = wave; t < n; t += kRouteUnionBlock / kWave) {
    int id;
    float g;
    route_token(logits + static_cast<size_t>(t) * E, E, K, lane, id, g);
    if (lane < K) {
      ids[static_cast<size_t>(t) * K + lane] = id;
      gates[static_cast<size_t>(t) * K + lane] = g;
      ids_lds[t * K + lane] = id;
    }
  }
  __syncthreads();
  build_union_256(ids_lds, n, K, E, U_out, union_ids, offsets, perm, slot_rank, sh);
}

hipError_t launch_route_union(const float* logits, int n, int E, int K, int32_t* ids,
                              float* gates, int32_t* U, int32_t* union_ids, int32_t* offsets,
                              int32_t* perm, int32_t* slot_rank, hipStream_t s) {
  hipLaunchKernelGGL(route_union_kernel, dim3(1), dim3(kRouteUnionBlock), 0, s, logits, n, E, K,
                     ids, gates, U, union_ids, offsets, perm, slot_rank);
  return hipGetLastError();
}

hipError_t launch_build_union(const int32_t* ids, int n, int K, int E, int32_t* U,
                              int32_t* union_ids, int32_t* offsets, int32_t* perm,
                              int32_t* slot_rank, hipStream_t s) {
  hipLaunchKernelGGL(build_union_kernel, dim3(1), dim3(kBlock), 0, s, ids, n, K, E, U, union_ids,
                     offsets, perm, slot_rank);
  return hipGetLastError();
}

}  // namespace moe
