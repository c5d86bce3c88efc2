// Router top-K and expert union of one verify pass: device functions shared
// by the routing kernels and the one-launch layer pass (gfx950).
//
// Top-K: "Making Every Verified Token Count: Adaptive Verification for MoE
// Speculative Decoding", Sec. 2.2, Eq. (4) — the indices of the K largest
// router scores, normalised (softmax over the K here).
// Union: "Less Experts, Faster Decoding", Sec. 3, Eq. (1), and the same page
// family's Eq. (5) / (A2): the distinct experts of all verified tokens; the
// slot permutation sorts rows by expert as the MLX-LM deduplicating engine
// does (expert-bytes page, Table 6).
//
// Both are integer-exact: top-K compares integer keys built from the fp32
// bit pattern (no float arithmetic decides a selection) with DPP maxima
// inside rows of 16 lanes and splits equal keys by the lowest id, and the
// union uses an LDS
// histogram per wavefront, DPP prefix sums and a ballot-based match of equal
// ids, so every output is deterministic.
#pragma once

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

// reductions over each row of 16 lanes; every lane of the row ends with it
__device__ __forceinline__ unsigned row_max_u32(unsigned v) {
  v = max(v, dpp<kDppQuadXor1>(v));
  v = max(v, dpp<kDppQuadXor2>(v));
  v = max(v, dpp<kDppHalfMirror>(v));  // 8 lanes
  return max(v, dpp<kDppMirror>(v));   // 16 lanes
}
__device__ __forceinline__ unsigned row_min_u32(unsigned v) {
  v = min(v, dpp<kDppQuadXor1>(v));
  v = min(v, dpp<kDppQuadXor2>(v));
  v = min(v, dpp<kDppHalfMirror>(v));
  return min(v, dpp<kDppMirror>(v));
}
__device__ __forceinline__ float row_sum_f32(float v) {
  v += __uint_as_float(dpp<kDppQuadXor1>(__float_as_uint(v)));
  v += __uint_as_float(dpp<kDppQuadXor2>(__float_as_uint(v)));
  v += __uint_as_float(dpp<kDppHalfMirror>(__float_as_uint(v)));
  return v + __uint_as_float(dpp<kDppMirror>(__float_as_uint(v)));
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

// Per-wavefront LDS scratch of the top-K (the rank loop serves up to 64
// experts; more take route_token_rounds, which keeps its keys in registers).
struct TopkLds {
  unsigned long long key[kWave];  // 64-bit keys of the token's experts (0 beyond E)
  int part[kWave];                // a team member's partial ranks (route_team_*)
  int sel_id[8];
  float sel_l[8];
};

// One wavefront routes one token (`row` in LDS or global memory) of at most
// 64 experts; lane l holds expert l (J = 1).  Every expert
// gets a 64-bit key (32-bit value key, then 255 - id, so a larger key is a
// larger logit or, for equal logits, a lower id), and its rank is the number
// of keys above it: the experts of rank < K are the top K, in order.  All
// comparisons are independent (no chain of K dependent rounds), and the keys
// are read back from LDS as broadcasts.  Lane k (< K) ends with the k-th
// selected id and its gate: the softmax over the K selected logits, whose
// first selection holds the maximum.
template <int J>
__device__ __forceinline__ void topk_keys(const float* __restrict__ row, int E, int lane,
                                          TopkLds& sc, float (&val)[J],
                                          unsigned long long (&key)[J]) {
#pragma unroll
  for (int j = 0; j < J; ++j) val[j] = row[min(lane + kWave * j, E - 1)];  // all loads first
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + kWave * j;
    key[j] = e < E ? (static_cast<unsigned long long>(topk_key(val[j])) << 8) |
                         static_cast<unsigned>(255 - e)
                   : 0ull;
    sc.key[e] = key[j];
  }
  __builtin_amdgcn_wave_barrier();  // LDS ops of one wavefront run in order
}

// rank[j] += the keys of sc.key[i0 .. i1) above key[j] (i0, i1 multiples of 16)
template <int J>
__device__ __forceinline__ void topk_count(const TopkLds& sc, int i0, int i1,
                                           const unsigned long long (&key)[J], int (&rank)[J]) {
#pragma unroll 1
  for (int i = i0; i < i1; i += 16) {
    // eight broadcast reads (the same address in every lane) in flight at once
    u32x4 kk[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) kk[q] = ld16(&sc.key[i + 2 * q]);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const unsigned long long k0 = (static_cast<unsigned long long>(kk[q].y) << 32) | kk[q].x;
      const unsigned long long k1 = (static_cast<unsigned long long>(kk[q].w) << 32) | kk[q].z;
#pragma unroll
      for (int j = 0; j < J; ++j) rank[j] += (k0 > key[j]) + (k1 > key[j]);
    }
  }
}

// lane k (< K) takes the k-th selection of sc.sel_id / sc.sel_l and its gate:
// the softmax over the K selected logits, whose first selection holds the
// maximum
__device__ __forceinline__ void topk_finish(int K, int lane, TopkLds& sc, int& my_id,
                                            float& my_gate) {
  __builtin_amdgcn_wave_barrier();
  my_id = lane < K ? sc.sel_id[lane] : 0;
  const float top = sc.sel_l[0];
  const float l = lane < K ? sc.sel_l[lane] : top;
  const float ex = lane < K ? expf(l - top) : 0.0f;
  // lanes 0..K-1 are all in the first row of 16: its DPP sum is the total
  my_gate = ex / row_sum_f32(ex);
  __builtin_amdgcn_wave_barrier();  // the scratch may be reused by the next token
}

// the experts of rank < K in rank order, and lane k's gate
template <int J>
__device__ __forceinline__ void topk_select(const float (&val)[J], const int (&rank)[J], int E,
                                            int K, int lane, TopkLds& sc, int& my_id,
                                            float& my_gate) {
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + kWave * j;
    if (e < E && rank[j] < K) {
      sc.sel_id[rank[j]] = e;
      sc.sel_l[rank[j]] = val[j];
    }
  }
  topk_finish(K, lane, sc, my_id, my_gate);
}

// The same selection by K rounds of a wavefront-wide maximum, for more than
// 64 experts: ranking every key costs E*E/64 comparisons per lane (the
// routing of a 256-expert layer then takes microseconds), K rounds cost
// K*(E/64 + a dozen cross-lane steps).  Round k takes the largest remaining
// 32-bit value key and, among the experts holding it, the lowest id: the
// expert the rank loop ranks k-th.  Lane l holds experts l, l+64, ...
template <int J>
__device__ __forceinline__ void route_token_rounds(const float* __restrict__ row, int E, int K,
                                                   int lane, TopkLds& sc, int& my_id,
                                                   float& my_gate) {
  float val[J];
  unsigned vk[J];
#pragma unroll
  for (int j = 0; j < J; ++j) val[j] = row[min(lane + kWave * j, E - 1)];  // all loads first
#pragma unroll
  for (int j = 0; j < J; ++j) vk[j] = lane + kWave * j < E ? topk_key(val[j]) : 0u;
  for (int k = 0; k < K; ++k) {
    unsigned m = vk[0];
#pragma unroll
    for (int j = 1; j < J; ++j) m = max(m, vk[j]);
    m = row_max_u32(m);
    const unsigned top =
        max(max(static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(m), 0)),
                static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(m), 16))),
            max(static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(m), 32)),
                static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(m), 48))));
    unsigned cand = 0xFFFFu;  // this lane's lowest expert holding the top key
#pragma unroll
    for (int j = J - 1; j >= 0; --j)
      if (vk[j] == top) cand = static_cast<unsigned>(lane + kWave * j);
    cand = row_min_u32(cand);
    const unsigned id =
        min(min(static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(cand), 0)),
                static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(cand), 16))),
            min(static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(cand), 32)),
                static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(cand), 48))));
    if (lane == static_cast<int>(id & 63u)) {
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (j == static_cast<int>(id >> 6)) {
          vk[j] = 0u;  // taken
          sc.sel_id[k] = static_cast<int>(id);
          sc.sel_l[k] = val[j];
        }
    }
  }
  topk_finish(K, lane, sc, my_id, my_gate);
}

// up to 64 experts: lane l holds expert l
__device__ __forceinline__ void route_token_rank(const float* __restrict__ row, int E, int K,
                                                 int lane, TopkLds& sc, int& my_id,
                                                 float& my_gate) {
  float val[1];
  unsigned long long key[1];
  topk_keys<1>(row, E, lane, sc, val, key);
  int rank[1] = {0};
  topk_count<1>(sc, 0, kWave, key, rank);
  topk_select<1>(val, rank, E, K, lane, sc, my_id, my_gate);
}

// up to 64 experts: rank every key (one comparison per key and lane); more:
// K rounds of a wavefront maximum
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int K, int lane,
                                            TopkLds& sc, int& my_id, float& my_gate) {
  if (E <= kWave) {
    route_token_rank(row, E, K, lane, sc, my_id, my_gate);
  } else if (E <= 2 * kWave) {
    route_token_rounds<2>(row, E, K, lane, sc, my_id, my_gate);
  } else {
    route_token_rounds<4>(row, E, K, lane, sc, my_id, my_gate);
  }
}

// A team of S wavefronts routes one token (few tokens, idle wavefronts): the
// ranks are sums of counts over disjoint key slices, so they and the
// selection are the same integers as route_token's.  Member q counts the
// keys of slice q into its scratch (route_team_count); after a workgroup
// barrier the team's first member sums the S partial ranks and selects
// (route_team_select, `team` = the members' scratch, in member order).
template <int J>
__device__ __forceinline__ void route_team_count_j(const float* __restrict__ row, int E, int lane,
                                                   int q, int S, TopkLds& sc) {
  float val[J];
  unsigned long long key[J];
  topk_keys<J>(row, E, lane, sc, val, key);  // every member keeps its own copy
  const int sl = ((J * kWave + S - 1) / S + 15) / 16 * 16;
  const int i0 = min(J * kWave, q * sl), i1 = min(J * kWave, i0 + sl);
  int rank[J];
#pragma unroll
  for (int j = 0; j < J; ++j) rank[j] = 0;
  topk_count<J>(sc, i0, i1, key, rank);
#pragma unroll
  for (int j = 0; j < J; ++j) sc.part[lane + kWave * j] = rank[j];
}

template <int J>
__device__ __forceinline__ void route_team_select_j(const float* __restrict__ row, int E, int K,
                                                    int lane, TopkLds* team, int S, int& my_id,
                                                    float& my_gate) {
  float val[J];
  int rank[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    val[j] = row[min(lane + kWave * j, E - 1)];
    rank[j] = 0;
  }
  for (int q = 0; q < S; ++q)
#pragma unroll
    for (int j = 0; j < J; ++j) rank[j] += team[q].part[lane + kWave * j];
  topk_select<J>(val, rank, E, K, lane, team[0], my_id, my_gate);
}

// teams serve the rank loop only (E <= 64: one expert per lane)
__device__ __forceinline__ void route_team_count(const float* __restrict__ row, int E, int lane,
                                                 int q, int S, TopkLds& sc) {
  route_team_count_j<1>(row, E, lane, q, S, sc);
}

__device__ __forceinline__ void route_team_select(const float* __restrict__ row, int E, int K,
                                                  int lane, TopkLds* team, int S, int& my_id,
                                                  float& my_gate) {
  route_team_select_j<1>(row, E, K, lane, team, S, my_id, my_gate);
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

// Union of nk <= 64 slots in one wavefront (lane s holds slot s).  Ballots
// over the eight id bits give every lane the slots with a smaller id (lt)
// and those with the same id (eq); the sorted union, the exclusive scan of
// the per-expert counts, the stable permutation and the slot ranks are then
// population counts of those masks: no LDS round trip and no barrier.
__device__ __forceinline__ void build_union_wave(const int32_t* ids, int nk, int E, int lane,
                                                 int32_t* __restrict__ U_out,
                                                 int32_t* __restrict__ union_ids,
                                                 int32_t* __restrict__ offsets,
                                                 int32_t* __restrict__ perm,
                                                 int32_t* __restrict__ slot_rank) {
  const int cap = nk < E ? nk : E;
  const bool act = lane < nk;
  const int id = act ? ids[lane] : 0;
  if (__ballot(act && (id < 0 || id >= E))) {
    if (lane == 0) *U_out = -1;
    return;
  }
  unsigned long long eq = __ballot(act), lt = 0ull;
#pragma unroll
  for (int b = 7; b >= 0; --b) {  // ids < 256
    const bool bit = ((id >> b) & 1) != 0;
    const unsigned long long ones = __ballot(act && bit);
    if (bit) {
      lt |= eq & ~ones;
      eq &= ones;
    } else {
      eq &= ~ones;
    }
  }
  const unsigned long long below = (1ull << lane) - 1ull;
  const bool first = act && (eq & below) == 0ull;
  const unsigned long long fm = __ballot(first);
  const int U = __popcll(fm);
  const int start = __popcll(lt);  // slots with a smaller id
  if (act) {
    perm[start + __popcll(eq & below)] = lane;
    slot_rank[lane] = __popcll(lt & fm);
  }
  if (first) {
    union_ids[__popcll(lt & fm)] = id;
    offsets[__popcll(lt & fm)] = start;
  }
  for (int i = U + lane; i < cap; i += kWave) union_ids[i] = -1;
  for (int i = U + lane; i <= cap; i += kWave) offsets[i] = nk;
  if (lane == 0) *U_out = U;
}

// The union of one token's K slots, whose ids are distinct (the token's
// top-K): the ids in ascending order, one slot each.  Wavefront 0 builds it
// (the caller's next barrier publishes it); the same outputs as
// build_union_256 for such slots.
__device__ __forceinline__ void build_union_one_token(const int32_t* ids, int K, int E,
                                                      int32_t* __restrict__ U_out,
                                                      int32_t* __restrict__ union_ids,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ perm,
                                                      int32_t* __restrict__ slot_rank) {
  if ((threadIdx.x >> 6) != 0) return;
  const int lane = threadIdx.x & 63;
  const bool act = lane < K;
  const int id = act ? ids[lane] : 0;
  if (__ballot(act && (id < 0 || id >= E))) {
    if (lane == 0) *U_out = -1;
    return;
  }
  int r = 0;  // ids below mine: broadcast reads of the K ids, all in flight at once
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < K) r += ids[j] < id ? 1 : 0;
  if (act) {
    union_ids[r] = id;
    offsets[r] = r;
    perm[r] = lane;
    slot_rank[lane] = r;
  }
  if (lane == 0) {
    offsets[K] = K;
    *U_out = K;
  }
}

// Every thread of the workgroup calls this (it holds __syncthreads); threads
// 0..255 do the work.  Up to 64 slots, wavefront 0 alone builds the union
// (build_union_wave) and the caller's next barrier publishes it.
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
  if (nk <= kWave) {
    if (wave == 0) build_union_wave(ids, nk, E, lane, U_out, union_ids, offsets, perm, slot_rank);
    return;
  }
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


// ----------------------------------------------------------- expert budget
// LDS scratch of apply_budget.
struct BudgetLds {
  unsigned long long key[256];  // order key of union expert u (larger = kept first)
  int old_perm[256];            // the perm before the rewrite
  int newpos[256];              // u kept: its position in the budgeted union; dropped: -1
  int wkept[4], wslots[4], wdrop[4];
};

// Per-layer expert budget ("MoE-Spec: Expert Budgeting for Efficient
// Speculative Decoding", abstract: a layer loads at most C experts, those
// contributing most to the verified tokens).  An expert's contribution is the
// f32 sum of the gates of its slots in ascending slot order; the C largest
// are kept (equal contributions: the lower id; NaN below every number), in
// the order key of the router's top-K.  Rewrites, in place, the union arrays
// of build_union_256 for the same slots: the kept experts ascending, their
// slots grouped as before, offsets from the new U on = the kept slot count,
// the dropped slots after the kept ones in ascending order, slot_rank -1 for
// a dropped slot; a dropped slot's gate becomes 0 and, with renorm, the kept
// gates of a token that lost a slot are divided by their f32 sum (k
// ascending).  Every thread of the workgroup calls it (it holds
// __syncthreads; at least 256 threads); returns the new U.  Call only with
// 0 <= C < U.
__device__ __forceinline__ int apply_budget(int U, int C, int renorm, int n, int K, int cap,
                                            int32_t* union_ids, int32_t* offsets, int32_t* perm,
                                            int32_t* slot_rank, float* gates, BudgetLds& sh) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool mine = tid < 256;
  const int nk = n * K;
  const unsigned long long below = (1ull << lane) - 1ull;
  // contributions and order keys of the old union
  int my_id = 0, my_off = 0, my_cnt = 0;
  if (mine && tid < U) {
    my_id = union_ids[tid];
    my_off = offsets[tid];
    my_cnt = offsets[tid + 1] - my_off;
    float c = 0.0f;
    for (int i = 0; i < my_cnt; ++i) c += gates[perm[my_off + i]];
    sh.key[tid] = (static_cast<unsigned long long>(topk_key(c)) << 8) |
                  static_cast<unsigned>(255 - my_id);
  }
  if (mine && tid < nk) sh.old_perm[tid] = perm[tid];
  __syncthreads();

  // rank = number of keys above mine; kept iff rank < C
  bool kept = false;
  if (mine && tid < U) {
    const unsigned long long k = sh.key[tid];
    int r = 0;
    for (int v = 0; v < U; ++v) r += sh.key[v] > k ? 1 : 0;
    kept = r < C;
  }
  // new position: kept experts below mine; new offset: their slot counts
  const unsigned long long km = __ballot(kept);
  const int kc = kept ? my_cnt : 0;
  const int inc = wave_inclusive_sum(kc, lane);
  if (mine && lane == kWave - 1) {
    sh.wkept[wave] = __popcll(km);
    sh.wslots[wave] = inc;
  }
  __syncthreads();
  int bk = 0, bs = 0, Uk = 0, nkept = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave) {
      bk += sh.wkept[w];
      bs += sh.wslots[w];
    }
    Uk += sh.wkept[w];
    nkept += sh.wslots[w];
  }
  const int npos = kept ? bk + __popcll(km & below) : -1;
  if (mine) sh.newpos[tid] = npos;
  if (kept) {
    const int noff = bs + inc - kc;
    union_ids[npos] = my_id;
    offsets[npos] = noff;
    for (int i = 0; i < my_cnt; ++i) perm[noff + i] = sh.old_perm[my_off + i];
  }
  if (mine) {
    for (int i = Uk + tid; i < cap; i += 256) union_ids[i] = -1;
    for (int i = Uk + tid; i <= cap; i += 256) offsets[i] = nkept;
  }
  __syncthreads();

  // slot ranks, and the dropped slots after the kept ones
  const bool act = mine && tid < nk;
  const int nr = act ? sh.newpos[slot_rank[tid]] : 0;
  const bool drop = act && nr < 0;
  const unsigned long long dm = __ballot(drop);
  if (mine && lane == kWave - 1) sh.wdrop[wave] = __popcll(dm);
  __syncthreads();
  int bd = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    if (w < wave) bd += sh.wdrop[w];
  if (act) {
    slot_rank[tid] = nr;
    if (drop) perm[nkept + bd + __popcll(dm & below)] = tid;
  }
  __syncthreads();

  // gates of the dropped slots, and the kept ones renormalised
  if (tid < n) {
    float tot = 0.0f;
    bool lost = false;
    for (int k = 0; k < K; ++k) {
      if (slot_rank[tid * K + k] < 0) lost = true;
      else tot += gates[tid * K + k];
    }
    const bool div = renorm != 0 && lost;
    for (int k = 0; k < K; ++k) {
      const int s = tid * K + k;
      float g = gates[s];
      if (slot_rank[s] < 0) g = 0.0f;
      else if (div) g = tot > 0.0f ? g / tot : 0.0f;
      gates[s] = g;
    }
  }
  __syncthreads();
  return Uk;
}

}  // namespace moe
