// Router top-K and expert union for one verify pass (gfx950).
//
// Top-K: "Making Every Verified Token Count: Adaptive Verification for MoE
// Speculative Decoding", Sec. 2.2, Eq. (4) — the indices of the K largest
// router scores, normalised (softmax over the K here).
// Union: "Less Experts, Faster Decoding", Sec. 3, Eq. (1), and the same page
// family's Eq. (5) / (A2): the distinct experts of all verified tokens; the
// slot permutation sorts rows by expert as the MLX-LM deduplicating engine
// does (expert-bytes page, Table 6).
// Budget: "MoE-Spec: Expert Budgeting for Efficient Speculative Decoding",
// abstract — at most C experts per layer, those contributing most.
//
// Both are integer-exact: top-K compares integer keys built from the fp32
// bit pattern (no float arithmetic decides a selection) with DPP maxima
// inside rows of 16 lanes and splits equal keys by the lowest id, and the
// union uses an LDS
// histogram per wavefront, DPP prefix sums and a ballot-based match of equal
// ids, so every output is deterministic.
#include "route.h"

namespace moe {

__global__ __launch_bounds__(kBlock) void route_topk_kernel(const float* __restrict__ logits,
                                                            int n, int E, int K,
                                                            int32_t* __restrict__ ids,
                                                            float* __restrict__ gates) {
  __shared__ TopkLds sc[kBlock / kWave];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kBlock / kWave) + wave;
  if (t >= n) return;  // wave-uniform
  int id;
  float g;
  route_token(logits + static_cast<size_t>(t) * E, E, K, lane, sc[wave], id, g);
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
  __shared__ TopkLds sc[kRouteUnionBlock / kWave];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int t = wave; t < n; t += kRouteUnionBlock / kWave) {
    int id;
    float g;
    route_token(logits + static_cast<size_t>(t) * E, E, K, lane, sc[wave], id, g);
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


// Expert budget on a union of build_union_256 / route_union: one workgroup
// copies the union and the gates to LDS, rewrites them there (apply_budget)
// and stores them back.  Nothing changes when C >= U or U < 0 (ids outside
// [0, E)); the gates are copied to gates_out either way (which may be gates).
__global__ __launch_bounds__(kBlock) void expert_budget_kernel(
    const float* gates, int n, int K, int E, int C, int renorm, int32_t* __restrict__ U_io,
    int32_t* __restrict__ union_ids, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ slot_rank, float* gates_out) {
  __shared__ int32_t ui[256], off[257], pm[256], sr[256];
  __shared__ float g[256];
  __shared__ BudgetLds sh;
  const int tid = threadIdx.x, nk = n * K, cap = nk < E ? nk : E;
  const int U = *U_io;
  for (int i = tid; i < nk; i += kBlock) {
    pm[i] = perm[i];
    sr[i] = slot_rank[i];
    g[i] = gates[i];
  }
  for (int i = tid; i < cap; i += kBlock) ui[i] = union_ids[i];
  for (int i = tid; i <= cap; i += kBlock) off[i] = offsets[i];
  __syncthreads();
  if (U > C) {  // uniform
    const int Uk = apply_budget(U, C, renorm, n, K, cap, ui, off, pm, sr, g, sh);
    for (int i = tid; i < nk; i += kBlock) {
      perm[i] = pm[i];
      slot_rank[i] = sr[i];
    }
    for (int i = tid; i < cap; i += kBlock) union_ids[i] = ui[i];
    for (int i = tid; i <= cap; i += kBlock) offsets[i] = off[i];
    if (tid == 0) *U_io = Uk;
  }
  for (int i = tid; i < nk; i += kBlock) gates_out[i] = g[i];
}

hipError_t launch_expert_budget(const float* gates, int n, int K, int E, int C, int renorm,
                                int32_t* U, int32_t* union_ids, int32_t* offsets, int32_t* perm,
                                int32_t* slot_rank, float* gates_out, hipStream_t s) {
  hipLaunchKernelGGL(expert_budget_kernel, dim3(1), dim3(kBlock), 0, s, gates, n, K, E, C, renorm,
                     U, union_ids, offsets, perm, slot_rank, gates_out);
  return hipGetLastError();
}

}  // namespace moe
