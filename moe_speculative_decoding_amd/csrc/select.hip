// Draft-tree selection ahead of the verify pass (gfx950).
//
// EVICT ("Making Every Verified Token Count: Adaptive Verification for MoE
// Speculative Decoding", Sec. 3.1-3.2): every node's score is the product of
// the draft probabilities on its path (Eq. (7)); the top-k nodes by score form
// the truncated tree T_k, whose estimated accepted length is the sum of their
// scores (Eq. (8)); the verified prefix is k* = argmax_k E_hat(T_k) / C(k)
// with C the profiled step latency (Eqs. (9)-(10)), computed as prefix sums of
// the sorted scores, a division by the cost table and an argmax (Sec. 3.2.3).
//
// One workgroup holds the whole tree in LDS (N <= 1024 nodes, parent(v) < v).
// Scores are float64 products taken from the root outward, one tree level per
// step, so every score has the same value as the plain path product; nodes
// are ranked by counting the nodes ahead of them (equal scores: the lower
// index first, which keeps each T_k ancestor-closed even where q = 1).
#include "common.h"

namespace moe {

constexpr int kSelectBlock = 1024;

__global__ __launch_bounds__(kSelectBlock) void evict_kernel(
    const int32_t* __restrict__ parent, const float* __restrict__ q,
    const float* __restrict__ cost, int N, int32_t* __restrict__ order,
    double* __restrict__ scores_out, double* __restrict__ expected_out,
    int32_t* __restrict__ k_best, uint32_t* __restrict__ err) {
  __shared__ int par[kSelectBlock];
  __shared__ double s[kSelectBlock];
  __shared__ double scan[2][kSelectBlock];
  __shared__ unsigned char ready[2][kSelectBlock];
  __shared__ double best_u[kSelectBlock / kWave];
  __shared__ int best_k[kSelectBlock / kWave];
  __shared__ int bad;
  const int v = threadIdx.x;
  const bool mine = v < N;
  if (v == 0) bad = 0;
  __syncthreads();
  float qv = 0.0f;
  if (mine) {
    const int p = parent[v];
    qv = q[v];
    par[v] = p;
    const float cv = cost[v];
    if (p < -1 || p >= v || !(qv >= 0.0f && qv <= 1.0f) || !(cv > 0.0f && cv < 3.0e38f))
      atomicOr(&bad, 1);
  }
  ready[0][v] = 0;
  __syncthreads();
  if (bad) {  // uniform
    if (v == 0) {
      atomicOr(err, ERRBIT_BAD_TREE);
      *k_best = 0;
    }
    return;
  }

  // Eq. (7), one level per round: a node is scored once its parent is
  // (double-buffered ready flags, so a round reads only the previous one's)
  int cur = 0;
  bool done = !mine;
  while (__syncthreads_or(!done)) {
    unsigned char r = ready[cur][v];
    if (!done) {
      const int p = par[v];
      if (p < 0 || ready[cur][p]) {
        s[v] = (p < 0 ? 1.0 : s[p]) * static_cast<double>(qv);
        r = 1;
        done = true;
      }
    }
    ready[cur ^ 1][v] = r;
    cur ^= 1;
  }
  __syncthreads();

  // rank = number of nodes ahead (higher score, or equal score and lower index)
  if (mine) {
    const double sv = s[v];
    int rank = 0;
    int w = 0;
    for (; w + 8 <= N; w += 8) {
      double t[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t[i] = s[w + i];  // the same address in every lane
#pragma unroll
      for (int i = 0; i < 8; ++i) rank += (t[i] > sv) || (t[i] == sv && w + i < v);
    }
    for (; w < N; ++w) rank += (s[w] > sv) || (s[w] == sv && w < v);
    order[rank] = v;
    scan[0][rank] = sv;
    if (scores_out != nullptr) scores_out[v] = sv;
  }
  __syncthreads();

  // Eq. (8) for every k: inclusive prefix sums of the sorted scores
  int src = 0;
  for (int off = 1; off < N; off <<= 1) {
    if (mine) scan[src ^ 1][v] = scan[src][v] + (v >= off ? scan[src][v - off] : 0.0);
    __syncthreads();
    src ^= 1;
  }

  // Eq. (10): the first maximum of E_hat(T_k) / C(k), k = v + 1
  double u = -1.0;
  int k = N + 1;
  if (mine) {
    const double e = scan[src][v];
    if (expected_out != nullptr) expected_out[v] = e;
    u = e / static_cast<double>(cost[v]);
    k = v + 1;
  }
  for (int o = 32; o >= 1; o >>= 1) {
    const double u2 = __shfl_xor(u, o);
    const int k2 = __shfl_xor(k, o);
    if (u2 > u || (u2 == u && k2 < k)) {
      u = u2;
      k = k2;
    }
  }
  if ((v & (kWave - 1)) == 0) {
    best_u[v / kWave] = u;
    best_k[v / kWave] = k;
  }
  __syncthreads();
  if (v == 0) {
    double bu = best_u[0];
    int bk = best_k[0];
    for (int i = 1; i < kSelectBlock / kWave; ++i) {
      if (best_u[i] > bu || (best_u[i] == bu && best_k[i] < bk)) {
        bu = best_u[i];
        bk = best_k[i];
      }
    }
    *k_best = bk;
  }
}

hipError_t launch_evict(const int32_t* parent, const float* q, const float* cost, int N,
                        int32_t* order, double* scores, double* expected, int32_t* k_best,
                        uint32_t* err, hipStream_t s) {
  hipLaunchKernelGGL(evict_kernel, dim3(1), dim3(kSelectBlock), 0, s, parent, q, cost, N, order,
                     scores, expected, k_best, err);
  return hipGetLastError();
}

// ------------------------------------------------------------------ EcoSpec
// EcoSpec ("Less Experts, Faster Decoding: Cost-Aware Speculative Decoding for
// Mixture-of-Experts", Sec. 4.2, Algorithm 1): each node's path footprint is
// the union of the predicted (layer, expert) sets on its root path (Eq. (7));
// gamma times, every unselected node is scored P / (|footprint \ B| + eps)
// (Eqs. (8)-(9)), the best is selected and its footprint joins the buffer B.
//
// The footprints are bitsets of W 64-bit words held in LDS; a step's costs are
// popcounts of (footprint AND NOT B) summed per node with LDS atomics (an
// integer sum, so the order does not matter); scores are float64 divisions of
// the same operands on every side; equal scores select the lower index.
constexpr int kMaxSetWordsPerNode = 256;

__global__ __launch_bounds__(kSelectBlock) void ecospec_kernel(
    const int32_t* __restrict__ parent, const float* __restrict__ q,
    const uint64_t* __restrict__ pred, const uint64_t* __restrict__ buffer0, int N, int W,
    int gamma, double eps, int32_t* __restrict__ selected, uint64_t* __restrict__ buffer_out,
    uint32_t* __restrict__ err) {
  extern __shared__ __attribute__((aligned(16))) uint64_t traj[];  // [N][W]
  __shared__ int par[kSelectBlock];
  __shared__ double P[kSelectBlock];
  __shared__ int cost[kSelectBlock];
  __shared__ unsigned char ready[2][kSelectBlock];
  __shared__ unsigned char taken[kSelectBlock];
  __shared__ uint64_t B[kMaxSetWordsPerNode];
  __shared__ double best_s[kSelectBlock / kWave];
  __shared__ int best_t[kSelectBlock / kWave];
  __shared__ int pick, bad;
  const int v = threadIdx.x;
  const bool mine = v < N;
  if (v == 0) bad = 0;
  __syncthreads();
  float qv = 0.0f;
  if (mine) {
    const int p = parent[v];
    qv = q[v];
    par[v] = p;
    if (p < -1 || p >= v || !(qv >= 0.0f && qv <= 1.0f)) atomicOr(&bad, 1);
  }
  ready[0][v] = 0;
  taken[v] = 0;
  for (int i = v; i < N * W; i += kSelectBlock) traj[i] = pred[i];
  for (int w = v; w < W; w += kSelectBlock) B[w] = buffer0 != nullptr ? buffer0[w] : 0ull;
  __syncthreads();
  if (bad) {  // uniform
    if (v == 0) atomicOr(err, ERRBIT_BAD_TREE);
    return;
  }

  // P and footprints, one tree level per round (Eq. (7); P from the root out)
  int cur = 0;
  bool done = !mine;
  while (__syncthreads_or(!done)) {
    unsigned char r = ready[cur][v];
    if (!done) {
      const int p = par[v];
      if (p < 0 || ready[cur][p]) {
        P[v] = (p < 0 ? 1.0 : P[p]) * static_cast<double>(qv);
        if (p >= 0)
          for (int w = 0; w < W; ++w) traj[v * W + w] |= traj[p * W + w];
        r = 1;
        done = true;
      }
    }
    ready[cur ^ 1][v] = r;
    cur ^= 1;
  }
  __syncthreads();

  for (int it = 0; it < gamma; ++it) {
    if (mine) cost[v] = 0;
    __syncthreads();
    // Eq. (8): new experts of every unselected node's footprint
    for (int i = v; i < N * W; i += kSelectBlock) {
      const int t = i / W;
      if (!taken[t]) {
        const int c = __popcll(traj[i] & ~B[i - t * W]);
        if (c) atomicAdd(&cost[t], c);
      }
    }
    __syncthreads();
    // Eq. (9) and the argmax (equal scores: the lower index)
    double sc = -1.0;
    int t = N;
    if (mine && !taken[v]) {
      sc = P[v] / (static_cast<double>(cost[v]) + eps);
      t = v;
    }
    for (int o = 32; o >= 1; o >>= 1) {
      const double s2 = __shfl_xor(sc, o);
      const int t2 = __shfl_xor(t, o);
      if (s2 > sc || (s2 == sc && t2 < t)) {
        sc = s2;
        t = t2;
      }
    }
    if ((v & (kWave - 1)) == 0) {
      best_s[v / kWave] = sc;
      best_t[v / kWave] = t;
    }
    __syncthreads();
    if (v == 0) {
      double bs = best_s[0];
      int bt = best_t[0];
      for (int i = 1; i < kSelectBlock / kWave; ++i) {
        if (best_s[i] > bs || (best_s[i] == bs && best_t[i] < bt)) {
          bs = best_s[i];
          bt = best_t[i];
        }
      }
      pick = bt;
      taken[bt] = 1;
      selected[it] = bt;
    }
    __syncthreads();
    const int pk = pick;
    for (int w = v; w < W; w += kSelectBlock) B[w] |= traj[pk * W + w];  // buffer update
    __syncthreads();
  }
  if (buffer_out != nullptr)
    for (int w = v; w < W; w += kSelectBlock) buffer_out[w] = B[w];
}

hipError_t launch_ecospec(const int32_t* parent, const float* q, const uint64_t* pred,
                          const uint64_t* buffer0, int N, int W, int gamma, double eps,
                          int32_t* selected, uint64_t* buffer_out, uint32_t* err, hipStream_t s) {
  const size_t smem = static_cast<size_t>(N) * W * sizeof(uint64_t);
  hipLaunchKernelGGL(ecospec_kernel, dim3(1), dim3(kSelectBlock), smem, s, parent, q, pred,
                     buffer0, N, W, gamma, eps, selected, buffer_out, err);
  return hipGetLastError();
}

}  // namespace moe
