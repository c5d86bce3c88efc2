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
// One workgroup holds the whole tree in LDS (N <= 1024 nodes, parent(v) < v);
// its size follows N (one wavefront for the trees of 64 nodes or fewer that
// draft steps produce), so the barriers cost little.
// Scores are float64 products taken from the root outward, one tree level per
// step, so every score has the same value as the plain path product; nodes
// are ranked by counting the nodes ahead of them (equal scores: the lower
// index first, which keeps each T_k ancestor-closed even where q = 1).
#include "common.h"

namespace moe {

constexpr int kSelectMax = 1024;          // largest tree / workgroup
constexpr int kSelectWaves = kSelectMax / kWave;

__device__ __forceinline__ int wave_sum_i32(int v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// first maximum of (value, index) over the workgroup: equal values give the
// lower index.  Every thread calls it; thread 0 returns the index.
__device__ __forceinline__ int block_argmax(double u, int k, double* best_u, int* best_k) {
  for (int o = 32; o >= 1; o >>= 1) {
    const double u2 = __shfl_xor(u, o);
    const int k2 = __shfl_xor(k, o);
    if (u2 > u || (u2 == u && k2 < k)) {
      u = u2;
      k = k2;
    }
  }
  const int nw = static_cast<int>(blockDim.x) / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    best_u[threadIdx.x / kWave] = u;
    best_k[threadIdx.x / kWave] = k;
  }
  __syncthreads();
  int bk = best_k[0];
  if (threadIdx.x == 0) {
    double bu = best_u[0];
    for (int i = 1; i < nw; ++i) {
      if (best_u[i] > bu || (best_u[i] == bu && best_k[i] < bk)) {
        bu = best_u[i];
        bk = best_k[i];
      }
    }
  }
  return bk;
}

// the selection kernels' workgroup: threads >= nodes (tree level steps run a
// thread per node), a multiple of a wavefront
static int select_threads(int nodes, int want) {
  int t = nodes > want ? nodes : want;
  t = (t + kWave - 1) / kWave * kWave;
  return t > kSelectMax ? kSelectMax : t;
}

__global__ __launch_bounds__(kSelectMax) void evict_kernel(
    const int32_t* __restrict__ parent, const float* __restrict__ q,
    const float* __restrict__ cost, int N, int32_t* __restrict__ order,
    double* __restrict__ scores_out, double* __restrict__ expected_out,
    int32_t* __restrict__ k_best, uint32_t* __restrict__ err) {
  __shared__ int par[kSelectMax];
  __shared__ double s[kSelectMax];
  __shared__ double scan[2][kSelectMax];
  __shared__ unsigned char ready[2][kSelectMax];
  __shared__ double best_u[kSelectWaves];
  __shared__ int best_k[kSelectWaves];
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
  if (mine) {
    const double e = scan[src][v];
    if (expected_out != nullptr) expected_out[v] = e;
    u = e / static_cast<double>(cost[v]);
  }
  const int kb = block_argmax(u, mine ? v + 1 : N + 1, best_u, best_k);
  if (v == 0) *k_best = kb;
}

hipError_t launch_evict(const int32_t* parent, const float* q, const float* cost, int N,
                        int32_t* order, double* scores, double* expected, int32_t* k_best,
                        uint32_t* err, hipStream_t s) {
  hipLaunchKernelGGL(evict_kernel, dim3(1), dim3(select_threads(N, kWave)), 0, s, parent, q, cost,
                     N, order, scores, expected, k_best, err);
  return hipGetLastError();
}

// ------------------------------------------------------------------ EcoSpec
// EcoSpec ("Less Experts, Faster Decoding: Cost-Aware Speculative Decoding for
// Mixture-of-Experts", Sec. 4.2, Algorithm 1): each node's path footprint is
// the union of the predicted (layer, expert) sets on its root path (Eq. (7));
// gamma times, every unselected node is scored P / (|footprint \ B| + eps)
// (Eqs. (8)-(9)), the best is selected and its footprint joins the buffer B.
//
// The footprints are bitsets of W 64-bit words held in LDS; a step's cost of
// a node is the popcount of (footprint AND NOT B) summed by one wavefront
// (an integer sum, so the order does not matter); scores are float64
// divisions of the same operands on every side; equal scores select the
// lower index.
constexpr int kMaxSetWordsPerNode = 256;

__global__ __launch_bounds__(kSelectMax) void ecospec_kernel(
    const int32_t* __restrict__ parent, const float* __restrict__ q,
    const uint64_t* __restrict__ pred, const uint64_t* __restrict__ buffer0, int N, int W,
    int gamma, double eps, int32_t* __restrict__ selected, uint64_t* __restrict__ buffer_out,
    uint32_t* __restrict__ err) {
  extern __shared__ __attribute__((aligned(16))) uint64_t traj[];  // [N][W]
  __shared__ int par[kSelectMax];
  __shared__ double P[kSelectMax];
  __shared__ int cost[kSelectMax];
  __shared__ unsigned char ready[2][kSelectMax];
  __shared__ unsigned char fresh[kSelectMax];
  __shared__ unsigned char taken[kSelectMax];
  __shared__ uint64_t B[kMaxSetWordsPerNode];
  __shared__ double best_s[kSelectWaves];
  __shared__ int best_t[kSelectWaves];
  __shared__ int pick, bad;
  const int v = threadIdx.x, nthr = blockDim.x;
  const int wave = v / kWave, lane = v & (kWave - 1), nwaves = nthr / kWave;
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
  for (int i = v; i < N * W; i += nthr) traj[i] = pred[i];
  for (int w = v; w < W; w += nthr) B[w] = buffer0 != nullptr ? buffer0[w] : 0ull;
  __syncthreads();
  if (bad) {  // uniform
    if (v == 0) atomicOr(err, ERRBIT_BAD_TREE);
    return;
  }

  // P and footprints, one tree level per round (Eq. (7); P from the root out):
  // a node whose parent is complete takes its P, then every thread ORs the
  // parent's words into the fresh nodes' footprints
  int cur = 0;
  bool done = !mine;
  while (__syncthreads_or(!done)) {
    unsigned char f = 0;
    if (!done) {
      const int p = par[v];
      if (p < 0 || ready[cur][p]) {
        P[v] = (p < 0 ? 1.0 : P[p]) * static_cast<double>(qv);
        f = 1;
        done = true;
      }
    }
    fresh[v] = f;
    __syncthreads();
    for (int i = v; i < N * W; i += nthr) {
      const int t = i / W;
      if (fresh[t] && par[t] >= 0) traj[i] |= traj[par[t] * W + (i - t * W)];
    }
    ready[cur ^ 1][v] = ready[cur][v] | f;
    cur ^= 1;
  }
  __syncthreads();

  for (int it = 0; it < gamma; ++it) {
    // Eq. (8): new experts of every unselected node's footprint, a wavefront
    // per node
    for (int t = wave; t < N; t += nwaves) {
      if (taken[t]) continue;  // uniform in the wavefront
      int c = 0;
      for (int w = lane; w < W; w += kWave) c += __popcll(traj[t * W + w] & ~B[w]);
      c = wave_sum_i32(c);
      if (lane == 0) cost[t] = c;
    }
    __syncthreads();
    // Eq. (9) and the argmax (equal scores: the lower index)
    double sc = -1.0;
    if (mine && !taken[v]) sc = P[v] / (static_cast<double>(cost[v]) + eps);
    const int bt = block_argmax(sc, mine && !taken[v] ? v : N, best_s, best_t);
    if (v == 0) {
      pick = bt;
      taken[bt] = 1;
      selected[it] = bt;
    }
    __syncthreads();
    const int pk = pick;
    for (int w = v; w < W; w += nthr) B[w] |= traj[pk * W + w];  // the buffer update
    __syncthreads();
  }
  if (buffer_out != nullptr)
    for (int w = v; w < W; w += nthr) buffer_out[w] = B[w];
}

hipError_t launch_ecospec(const int32_t* parent, const float* q, const uint64_t* pred,
                          const uint64_t* buffer0, int N, int W, int gamma, double eps,
                          int32_t* selected, uint64_t* buffer_out, uint32_t* err, hipStream_t s) {
  const size_t smem = static_cast<size_t>(N) * W * sizeof(uint64_t);
  // a wavefront per node for the cost sums, up to 16
  const int threads = select_threads(N, kWave * (N < kSelectWaves ? N : kSelectWaves));
  hipLaunchKernelGGL(ecospec_kernel, dim3(1), dim3(threads), smem, s, parent, q, pred, buffer0, N,
                     W, gamma, eps, selected, buffer_out, err);
  return hipGetLastError();
}


// ----------------------------------------------------- Bellman draft lengths
// "The Limits of Speculation: Bounding Speculative Decoding in MoE", Sec. 4:
// over a reference sequence of N tokens, dp[i] = min_k sum_{a=0..k}
// P(a | k) (Cost(i, k, a) + dp[min(i + a + 1, N)]) with dp[N] = 0 (Eq. (8)),
// P(a | k) = (prod_{j<a} p_j)(1 - p_a) for a < k, P(k | k) = prod_{j<k} p_j
// (Eq. (7)), p_j = q[i + j] (0 past the end).  Backward induction is a chain
// of N dependent steps, so one wavefront runs it: lane k - 1 evaluates draft
// length k from its cost row (read from LDS into registers at the start of
// the step); the q values and dp values ahead sit in register windows that
// every lane holds alike (a step shifts them by one), so the products of
// Eq. (7) need no cross-lane traffic, and the smallest expected cost comes
// from a DPP minimum and a ballot (equal costs: the lowest lane, the shorter
// draft).  Every product and sum is
// a separately rounded float64 operation in the order of the equations (a
// ascending), so dp and the policy are reproducible bit for bit.  The other
// three wavefronts stage the next block of cost rows and q values into LDS
// while wavefront 0 works through the current one.
constexpr int kBellmanBlock = 256;
constexpr int kBellmanCostLds = 2048;  // doubles of cost rows per staging buffer

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const unsigned long long b = __double_as_longlong(v);
  const unsigned lo = __builtin_amdgcn_readlane(static_cast<unsigned>(b), lane);
  const unsigned hi = __builtin_amdgcn_readlane(static_cast<unsigned>(b >> 32), lane);
  return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const unsigned long long b = __double_as_longlong(v);
  const unsigned lo = static_cast<unsigned>(__builtin_amdgcn_update_dpp(
      0, static_cast<int>(static_cast<unsigned>(b)), CTRL, 0xF, 0xF, false));
  const unsigned hi = static_cast<unsigned>(__builtin_amdgcn_update_dpp(
      0, static_cast<int>(static_cast<unsigned>(b >> 32)), CTRL, 0xF, 0xF, false));
  return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo));
}
// minimum over the wavefront (no NaN): DPP inside rows of 16, then the rows
__device__ __forceinline__ double wave_min_f64(double v) {
  v = fmin(v, dpp_f64<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmin(v, dpp_f64<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmin(v, dpp_f64<0x141>(v));  // row_half_mirror
  v = fmin(v, dpp_f64<0x140>(v));  // row_mirror
  return fmin(fmin(readlane_f64(v, 0), readlane_f64(v, 16)),
              fmin(readlane_f64(v, 32), readlane_f64(v, 48)));
}

template <int LM>  // L <= LM: the cost row of a lane fits LM + 1 registers
__global__ __launch_bounds__(kBellmanBlock) void bellman_kernel(const double* __restrict__ q,
                                                                const double* __restrict__ cost,
                                                                int N, int L,
                                                                double* __restrict__ dp_out,
                                                                int32_t* __restrict__ k_out,
                                                                uint32_t* __restrict__ err) {
#pragma clang fp contract(off)  // every product and sum rounded on its own, as the equations read
  __shared__ double cst[2][kBellmanCostLds];
  __shared__ double qs[2][kBellmanCostLds / 2];
  __shared__ int bad;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rowd = L * (L + 1);
  const int T = kBellmanCostLds / rowd > 1 ? kBellmanCostLds / rowd : 1;
  const int nb = (N + T - 1) / T;
  if (tid == 0) {
    bad = 0;
    dp_out[N] = 0.0;
  }
  __syncthreads();
  // block b holds positions [lo, hi), hi = N - b T; threads [t0, t0 + nt) stage it
  auto stage = [&](int b, int t0, int nt) {
    const int hi = N - b * T, lo = hi - T > 0 ? hi - T : 0;
    const int buf = b & 1;
    const int cnt = (hi - lo) * rowd;
    int flag = 0;
    for (int x = tid - t0; x < cnt; x += nt) {
      const double v = cost[static_cast<size_t>(lo) * rowd + x];
      flag |= !__builtin_isfinite(v);
      cst[buf][x] = v;
    }
    for (int x = tid - t0; x < hi - lo; x += nt) {
      const double v = q[lo + x];
      flag |= !(v >= 0.0 && v <= 1.0);
      qs[buf][x] = v;
    }
    if (flag) bad = 1;
  };
  stage(0, 0, kBellmanBlock);
  __syncthreads();

  const double inf = __longlong_as_double(0x7ff0000000000000ll);
  // windows ahead of position i, the same in every lane: qw[a] = q[i + a]
  // (p_a), dw[a] = dp[i + 1 + a]; positions at or past N hold 0 (dp[N] = 0,
  // and min(i + a + 1, N) = N there).  A step shifts both by one.
  double qw[LM], dw[LM + 1];
#pragma unroll
  for (int a = 0; a < LM; ++a) qw[a] = 0.0;
#pragma unroll
  for (int a = 0; a <= LM; ++a) dw[a] = 0.0;
  const int k = lane + 1;
  const bool act = k <= L;
  for (int b = 0; b < nb; ++b) {
    if (wave != 0) {
      if (b + 1 < nb) stage(b + 1, kWave, kBellmanBlock - kWave);
    } else {
      const int hi = N - b * T, lo = hi - T > 0 ? hi - T : 0;
      const int buf = b & 1;
      for (int i = hi - 1; i >= lo; --i) {
        const double* crow = &cst[buf][(i - lo) * rowd + (k - 1) * (L + 1)];
        double c[LM + 1];
#pragma unroll
        for (int a = 0; a <= LM; ++a) c[a] = (act && a <= k) ? crow[a] : 0.0;
#pragma unroll
        for (int a = LM - 1; a > 0; --a) qw[a] = qw[a - 1];
        qw[0] = qs[buf][i - lo];
        // Eq. (7) along the window (the same in every lane): pre_a = prod_{j<a}
        // p_j, and P(a | k) = pre_a (1 - p_a) for a < k, pre_k for a = k
        double pre[LM + 1], stop[LM];
        pre[0] = 1.0;
#pragma unroll
        for (int a = 0; a < LM; ++a) {
          stop[a] = pre[a] * (1.0 - qw[a]);
          pre[a + 1] = pre[a] * qw[a];
        }
        // Eq. (8) for draft length k = lane + 1, a ascending
        double acc = 0.0;
#pragma unroll
        for (int a = 0; a <= LM; ++a) {
          const double P = a < k ? (a < LM ? stop[a] : 0.0) : pre[a];
          const double t = acc + P * (c[a] + dw[a]);  // not fused: contraction is off here
          acc = (act && a <= k) ? t : acc;
        }
        const double v = act ? acc : inf;
        const double vmin = wave_min_f64(v);
        const int kk = __ffsll(static_cast<unsigned long long>(__ballot(act && v == vmin)));
#pragma unroll
        for (int a = LM; a > 0; --a) dw[a] = dw[a - 1];
        dw[0] = vmin;
        if (lane == 0) {
          dp_out[i] = vmin;
          k_out[i] = kk;
        }
      }
    }
    __syncthreads();
  }
  if (tid == 0 && bad) atomicOr(err, ERRBIT_BAD_TREE);
}

hipError_t launch_bellman(const double* q, const double* cost, int N, int L, double* dp,
                          int32_t* k_best, uint32_t* err, hipStream_t s) {
  if (L <= 4)
    hipLaunchKernelGGL(bellman_kernel<4>, dim3(1), dim3(kBellmanBlock), 0, s, q, cost, N, L, dp,
                       k_best, err);
  else if (L <= 8)
    hipLaunchKernelGGL(bellman_kernel<8>, dim3(1), dim3(kBellmanBlock), 0, s, q, cost, N, L, dp,
                       k_best, err);
  else if (L <= 16)
    hipLaunchKernelGGL(bellman_kernel<16>, dim3(1), dim3(kBellmanBlock), 0, s, q, cost, N, L, dp,
                       k_best, err);
  else
    hipLaunchKernelGGL(bellman_kernel<32>, dim3(1), dim3(kBellmanBlock), 0, s, q, cost, N, L, dp,
                       k_best, err);
  return hipGetLastError();
}

}  // namespace moe
