// Unit partition arithmetic of the one-launch pass (host and device): range
// bounds, the cost of a unit under the weighted split, and the owners of a
// group's units, so the host can check the device's partition.
#pragma once

namespace moe {

constexpr int kCostGroups = 256 + 8;  // cost tables: U + S <= 256 + 4 groups

// floor(a / b) for 0 <= a < 2^52 and 0 < b < 2^31 without the 64-bit
// integer division routine (a few hundred instructions, paid at the start of
// every phase): the rounded double quotient is within one of the floor,
// which exact integer products then correct
__host__ __device__ __forceinline__ long long div_small(long long a, long long b) {
  long long q = static_cast<long long>(static_cast<double>(a) / static_cast<double>(b));
  if (q * b > a) {
    --q;
  } else if ((q + 1) * b <= a) {
    ++q;
  }
  return q;
}

// cost of one unit of a group of cnt tokens under the weighted split (UP:
// tile tcp of the UP phase, one pass per tile beyond the first; DOWN: the
// matrix-core work per four tokens of each tile); stream.h, phase_costs
__host__ __device__ __forceinline__ int unit_cost(int cnt, int tcp, bool up) {
  if (up) return cnt <= tcp ? 8 : 9 * ((cnt + tcp - 1) / tcp);
  int w = 0;
  for (int t = 0; t < cnt; t += tcp) {
    const int c = cnt - t < tcp ? cnt - t : tcp;
    w += 3 + (c + 3) / 4;
  }
  return w > 0 ? w : 4;
}

// first unit of workgroup c under the weighted partition: the first u with
// P(u) * G >= ctot * c (nu for c = G)
__host__ __device__ __forceinline__ long long weighted_first_unit(const int* cpre, int NG,
                                                                  int upg, long long ctot, int G,
                                                                  int c, long long nu) {
  if (c >= G) return nu;
  const long long X = ctot * c;
  // the first group whose last unit qualifies ((cpre[g+1] - w_g) grows with g)
  int a = 0, z = NG;
  while (a < z) {
    const int m = (a + z) >> 1;
    const long long w = (cpre[m + 1] - cpre[m]) / upg;
    if ((static_cast<long long>(cpre[m + 1]) - w) * G >= X) {
      z = m;
    } else {
      a = m + 1;
    }
  }
  if (a >= NG) return nu;
  const long long w = (cpre[a + 1] - cpre[a]) / upg;
  const long long need = X - static_cast<long long>(cpre[a]) * G;
  const long long t = need <= 0 ? 0 : (need + w * G - 1) / (w * G);
  return static_cast<long long>(a) * upg + t;
}

// The workgroups [c_lo, c_hi] that own the units of group g: with the
// weighted partition (cpre set), the owner of unit u is floor(P(u) * grid /
// ctot), P(u) the cost of the units before u (group g's units cost w each);
// otherwise the largest c with floor(nu * c / grid) <= u.
__host__ __device__ __forceinline__ void group_owners(const int* cpre, long long ctot,
                                                      long long nu, int grid, int upg, int g,
                                                      int& c_lo, int& c_hi) {
  if (cpre != nullptr) {
    const long long p0 = cpre[g], p1 = cpre[g + 1];
    const long long w = (p1 - p0) / upg;
    c_lo = static_cast<int>(div_small(p0 * grid, ctot));
    c_hi = static_cast<int>(div_small((p1 - w) * grid, ctot));
  } else {
    const long long u0 = static_cast<long long>(g) * upg;
    const long long u1 = u0 + upg - 1;
    c_lo = static_cast<int>(div_small((u0 + 1) * grid - 1, nu));
    c_hi = static_cast<int>(div_small((u1 + 1) * grid - 1, nu));
  }
}

}  // namespace moe
