// Combine of the slot outputs, workspace fill and the fp8 decode diagnostic (gfx950).
//
// Combine: the layer output of a MoE layer is the gate-weighted sum of its
// selected experts' outputs ("Making Every Verified Token Count: Adaptive
// Verification for MoE Speculative Decoding", Sec. 2.2), plus the shared
// experts, which every token uses with weight 1.
#include "common.h"

namespace moe {

// One lane: four consecutive columns of one token.  Every load of the lane
// (K slot rows, S shared rows) is issued before the first use, so the kernel
// waits for memory once; the sum runs k ascending, then the shared experts.
constexpr int kCombineBlock = 64;

__global__ __launch_bounds__(kCombineBlock) void combine_kernel(
    const float* __restrict__ y_slots, const float* __restrict__ gates,
    const float* __restrict__ y_shared, int n, int K, int S, int d, void* __restrict__ out,
    int out_bf16) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * kCombineBlock + threadIdx.x) * 4;
  if (t >= n || c >= d) return;
  const float* g = gates + static_cast<size_t>(t) * K;
  const float* y = y_slots + static_cast<size_t>(t) * K * d + c;
  f32x4 yv[8], sv[4];
  float gv[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k < K) {
      yv[k] = *reinterpret_cast<const f32x4*>(y + static_cast<size_t>(k) * d);
      gv[k] = g[k];
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (q < S)
      sv[q] = *reinterpret_cast<const f32x4*>(y_shared + (static_cast<size_t>(t) * S + q) * d + c);
  }
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k < K) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(gv[k], yv[k][i], acc[i]);
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (q < S) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += sv[q][i];
    }
  }
  const size_t o = static_cast<size_t>(t) * d + c;
  if (out_bf16) {
    uint2 packed;
    packed.x = f32_to_bf16_bits(acc[0]) | (static_cast<unsigned>(f32_to_bf16_bits(acc[1])) << 16);
    packed.y = f32_to_bf16_bits(acc[2]) | (static_cast<unsigned>(f32_to_bf16_bits(acc[3])) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + o) = packed;
  } else {
    f32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = acc[i];
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + o) = r;
  }
}

hipError_t launch_combine(const float* y_slots, const float* gates, const float* y_shared,
                          int n, int K, int S, int d, void* out, int out_bf16, hipStream_t s) {
  const int lanes = (d + 3) / 4;
  dim3 grid((lanes + kCombineBlock - 1) / kCombineBlock, n);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(kCombineBlock), 0, s, y_slots, gates, y_shared,
                     n, K, S, d, out, out_bf16);
  return hipGetLastError();
}

// Batched transpose [count][R][C] -> [count][C][R] of T elements through a
// 64 x 64 LDS tile (one column of padding, so the transposed reads hit 64
// different banks): the layout transform of moe_pack_weights.  blockIdx.z is
// the matrix, blockIdx.y the tile row, blockIdx.x the tile column; every
// access is bounds-checked, so R and C need not be multiples of 64.
constexpr int kTile = 64;
constexpr int kTileRows = 4;  // 256 threads: 64 columns x 4 rows per pass

template <typename T>
__global__ __launch_bounds__(kTile * kTileRows) void transpose_kernel(
    const T* __restrict__ src, T* __restrict__ dst, int R, int C) {
  __shared__ T tile[kTile][kTile + 1];
  const size_t mat = static_cast<size_t>(R) * C;
  const T* a = src + blockIdx.z * mat;
  T* b = dst + blockIdx.z * mat;
  const int r0 = blockIdx.y * kTile, c0 = blockIdx.x * kTile;
  const int tx = threadIdx.x % kTile, ty = threadIdx.x / kTile;
  for (int i = ty; i < kTile; i += kTileRows) {
    const int r = r0 + i, c = c0 + tx;
    if (r < R && c < C) tile[i][tx] = a[static_cast<size_t>(r) * C + c];
  }
  __syncthreads();
  for (int i = ty; i < kTile; i += kTileRows) {
    const int c = c0 + i, r = r0 + tx;  // row c of the result holds column c of the source
    if (c < C && r < R) b[static_cast<size_t>(c) * R + r] = tile[tx][i];
  }
}

hipError_t launch_transpose(const void* src, void* dst, int count, int R, int C, int elem,
                            hipStream_t s) {
  if (count == 0 || R == 0 || C == 0) return hipSuccess;
  const dim3 grid((C + kTile - 1) / kTile, (R + kTile - 1) / kTile, count);
  const dim3 block(kTile * kTileRows);
  switch (elem) {
    case 1:
      hipLaunchKernelGGL(transpose_kernel<uint8_t>, grid, block, 0, s,
                         static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), R, C);
      break;
    case 2:
      hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, block, 0, s,
                         static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), R, C);
      break;
    case 4:
      hipLaunchKernelGGL(transpose_kernel<uint32_t>, grid, block, 0, s,
                         static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), R, C);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Zero fill with a kernel (no memset node, so it is safe inside captured graphs).
__global__ __launch_bounds__(kBlock) void fill_zero_kernel(uint32_t* __restrict__ p, size_t words) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kBlock;
  for (size_t i = static_cast<size_t>(blockIdx.x) * kBlock + threadIdx.x; i < words; i += stride)
    p[i] = 0u;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  size_t blocks = (words + kBlock - 1) / kBlock;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, s,
                     static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

// Each lane decodes one code with the conversion the fp8 FFN kernels use,
// picking its byte position inside the aligned dword that holds it.
__global__ __launch_bounds__(kBlock) void decode_fp8_kernel(const uint8_t* __restrict__ codes,
                                                            float* __restrict__ out,
                                                            long long count) {
  const long long i = static_cast<long long>(blockIdx.x) * kBlock + threadIdx.x;
  if (i >= count) return;
  const int pos = static_cast<int>(i & 3);
  unsigned word = 0;
  // assemble the dword from bytes that exist (the buffer may end mid-dword)
  const long long base = i - pos;
  for (int b = 0; b < 4; ++b)
    if (base + b < count) word |= static_cast<unsigned>(codes[base + b]) << (8 * b);
  const bf16x2 v = (pos < 2) ? fp8x2_to_bf16x2<false>(word) : fp8x2_to_bf16x2<true>(word);
  const unsigned pair = __builtin_bit_cast(unsigned, v);
  const uint16_t bits = (pos & 1) ? static_cast<uint16_t>(pair >> 16) : static_cast<uint16_t>(pair);
  out[i] = bf16_bits_to_f32(bits);
}

hipError_t launch_decode_fp8(const uint8_t* codes, float* out, long long count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  const long long blocks = (count + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(decode_fp8_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, s,
                     codes, out, count);
  return hipGetLastError();
}

}  // namespace moe
