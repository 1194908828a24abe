// Dense products of the builder.
//
//   C[m, n] = sum_k A[m, k] * Bt[n, k] (+ bias[n]),  fp32 accumulate and output.
//
// Uses: the one-time fold of the GRU input weights into the embedding table,
// G = E W_ih^T + b_ih ([V, 3 d_s]), which turns the per-node GRU input term
// W_ih E[token] of the Domino head (Domino summary, 核心方法) into a row
// lookup; and the per-round hoist P = H W1_H of the path-independent half of
// the correction's first projection (H_d is shared by every path: DominoTree
// technical summary, Componenti Core 1).
//
// bf16: a 128 x 128 block tile, 256 threads (2 x 2 waves of 64 x 64), MFMA
// v_mfma_f32_32x32x16_bf16 with operands staged through LDS 32 k at a time.
// fp32: one thread per output element (small shapes only).
#include "common.h"
#include "kernels.h"

namespace dt {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int GT = 128;          // block tile (M and N)
constexpr int GK = 32;           // k per stage
constexpr int LDS_ROW = GK + 8;  // bf16 elements per LDS row (padded: 80 B)

__device__ __forceinline__ uint4 load_row8(const uint16_t* base, int row, int rows, int k0, int K,
                                           size_t ld) {
  // 8 consecutive bf16 of one row, zero outside the matrix (K % 8 == 0)
  if (row < rows && k0 < K) return *reinterpret_cast<const uint4*>(base + (size_t)row * ld + k0);
  return make_uint4(0, 0, 0, 0);
}

__global__ __launch_bounds__(256) void gemm_bf16_kernel(const uint16_t* __restrict__ A,
                                                        const uint16_t* __restrict__ Bt,
                                                        const float* __restrict__ bias,
                                                        float* __restrict__ C, int M, int N, int K,
                                                        int ldc) {
  __shared__ uint16_t sa[GT * LDS_ROW];
  __shared__ uint16_t sb[GT * LDS_ROW];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int m0 = blockIdx.y * GT, n0 = blockIdx.x * GT;
  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // each thread stages 2 x 16 B of A and of B per k stage
  const int lr = tid >> 2;         // 0..63
  const int lk = (tid & 3) * 8;    // 0, 8, 16, 24
  for (int k0 = 0; k0 < K; k0 += GK) {
    uint4 a0 = load_row8(A, m0 + lr, M, k0 + lk, K, K);
    uint4 a1 = load_row8(A, m0 + lr + 64, M, k0 + lk, K, K);
    uint4 b0 = load_row8(Bt, n0 + lr, N, k0 + lk, K, K);
    uint4 b1 = load_row8(Bt, n0 + lr + 64, N, k0 + lk, K, K);
    __syncthreads();
    *reinterpret_cast<uint4*>(&sa[lr * LDS_ROW + lk]) = a0;
    *reinterpret_cast<uint4*>(&sa[(lr + 64) * LDS_ROW + lk]) = a1;
    *reinterpret_cast<uint4*>(&sb[lr * LDS_ROW + lk]) = b0;
    *reinterpret_cast<uint4*>(&sb[(lr + 64) * LDS_ROW + lk]) = b1;
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < GK; ks += 16) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const bf16x8*>(&sa[row * LDS_ROW + ks + 8 * (lane >> 5)]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = wn + j * 32 + (lane & 31);
        bfr[j] = *reinterpret_cast<const bf16x8*>(&sb[col * LDS_ROW + ks + 8 * (lane >> 5)]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }
  // D layout: lane holds column (lane & 31), rows 8 (e / 4) + 4 (lane >> 5) + (e % 4)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn + j * 32 + (lane & 31);
      if (col >= N) continue;
      const float bv = bias ? bias[col] : 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (row < M) C[(size_t)row * ldc + col] = acc[i][j][e] + bv;
      }
    }
}

__global__ void gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ Bt,
                                const float* __restrict__ bias, float* __restrict__ C, int M, int N,
                                int K, int ldc) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)M * N) return;
  const int m = (int)(idx / N), n = (int)(idx % N);
  const float* a = A + (size_t)m * K;
  const float* b = Bt + (size_t)n * K;
  float s = 0.f;
  for (int k = 0; k < K; ++k) s = fmaf(a[k], b[k], s);
  C[(size_t)m * ldc + n] = s + (bias ? bias[n] : 0.f);
}

// Small outputs (few 128 x 128 tiles): one 32 x 32 output tile per block, the
// four waves split K and their partial tiles are summed in LDS in a fixed
// order.  Operands are read straight from global memory (16 bytes per lane).
__global__ __launch_bounds__(256) void gemm_bf16_small_kernel(const uint16_t* __restrict__ A,
                                                              const uint16_t* __restrict__ Bt,
                                                              const float* __restrict__ bias,
                                                              float* __restrict__ C, int M, int N, int K,
                                                              int ldc) {
  __shared__ float part[4][32 * 32];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int m0 = blockIdx.y * 32, n0 = blockIdx.x * 32;
  const int kq = ((K + 15) / 16 + 3) / 4 * 16;  // k per wave, a multiple of 16
  const int kb = w * kq, ke = min(K, kb + kq);
  floatx16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  const int ar = m0 + (lane & 31), bc = n0 + (lane & 31), ko = 8 * (lane >> 5);
  for (int k = kb; k < ke; k += 64) {
    bf16x8 av[4], bv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 a = load_row8(A, ar, M, k + 16 * q + ko, ke, K);
      const uint4 b = load_row8(Bt, bc, N, k + 16 * q + ko, ke, K);
      av[q] = *reinterpret_cast<const bf16x8*>(&a);
      bv[q] = *reinterpret_cast<const bf16x8*>(&b);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[q], bv[q], acc, 0, 0, 0);
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) part[w][(8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) * 32 + (lane & 31)] = acc[e];
  __syncthreads();
  for (int i = tid; i < 32 * 32; i += 256) {
    const int row = m0 + i / 32, col = n0 + i % 32;
    if (row < M && col < N)
      C[(size_t)row * ldc + col] = ((part[0][i] + part[1][i]) + (part[2][i] + part[3][i])) + (bias ? bias[col] : 0.f);
  }
}

hipError_t launch_gemm_bf16(const uint16_t* A, const int32_t* rows, const uint16_t* Bt, const float* bias,
                            float* C, int M, int N, int K, int ldc, hipStream_t stream) {
  if (rows != nullptr || (K & 7) != 0) return hipErrorInvalidValue;
  const long tiles = (long)((N + GT - 1) / GT) * ((M + GT - 1) / GT);
  if (tiles < 256) {
    dim3 grid((N + 31) / 32, (M + 31) / 32);
    hipLaunchKernelGGL(gemm_bf16_small_kernel, grid, dim3(256), 0, stream, A, Bt, bias, C, M, N, K, ldc);
    return hipGetLastError();
  }
  dim3 grid((N + GT - 1) / GT, (M + GT - 1) / GT);
  hipLaunchKernelGGL(gemm_bf16_kernel, grid, dim3(256), 0, stream, A, Bt, bias, C, M, N, K, ldc);
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const float* A, const int32_t* rows, const float* Bt, const float* bias,
                           float* C, int M, int N, int K, int ldc, hipStream_t stream) {
  if (rows != nullptr) return hipErrorInvalidValue;
  const size_t n = (size_t)M * N;
  hipLaunchKernelGGL(gemm_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, A, Bt, bias,
                     C, M, N, K, ldc);
  return hipGetLastError();
}

}  // namespace dt

