// Weight re-layout done once when a handle is created.
#include "common.h"
#include "kernels.h"

namespace dt {

template <typename T>
__global__ void transpose_kernel(const T* __restrict__ in, T* __restrict__ out, int R, int C) {
  __shared__ T tile[32][33];
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8 threads
  for (int i = ty; i < 32; i += 8) {
    const int r = r0 + i, c = c0 + tx;
    if (r < R && c < C) tile[i][tx] = in[(size_t)r * C + c];
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int c = c0 + i, r = r0 + tx;
    if (r < R && c < C) out[(size_t)c * R + r] = tile[tx][i];
  }
}

hipError_t launch_transpose(const void* in, void* out, int R, int C, int elem_bytes, hipStream_t stream) {
  dim3 grid((C + 31) / 32, (R + 31) / 32);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, dim3(256), 0, stream, (const uint16_t*)in,
                       (uint16_t*)out, R, C);
  else if (elem_bytes == 4)
    hipLaunchKernelGGL(transpose_kernel<uint32_t>, grid, dim3(256), 0, stream, (const uint32_t*)in,
                       (uint32_t*)out, R, C);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// Combined per-node weights Wc [rows, ds]: rows 0..3ds-1 are W_hh (gate blocks
// r, z, n); rows 3ds..3ds+r-1 are the columns of W1_S (W1 rows h..h+ds-1).
// Rows are padded to a multiple of 16 and k to a multiple of 32 with zeros.
template <typename T>
__global__ void pack_node_tiles_kernel(const T* __restrict__ w_hh, const T* __restrict__ w1, int h,
                                       int ds, int r, T* __restrict__ out, int rows_p, int kp) {
  const size_t total = (size_t)rows_p * kp;
  const int nkb = kp / 32;
  for (size_t o = (size_t)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (size_t)gridDim.x * blockDim.x) {
    // o = (((t * nkb + kb) * 4 + kg) * 16 + rr) * 8 + e
    const int e = (int)(o & 7);
    const int rr = (int)((o >> 3) & 15);
    const int kg = (int)((o >> 7) & 3);
    const size_t q = o >> 9;
    const int kb = (int)(q % nkb);
    const int t = (int)(q / nkb);
    const int row = t * 16 + rr;
    const int k = kb * 32 + kg * 8 + e;
    T v = T(0);
    if (k < ds) {
      if (row < 3 * ds) v = w_hh[(size_t)row * ds + k];
      else if (row < 3 * ds + r) v = w1[(size_t)(h + k) * r + (row - 3 * ds)];
    }
    out[o] = v;
  }
}

hipError_t launch_pack_node_tiles(const void* w_hh, const void* w1, int h, int ds, int r, int elem_bytes,
                                  void* out, hipStream_t stream) {
  const int rows_p = (3 * ds + r + 15) / 16 * 16;
  const int kp = (ds + 31) / 32 * 32;
  const size_t total = (size_t)rows_p * kp;
  const unsigned blocks = (unsigned)((total + 255) / 256 < 65535 ? (total + 255) / 256 : 65535);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(pack_node_tiles_kernel<uint16_t>, dim3(blocks), dim3(256), 0, stream,
                       (const uint16_t*)w_hh, (const uint16_t*)w1, h, ds, r, (uint16_t*)out, rows_p, kp);
  else if (elem_bytes == 4)
    hipLaunchKernelGGL(pack_node_tiles_kernel<float>, dim3(blocks), dim3(256), 0, stream, (const float*)w_hh,
                       (const float*)w1, h, ds, r, (float*)out, rows_p, kp);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, size_t n, hipStream_t stream) {
  const unsigned blocks = (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(blocks ? blocks : 1), dim3(256), 0, stream, p, v, n);
  return hipGetLastError();
}

}  // namespace dt
