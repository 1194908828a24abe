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
// bf16, large outputs with row-major operands (the fold E W_ih^T):
// gemm_bf16_big_kernel, a 256 x 256 block tile, 256 threads (2 x 2 waves of
// 128 x 128, sixteen 32 x 32 accumulator tiles per wave),
// v_mfma_f32_32x32x16_bf16.  Operands go from global memory straight into a
// four-stage LDS ring (32 k per stage, three stages in flight while the
// fourth is read), one barrier per stage.  Blocks are mapped to tiles XCD by
// XCD, so the blocks on one XCD (and its L2) cover a contiguous run of tiles,
// those that share a tile of the larger operand together.
// The LM head H W_lm: gemm_lm_half_kernel, the same pipeline on 128 x 256
// tiles (four waves of 64 x 128, a three-stage ring of 24 KB) so that two
// blocks share a CU, with both operands in a tiled order -- W_lm once per
// handle, H per call (a 4 MB re-layout) -- in which each 32-k stage of a
// 256-row operand block is one contiguous, already swizzled 16 KB piece:
// every wave load instruction moves eight whole 128-byte lines.  Measured
// against the 256 x 256 kernel on the same tiled operands, 7 % faster (two
// independent load streams per CU), and that one 7 % faster than with H
// row-major (whose 64-byte row pieces take twice the requests).
// bf16, other shapes: a 128 x 128 block tile (2 x 2 waves of 64 x 64), 32 k
// per stage, or (few tiles) 32 x 32 tiles with sixteen waves splitting K.
// fp32: one thread per output element (small shapes only).
#include <algorithm>

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

constexpr int BT = 256;    // big tile (M and N)
constexpr int BK = 32;     // k per stage: one 64-byte row piece per operand row
constexpr int BNS = 4;     // stages in the LDS ring (three in flight while one is read)
constexpr int BOPND = BT * BK;          // bf16 per operand per stage (16 KB)
constexpr int BSTAGE = 2 * BOPND;       // bf16 per stage (A rows, then B rows)
constexpr size_t BIG_LDS = (size_t)BNS * BSTAGE * sizeof(uint16_t);  // 131072 B

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef const __attribute__((address_space(1))) void* glb_ptr;

// LDS layout of one operand stage: row r (0..255) at r * 64 bytes, its four
// 16-byte k pieces permuted by r's swizzle: piece c sits in slot c ^ swz(r),
// swz(r) = ((r >> 1) & 3) ^ 3 ((r >> 3) & 1).  The 16-byte MFMA operand reads
// of 16 consecutive rows then fall in 16 distinct 16-byte bank groups, and of
// any 8 aligned rows in 8.
__device__ __forceinline__ int big_swz(int r) { return ((r >> 1) & 3) ^ (((r >> 3) & 1) * 3); }

// s_waitcnt vmcnt(n), the other counters left alone (gfx9 encoding)
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_bf16_big_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bt, const float* __restrict__ bias,
    float* __restrict__ C, int M, int N, int K, int ldc, int tm, int tiles, int per_xcd) {
  extern __shared__ __attribute__((aligned(16))) uint16_t glds[];
  // blockIdx.x runs round-robin over the 8 XCDs: XCD x takes tiles
  // [x per_xcd, (x + 1) per_xcd), the dimension with fewer tiles fastest (the
  // blocks on an XCD then share the tile of the larger operand)
  const int t = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (t >= tiles) return;
  const int tn = tiles / tm;
  const int m0 = (tm <= tn ? t % tm : t / tn) * BT, n0 = (tm <= tn ? t / tm : t % tn) * BT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = (w >> 1) * 128, wn = (w & 1) * 128;

  // Operand loads go straight to LDS (global_load_lds_dwordx4): one wave
  // instruction fills 1 KB = 16 rows x 64 bytes, lane l the slot (l & 3) of
  // row l >> 2, so it fetches the k piece (l & 3) ^ swz(row).  Wave w fills
  // row blocks 4w..4w+3 of each operand; rows past the matrix repeat its last
  // row (their outputs are not stored).
  const int lr = lane >> 2, lk = 8 * ((lane & 3) ^ big_swz(lr));
  const int nk = K / BK;
  const uint16_t* a_base = A + (size_t)m0 * K;
  const uint16_t* b_base = Bt + (size_t)n0 * K;
  uint32_t a_off[4], b_off[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 16 * (4 * w + q) + lr;
    a_off[q] = (uint32_t)((min(m0 + r, M - 1) - m0) * K + lk);
    b_off[q] = (uint32_t)((min(n0 + r, N - 1) - n0) * K + lk);
  }
  auto issue = [&](int stage) {
    // the stages past the last one load the last k block again (uniform
    // wait counts; the buffer they fill is not read any more)
    const int k0 = min(stage, nk - 1) * BK;
    uint16_t* dst = glds + (stage % BNS) * BSTAGE + (4 * w) * 16 * BK;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      __builtin_amdgcn_global_load_lds((glb_ptr)(a_base + a_off[q] + k0), (lds_ptr)(dst + q * 16 * BK), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((glb_ptr)(b_base + b_off[q] + k0), (lds_ptr)(dst + BOPND + q * 16 * BK), 16,
                                       0, 0);
    }
  };
  // operand reads: lane reads row (lane & 31) of a 32-row block, k piece
  // 2 h + (lane >> 5) (h = 0, 1: the two 16-k halves of a stage), at its
  // swizzled slot
  const int fr = lane & 31;
  const int p0 = 8 * ((lane >> 5) ^ big_swz(fr & 15)), p1 = p0 ^ 16;
  auto frags = [&](int stage, bf16x8 (&af)[2][4], bf16x8 (&bf)[2][4]) {
    const uint16_t* sa = glds + (stage % BNS) * BSTAGE;
    const uint16_t* sb = sa + BOPND;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        af[h][x] = *reinterpret_cast<const bf16x8*>(&sa[(wm + 32 * x + fr) * BK + (h ? p1 : p0)]);
        bf[h][x] = *reinterpret_cast<const bf16x8*>(&sb[(wn + 32 * x + fr) * BK + (h ? p1 : p0)]);
      }
  };
  // this thread's loads of `stage` are in LDS (the BNS - 2 later stages
  // still in flight), then the barrier: every thread's are.  A bare s_barrier:
  // __syncthreads' release fence would wait for every load in flight.  The
  // empty asm statements keep memory accesses on their side of it.
  auto stage_ready = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<8 * (BNS - 2)>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // Pipeline: while the MFMAs of stage i run, stage i + 1 is made ready, the
  // loads of stage i + BNS go out into the buffer stage i used (its operands
  // are in registers by then: the first MFMA of stage i waited for them) and
  // the operands of stage i + 1 are read.
#pragma unroll
  for (int st = 0; st < BNS - 1; ++st) issue(st);
  stage_ready();
  issue(BNS - 1);
  bf16x8 fa[2][2][4], fb[2][2][4];
  frags(0, fa[0], fb[0]);
  auto step = [&](int i, bf16x8 (&ca)[2][4], bf16x8 (&cb)[2][4], bf16x8 (&na)[2][4], bf16x8 (&nb)[2][4]) {
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[0][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ca[0][0], cb[0][y], acc[0][y], 0, 0, 0);
    stage_ready();
    issue(i + BNS);
    frags(i + 1, na, nb);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
          if (h || x) acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ca[h][x], cb[h][y], acc[x][y], 0, 0, 0);
    // schedule: the stage's loads, then its LDS reads spread over the MFMAs
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 12, 0);
  };
  for (int i = 0; i < nk; i += 2) {
    step(i, fa[0], fb[0], fa[1], fb[1]);
    step(i + 1, fa[1], fb[1], fa[0], fb[0]);
  }
  wait_vm<0>();        // no load may still be writing LDS when the block ends
  // D layout: lane holds column (lane & 31), rows 8 (e / 4) + 4 (lane >> 5) + (e % 4)
#pragma unroll
  for (int y = 0; y < 4; ++y) {
    const int col = n0 + wn + 32 * y + fr;
    if (col >= N) continue;
    const float bv = bias ? bias[col] : 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm + 32 * x + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (row < M) C[(size_t)row * ldc + col] = acc[x][y][e] + bv;
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

// Small outputs (few 128 x 128 tiles): one 32 x 32 output tile per block of
// sixteen waves; the waves split K (a multiple of 16 each, at most four
// 64-k steps at K = 4096) so that each wave's operand loads are few and go
// out together, and their partial tiles are summed in LDS in a fixed order.
// Operands are read straight from global memory (16 bytes per lane).
constexpr int SW = 16;  // waves per block
__global__ __launch_bounds__(64 * SW) void gemm_bf16_small_kernel(const uint16_t* __restrict__ A,
                                                                  const uint16_t* __restrict__ Bt,
                                                                  const float* __restrict__ bias,
                                                                  float* __restrict__ C, int M, int N, int K,
                                                                  int ldc) {
  __shared__ float part[SW][32 * 32];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int m0 = blockIdx.y * 32, n0 = blockIdx.x * 32;
  const int kq = ((K + 15) / 16 + SW - 1) / SW * 16;  // k per wave, a multiple of 16
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
  // one output element per thread: the sixteen partials summed pairwise
  const int i = tid;
  float t[SW];
#pragma unroll
  for (int x = 0; x < SW; ++x) t[x] = part[x][i];
#pragma unroll
  for (int h = SW / 2; h >= 1; h >>= 1)
#pragma unroll
    for (int x = 0; x < h; ++x) t[x] = t[x] + t[x + h];
  const int row = m0 + i / 32, col = n0 + i % 32;
  if (row < M && col < N) C[(size_t)row * ldc + col] = t[0] + (bias ? bias[col] : 0.f);
}

hipError_t launch_gemm_bf16(const uint16_t* A, const int32_t* rows, const uint16_t* Bt, const float* bias,
                            float* C, int M, int N, int K, int ldc, hipStream_t stream) {
  if (rows != nullptr || (K & 7) != 0) return hipErrorInvalidValue;
  const long big_tiles = (long)((N + BT - 1) / BT) * ((M + BT - 1) / BT);
  if (K % (2 * BK) == 0 && K >= 2 * BK && big_tiles >= 256 && (size_t)BT * K < (1u << 31)) {
    const int tm = (M + BT - 1) / BT, tiles = (int)big_tiles, per_xcd = (tiles + 7) / 8;
    hipError_t e = hipFuncSetAttribute((const void*)gemm_bf16_big_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)BIG_LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gemm_bf16_big_kernel, dim3(8 * per_xcd), dim3(256), BIG_LDS, stream, A, Bt,
                       bias, C, M, N, K, ldc, tm, tiles, per_xcd);
    return hipGetLastError();
  }
  const long tiles = (long)((N + GT - 1) / GT) * ((M + GT - 1) / GT);
  if (tiles < 256) {
    dim3 grid((N + 31) / 32, (M + 31) / 32);
    hipLaunchKernelGGL(gemm_bf16_small_kernel, grid, dim3(64 * SW), 0, stream, A, Bt, bias, C, M, N, K, ldc);
    return hipGetLastError();
  }
  dim3 grid((N + GT - 1) / GT, (M + GT - 1) / GT);
  hipLaunchKernelGGL(gemm_bf16_kernel, grid, dim3(256), 0, stream, A, Bt, bias, C, M, N, K, ldc);
  return hipGetLastError();
}

bool gemm_b_tiles_ok(int N, int K) { return K >= 2 * BK && K % (2 * BK) == 0 && (size_t)BT * K < (1u << 31) && N > 0; }

// The LM-head GEMM: 128 x 256 tiles (A rows x B rows), both operands in the
// tiled order of launch_pack_b_tiles / pack_a_tiles_kernel, four waves of
// 64 x 128, a three-stage ring of 24 KB stages (72 KB), two blocks per CU.
constexpr int HM = 128;                      // A rows per tile
constexpr int HNS = 3;                       // ring stages
constexpr int HSTAGE = (HM + BT) * BK;       // bf16 per stage (A rows, then B rows)
constexpr size_t HALF_LDS = (size_t)HNS * HSTAGE * sizeof(uint16_t);  // 73728 B

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_lm_half_kernel(
    const uint16_t* __restrict__ At, const uint16_t* __restrict__ Bt, float* __restrict__ C, int M, int N, int K,
    int ldc, int tm, int tiles, int per_xcd) {
  extern __shared__ __attribute__((aligned(16))) uint16_t glds[];
  const int t = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (t >= tiles) return;
  const int m0 = (t % tm) * HM, n0 = (t / tm) * BT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = (w >> 1) * 64, wn = (w & 1) * 128;
  const int nk = K / BK;
  // A: the 128-row half of a 256-row tiled block (rows are contiguous and
  // the swizzle depends on row & 15 only); wave w fills 16-row blocks 2w, 2w+1
  const uint16_t* a_base = At + (size_t)(m0 / BT) * nk * BOPND + (size_t)(m0 % BT) * BK + (2 * w) * 16 * BK + 8 * lane;
  const uint16_t* b_base = Bt + (size_t)(n0 / BT) * nk * BOPND + (4 * w) * 16 * BK + 8 * lane;
  auto issue = [&](int stage) {
    const int ks = min(stage, nk - 1);
    uint16_t* dst = glds + (stage % HNS) * HSTAGE;
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_global_load_lds((glb_ptr)(a_base + (size_t)ks * BOPND + q * 16 * BK),
                                       (lds_ptr)(dst + (2 * w + q) * 16 * BK), 16, 0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_global_load_lds((glb_ptr)(b_base + (size_t)ks * BOPND + q * 16 * BK),
                                       (lds_ptr)(dst + HM * BK + (4 * w + q) * 16 * BK), 16, 0, 0);
  };
  const int fr = lane & 31;
  const int p0 = 8 * ((lane >> 5) ^ big_swz(fr & 15)), p1 = p0 ^ 16;
  auto frags = [&](int stage, bf16x8 (&af)[2][2], bf16x8 (&bf)[2][4]) {
    const uint16_t* sa = glds + (stage % HNS) * HSTAGE;
    const uint16_t* sb = sa + HM * BK;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int x = 0; x < 2; ++x)
        af[h][x] = *reinterpret_cast<const bf16x8*>(&sa[(wm + 32 * x + fr) * BK + (h ? p1 : p0)]);
#pragma unroll
      for (int y = 0; y < 4; ++y)
        bf[h][y] = *reinterpret_cast<const bf16x8*>(&sb[(wn + 32 * y + fr) * BK + (h ? p1 : p0)]);
    }
  };
  auto stage_ready = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<6 * (HNS - 2)>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  floatx16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
#pragma unroll
  for (int st = 0; st < HNS - 1; ++st) issue(st);
  stage_ready();
  issue(HNS - 1);
  bf16x8 fa[2][2][2], fb[2][2][4];
  frags(0, fa[0], fb[0]);
  auto step = [&](int i, bf16x8 (&ca)[2][2], bf16x8 (&cb)[2][4], bf16x8 (&na)[2][2], bf16x8 (&nb)[2][4]) {
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[0][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ca[0][0], cb[0][y], acc[0][y], 0, 0, 0);
    stage_ready();
    issue(i + HNS);
    frags(i + 1, na, nb);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
          if (h || x) acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ca[h][x], cb[h][y], acc[x][y], 0, 0, 0);
#pragma unroll
    for (int g = 0; g < 6; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
  };
  for (int i = 0; i < nk; i += 2) {
    step(i, fa[0], fb[0], fa[1], fb[1]);
    step(i + 1, fa[1], fb[1], fa[0], fb[0]);
  }
  wait_vm<0>();
#pragma unroll
  for (int y = 0; y < 4; ++y) {
    const int col = n0 + wn + 32 * y + fr;
    if (col >= N) continue;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm + 32 * x + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (row < M) C[(size_t)row * ldc + col] = acc[x][y][e];
      }
  }
}

// A [M, K] row-major into the same tile order as launch_pack_b_tiles' (block
// (mt, s): rows 256 mt .. 256 mt + 255, k 32 s .. 32 s + 31, swizzled, rows
// past M zero).  One thread per 64-byte row piece.
__global__ __launch_bounds__(256) void pack_a_tiles_kernel(const uint16_t* __restrict__ A, uint16_t* __restrict__ out,
                                                           int M, int K) {
  const int nk = K / BK;
  const size_t n = (size_t)((M + BT - 1) / BT) * BT * nk;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const int st = (int)(i % nk);
    const size_t rowg = i / nk;  // global row
    const int mt = (int)(rowg / BT), r = (int)(rowg % BT);
    uint4 q[BK / 8];
#pragma unroll
    for (int c = 0; c < BK / 8; ++c)
      q[c] = rowg < (size_t)M ? *reinterpret_cast<const uint4*>(A + rowg * K + st * BK + 8 * c) : make_uint4(0, 0, 0, 0);
    uint16_t* o = out + ((size_t)mt * nk + st) * BOPND + (size_t)r * BK;
    const int sw = big_swz(r & 15);
#pragma unroll
    for (int c = 0; c < BK / 8; ++c) *reinterpret_cast<uint4*>(o + 8 * (c ^ sw)) = q[c];
  }
}

size_t gemm_a_tiles_elems(int M, int K) { return (size_t)((M + BT - 1) / BT) * BT * K; }

hipError_t launch_gemm_bf16_btiled(const uint16_t* A, const uint16_t* Btiled, float* C, int M, int N, int K,
                                   int ldc, uint16_t* a_tiles, hipStream_t stream) {
  if (!gemm_b_tiles_ok(N, K) || M <= 0 || !a_tiles) return hipErrorInvalidValue;
  const int nk = K / BK;
  const size_t n = (size_t)((M + BT - 1) / BT) * BT * nk;
  hipLaunchKernelGGL(pack_a_tiles_kernel, dim3((unsigned)std::min<size_t>((n + 255) / 256, 4096)), dim3(256), 0,
                     stream, A, a_tiles, M, K);
  const int tm = (M + HM - 1) / HM, tiles = tm * ((N + BT - 1) / BT), per_xcd = (tiles + 7) / 8;
  hipError_t e = hipFuncSetAttribute((const void*)gemm_lm_half_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)HALF_LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gemm_lm_half_kernel, dim3(8 * per_xcd), dim3(256), HALF_LDS, stream, a_tiles, Btiled, C, M, N,
                     K, ldc, tm, tiles, per_xcd);
  return hipGetLastError();
}

// Bt tiled from W [K, N] (row-major, the math layout x W): block (nt, s) holds
// rows n = 256 nt .. 256 nt + 255 of W^T, k = 32 s .. 32 s + 31, row r at
// r * 32 elements with its k piece c (8 elements) in slot c ^ big_swz(r);
// rows past N are zero.  One thread per row of a block: 32 coalesced reads of
// W's rows, 64 contiguous bytes written.
__global__ __launch_bounds__(256) void pack_b_tiles_kernel(const uint16_t* __restrict__ W, uint16_t* __restrict__ out,
                                                           int K, int N) {
  const int nt = blockIdx.x, st = blockIdx.y, r = threadIdx.x;
  const int n = nt * BT + r;
  uint16_t v[BK];
#pragma unroll
  for (int k = 0; k < BK; ++k) v[k] = n < N ? W[(size_t)(st * BK + k) * N + n] : (uint16_t)0;
  uint16_t* o = out + ((size_t)nt * (K / BK) + st) * BOPND + (size_t)r * BK;
  const int sw = big_swz(r & 15);
#pragma unroll
  for (int c = 0; c < BK / 8; ++c) {
    uint4 q;
    q.x = v[8 * c + 0] | ((uint32_t)v[8 * c + 1] << 16);
    q.y = v[8 * c + 2] | ((uint32_t)v[8 * c + 3] << 16);
    q.z = v[8 * c + 4] | ((uint32_t)v[8 * c + 5] << 16);
    q.w = v[8 * c + 6] | ((uint32_t)v[8 * c + 7] << 16);
    *reinterpret_cast<uint4*>(o + 8 * (c ^ sw)) = q;
  }
}

size_t gemm_b_tiles_elems(int N, int K) { return (size_t)((N + BT - 1) / BT) * BT * K; }

hipError_t launch_pack_b_tiles(const uint16_t* W, uint16_t* out, int K, int N, hipStream_t stream) {
  if (!gemm_b_tiles_ok(N, K)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_b_tiles_kernel, dim3((N + BT - 1) / BT, K / BK), dim3(256), 0, stream, W, out, K, N);
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

