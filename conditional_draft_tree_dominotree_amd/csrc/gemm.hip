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

// acc = the 128 x 256 tile (m0, n0) of At Bt^T.  Lane layout of acc[x][y]
// (wave w: rows 64 (w >> 1) + 32 x, columns 128 (w & 1) + 32 y): column
// (lane & 31), rows 8 (e / 4) + 4 (lane >> 5) + (e % 4) of element e.
__device__ __forceinline__ void lm_mainloop(const uint16_t* __restrict__ At, const uint16_t* __restrict__ Bt, int K,
                                            int m0, int n0, uint16_t* glds, floatx16 (&acc)[2][4]) {
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
}

// Store a wave's share of the tile (rows < M, columns < N) into C.
__device__ __forceinline__ void lm_store(const floatx16 (&acc)[2][4], float* __restrict__ C, int M, int N, int ldc,
                                         int m0, int n0) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = (w >> 1) * 64, wn = (w & 1) * 128;
#pragma unroll
  for (int y = 0; y < 4; ++y) {
    const int col = n0 + wn + 32 * y + (lane & 31);
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

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_lm_half_kernel(
    const uint16_t* __restrict__ At, const uint16_t* __restrict__ Bt, float* __restrict__ C, int M, int N, int K,
    int ldc, int tm, int tiles, int per_xcd) {
  extern __shared__ __attribute__((aligned(16))) uint16_t glds[];
  const int t = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (t >= tiles) return;
  const int m0 = (t % tm) * HM, n0 = (t / tm) * BT;
  floatx16 acc[2][4];
  lm_mainloop(At, Bt, K, m0, n0, glds, acc);
  lm_store(acc, C, M, N, ldc, m0, n0);
}

// ---------------------------------------------------------------------------
// The LM head fused with the per-depth candidate selection.  Base logits are
// the LM head applied to the draft block's hidden states (Domino summary,
// 方法步骤详情), and the tree needs only each depth's top-M of them and their
// log-sum-exp (DominoTree summary, Componenti Core 2).  So the GEMM's
// epilogue keeps, for each row and each 128 columns of its tile (a list), the
// LM_KT largest logits as (value, id) composites and the list's statistics
// (its max m and the sum of exp((x - m) / T)); the logits need not reach
// memory (41 MB of lists and statistics instead of 292 MB at 480 x 151936).
// lm_select_kernel then merges a row's lists.  A list whose LM_KT-th key still
// beats the row's M-th selected key may hold more of the row's top M than it
// listed; the merge recomputes that list's 128 logits of the row (an fp32
// dot product per column) and selects again.  At most ceil(M / LM_KT) lists can
// be in that state (each has LM_KT keys above the M-th), and once they are
// recomputed the M-th key can only rise, so one such round is enough.

constexpr int LM_COLS = 128;            // columns per list (a wave's share of a tile)
constexpr int LM_KT = 8;                // keys per list
constexpr int LM_STRIDE = LM_COLS + 4;  // staged row stride (floats)
constexpr int LM_POOL = 1024;           // merge: candidates ranked pairwise
constexpr int LM_HEADS = 24;            // merge: list heads per lane kept in registers (nl <= 1536)
constexpr int LM_REDO_CAP = 2 * (DT_TOPM_MAX + LM_KT - 1) / LM_KT;  // merge: lists recomputed at most

static_assert(4 * 32 * LM_STRIDE * 4 <= (int)HALF_LDS, "the epilogue stages 32 rows per wave in the ring");

// insert k into the descending list t (k above t's last entry)
__device__ __forceinline__ void topk_insert(uint64_t (&t)[LM_KT], uint64_t k) {
#pragma unroll
  for (int i = LM_KT - 1; i > 0; --i) t[i] = k > t[i - 1] ? t[i - 1] : (k > t[i] ? k : t[i]);
  t[0] = k > t[0] ? k : t[0];
}

// the LM_KT largest of two descending lists, descending (a bitonic merge)
__device__ __forceinline__ void topk_merge(uint64_t (&a)[LM_KT], const uint64_t (&b)[LM_KT]) {
#pragma unroll
  for (int i = 0; i < LM_KT; ++i) a[i] = a[i] > b[LM_KT - 1 - i] ? a[i] : b[LM_KT - 1 - i];
#pragma unroll
  for (int d = LM_KT / 2; d >= 1; d >>= 1)
#pragma unroll
    for (int i = 0; i < LM_KT; ++i)
      if ((i & d) == 0) {
        const uint64_t x = a[i], y = a[i + d];
        a[i] = x > y ? x : y;
        a[i + d] = x > y ? y : x;
      }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_lm_topk_kernel(
    const uint16_t* __restrict__ At, const uint16_t* __restrict__ Bt, int M, int N, int K, int tm, int tiles,
    int per_xcd, float l2t, int nl, uint64_t* __restrict__ lists, float2* __restrict__ stats, float* __restrict__ C,
    int ldc) {
  extern __shared__ __attribute__((aligned(16))) uint16_t glds[];
  const int t = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (t >= tiles) return;
  const int m0 = (t % tm) * HM, n0 = (t / tm) * BT;
  floatx16 acc[2][4];
  lm_mainloop(At, Bt, K, m0, n0, glds, acc);
  if (C) lm_store(acc, C, M, N, ldc, m0, n0);
  __syncthreads();  // every wave is done with the ring: each stages its rows in a quarter of it
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = (w >> 1) * 64, wn = (w & 1) * 128;
  float* st = reinterpret_cast<float*>(glds) + w * 32 * LM_STRIDE;
  const int lr = lane & 31, lh = lane >> 5;   // the row this lane scans, and which 64 of its columns
  const int list = 2 * (n0 / BT) + (w & 1);
  const int c0 = n0 + wn + 64 * lh;
  const int ncol = min(64, N - c0);           // columns of this lane inside the matrix (may be <= 0)
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    // stage the wave's rows 32 x .. 32 x + 31 (row-major, LM_STRIDE floats a row)
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        st[(8 * (e >> 2) + 4 * lh + (e & 3)) * LM_STRIDE + 32 * y + lr] = acc[x][y][e];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's writes are in LDS (one wave: no barrier)
    const float* srcf = st + lr * LM_STRIDE + 64 * lh;
    const float4* src = reinterpret_cast<const float4*>(srcf);
    // pass 1: the row's max over both lanes' columns, and a lower bound tau
    // of its LM_KT-th largest value: the smallest of eight group maxima (the
    // lane's four groups of 16 columns and its partner's), eight distinct
    // values at or above it (-inf when a group is empty, at the matrix edge)
    float g[4];
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      g[gi] = -INFINITY;
#pragma unroll
      for (int q = 4 * gi; q < 4 * gi + 4; ++q) {
        const float4 v = src[q];
        if (4 * q < ncol) g[gi] = fmaxf(g[gi], v.x);
        if (4 * q + 1 < ncol) g[gi] = fmaxf(g[gi], v.y);
        if (4 * q + 2 < ncol) g[gi] = fmaxf(g[gi], v.z);
        if (4 * q + 3 < ncol) g[gi] = fmaxf(g[gi], v.w);
      }
    }
    float m = fmaxf(fmaxf(g[0], g[1]), fmaxf(g[2], g[3]));
    float tau = fminf(fminf(g[0], g[1]), fminf(g[2], g[3]));
    m = fmaxf(m, __shfl_xor(m, 32));
    tau = fminf(tau, __shfl_xor(tau, 32));
    // pass 2: every term of the sum relative to the row's max (the merge
    // recomputes a listed term with the same expression), and the columns at
    // or above tau
    const float mb = m * l2t;
    float s = 0.f;
    uint64_t cmask = 0ull;
    if (m > -INFINITY) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float4 v = src[q];
        const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (4 * q + j < ncol) {
            s += __builtin_amdgcn_exp2f(__builtin_fmaf(vv[j], l2t, -mb));
            if (vv[j] >= tau) cmask |= 1ull << (4 * q + j);
          }
        }
      }
    }
    // pass 3: the candidates into the descending list
    uint64_t top[LM_KT];
#pragma unroll
    for (int i = 0; i < LM_KT; ++i) top[i] = 0ull;
    while (cmask) {
      const int q = __builtin_ctzll(cmask);
      cmask &= cmask - 1ull;
      const uint64_t k = cand_pack(f32_key(srcf[q]), (uint32_t)(c0 + q));
      if (k > top[LM_KT - 1]) topk_insert(top, k);
    }
    s += __shfl_xor(s, 32);
    uint64_t other[LM_KT];
#pragma unroll
    for (int i = 0; i < LM_KT; ++i) other[i] = shfl_xor_u64(top[i], 32);
    topk_merge(top, other);
    const int row = m0 + wm + 32 * x + lr;
    if (lh == 0 && row < M) {  // a list past the last column is written empty (m = -inf)
      uint4* o = reinterpret_cast<uint4*>(lists + ((size_t)row * nl + list) * LM_KT);
#pragma unroll
      for (int i = 0; i < LM_KT; i += 2)
        o[i / 2] = make_uint4((uint32_t)top[i], (uint32_t)(top[i] >> 32), (uint32_t)top[i + 1],
                              (uint32_t)(top[i + 1] >> 32));
      stats[(size_t)row * nl + list] = make_float2(m, s);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the reads are done before the next rows overwrite them
  }
}

// sum_k h[k] W_lm[k, col] in fp32, k ascending, from W_lm in the tiled order
// of launch_pack_b_tiles (a column's 32 k of a stage are 64 contiguous bytes,
// their four 16-byte pieces swizzled)
__device__ __forceinline__ float wlm_dot(const uint16_t* __restrict__ Bt, int nk, int col, const float* h) {
  const int nt = col / BT, r = col % BT, sw = big_swz(r & 15);
  const uint16_t* base = Bt + (size_t)nt * nk * BOPND + (size_t)r * BK;
  float acc = 0.f;
  for (int st = 0; st < nk; ++st) {
#pragma unroll
    for (int c = 0; c < BK / 8; ++c) {
      const uint4 q = *reinterpret_cast<const uint4*>(base + (size_t)st * BOPND + 8 * (c ^ sw));
      const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
      const float* hk = h + st * BK + 8 * c;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = __builtin_fmaf(hk[2 * e], __uint_as_float(wd[e] << 16), acc);
        acc = __builtin_fmaf(hk[2 * e + 1], __uint_as_float(wd[e] & 0xFFFF0000u), acc);
      }
    }
  }
  return acc;
}

// One block per row: the row's M candidates (value desc, id asc), the LSE of
// base / T over the whole row and over the tokens left out (tail), from its
// nl lists.  lists_out/stat are read; `hidden` ([rows, K] bf16 row-major) and
// Bt (W_lm tiled) serve the recomputation.  user_logits (optional) holds the
// GEMM's logits; recomputed ones are written there too.
__global__ __launch_bounds__(256) void lm_select_kernel(
    const uint64_t* __restrict__ lists, const float2* __restrict__ stats, int nl, int M, float T, float l2t,
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ Bt, int K, int N,
    int32_t* __restrict__ ids_out, float* __restrict__ vals_out, float* __restrict__ lse_out,
    float* __restrict__ tail_out, int32_t* __restrict__ tokrank_out, int32_t* __restrict__ user_ids,
    float* __restrict__ user_vals, float* __restrict__ user_lse, float* __restrict__ user_logits,
    int* __restrict__ err) {
  extern __shared__ float2 sst[];               // [nl] list statistics, [nl] lists' last keys, [nl] heads' value keys
  __shared__ uint64_t pool[LM_POOL];            // candidates
  __shared__ uint64_t best[DT_TOPM_MAX];        // the row's M, descending
  __shared__ float redo_v[LM_REDO_CAP][LM_COLS];  // recomputed lists' logits
  __shared__ int redo_l[LM_REDO_CAP];             // their list indices
  __shared__ float hrow[8192];                  // the row's hidden state (recomputation)
  __shared__ int npool, nredo, nnew, nbest;
  __shared__ uint32_t bound;
  __shared__ float red[4];
  __shared__ int ired[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int row = blockIdx.x;
  const uint64_t* L = lists + (size_t)row * nl * LM_KT;
  uint64_t* lastk = reinterpret_cast<uint64_t*>(sst + nl);   // set for the lists read into the pool
  uint32_t* hk = reinterpret_cast<uint32_t*>(lastk + nl);
  // every thread's loads in flight together
  for (int i0 = 0; i0 < nl; i0 += 256 * 8) {
    float2 sv[8];
    uint32_t hv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = min(i0 + u * 256 + tid, nl - 1);   // clamped: valid addresses
      sv[u] = stats[(size_t)row * nl + i];
      hv[u] = (uint32_t)(L[(size_t)i * LM_KT] >> 32);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * 256 + tid;
      if (i < nl) {
        sst[i] = sv[u];
        hk[i] = hv[u];
      }
    }
  }
  if (tid == 0) nredo = 0;
  __syncthreads();

  // entry j of list t: the listed keys, or the recomputed values of a redone list
  auto list_len = [&](int t, int& r) {
    r = -1;
    for (int q = 0; q < nredo; ++q)
      if (redo_l[q] == t) r = q;
    return r >= 0 ? LM_COLS : LM_KT;
  };
  auto entry = [&](int t, int r, int j) -> uint64_t {
    if (r < 0) return L[(size_t)t * LM_KT + j];
    const int col = t * LM_COLS + j;
    return col < N ? cand_pack(f32_key(redo_v[r][j]), (uint32_t)col) : 0ull;
  };

  for (int round = 0;; ++round) {
    // 1. a lower bound of the row's M-th value key: the M-th largest list head
    //    (M distinct entries reach it); wave 0 finds it bit by bit
    if (wv == 0) {
      uint32_t p = 0;
      if (nl <= 64 * LM_HEADS) {
        // the heads in registers, counted with ballots
        uint32_t hv[LM_HEADS];
#pragma unroll
        for (int j = 0; j < LM_HEADS; ++j) hv[j] = lane + 64 * j < nl ? hk[lane + 64 * j] : 0u;
        for (int b = 31; b >= 0; --b) {
          const uint32_t c = p | (1u << b);
          int cnt = 0;
#pragma unroll
          for (int j = 0; j < LM_HEADS; ++j) cnt += (int)__popcll(__ballot(hv[j] >= c));
          if (cnt >= M) p = c;
        }
      } else {
        for (int b = 31; b >= 0; --b) {
          const uint32_t c = p | (1u << b);
          int cnt = 0;
          for (int t = lane; t < nl; t += 64) cnt += hk[t] >= c;
          cnt = wave_reduce_add(cnt);
          if (cnt >= M) p = c;
        }
      }
      if (lane == 0) {
        bound = p;
        npool = 0;
      }
    }
    __syncthreads();
    // 2. every entry at or above the bound (a list's 8 keys in four 16-byte
    //    loads; a recomputed list's values from LDS)
    const uint32_t bd = bound;
    for (int t = tid; t < nl; t += 256) {
      if (hk[t] < bd) continue;
      int r;
      const int len = list_len(t, r);
      if (r < 0) {
        const uint4* src = reinterpret_cast<const uint4*>(L + (size_t)t * LM_KT);
        uint4 q[LM_KT / 2];
#pragma unroll
        for (int i = 0; i < LM_KT / 2; ++i) q[i] = src[i];
        lastk[t] = (uint64_t)q[LM_KT / 2 - 1].w << 32 | q[LM_KT / 2 - 1].z;
#pragma unroll
        for (int i = 0; i < LM_KT; ++i) {
          const uint64_t k = (i & 1) ? ((uint64_t)q[i / 2].w << 32 | q[i / 2].z) : ((uint64_t)q[i / 2].y << 32 | q[i / 2].x);
          if (k != 0ull && cand_key(k) >= bd) {
            const int slot = atomicAdd(&npool, 1);
            if (slot < LM_POOL) pool[slot] = k;
          }
        }
      } else {
        for (int j = 0; j < len; ++j) {
          const uint64_t k = entry(t, r, j);
          if (k != 0ull && cand_key(k) >= bd) {
            const int slot = atomicAdd(&npool, 1);
            if (slot < LM_POOL) pool[slot] = k;
          }
        }
      }
    }
    __syncthreads();
    const int C = npool;
    if (C <= LM_POOL) {
      // 3. exact ranks among the candidates (composites are unique)
      for (int i = tid; i < C; i += 256) {
        const uint64_t k = pool[i];
        int rk = 0;
#pragma unroll 8
        for (int j = 0; j < C; ++j) rk += pool[j] > k;
        if (rk < M) best[rk] = k;
      }
      if (tid == 0) nbest = min(C, M);
    } else {
      // 3'. many entries at the bound (equal values): the M-th largest
      //     composite bit by bit, then the entries at or above it
      uint64_t p = 0;
      for (int b = 63; b >= 0; --b) {
        const uint64_t c = p | (1ull << b);
        int cnt = 0;
        for (int t = tid; t < nl; t += 256) {
          int r;
          const int len = list_len(t, r);
          for (int j = 0; j < len; ++j) {
            const uint64_t k = entry(t, r, j);
            if (k >= c) ++cnt;
            else if (r < 0) break;
          }
        }
        cnt = block_reduce_add(cnt, ired);
        if (cnt >= M) p = c;
      }
      if (tid == 0) npool = 0;
      __syncthreads();
      for (int t = tid; t < nl; t += 256) {
        int r;
        const int len = list_len(t, r);
        for (int j = 0; j < len; ++j) {
          const uint64_t k = entry(t, r, j);
          if (k >= p && k != 0ull) {
            const int slot = atomicAdd(&npool, 1);
            if (slot < DT_TOPM_MAX) best[slot] = k;
          } else if (r < 0) {
            break;
          }
        }
      }
      __syncthreads();
      if (wv == 0) {
        uint64_t v = lane < min(npool, M) ? best[lane] : 0ull;
        v = wave_sort_desc_u64(v);
        if (lane < DT_TOPM_MAX) best[lane] = v;
      }
      if (tid == 0) nbest = min(npool, M);
    }
    __syncthreads();
    // 4. lists not yet recomputed that may hold more of the row's M than they
    //    listed: full, with their last key above the M-th
    const uint64_t kth = nbest == M ? best[M - 1] : 0ull;
    const int before = nredo;
    if (tid == 0) nnew = 0;
    __syncthreads();
    for (int t = tid; t < nl; t += 256) {
      // a list whose head is below the bound has no key above the M-th
      if (hk[t] < bd || (uint64_t)hk[t] < (kth >> 32)) continue;
      int r;
      list_len(t, r);
      if (r >= 0) continue;
      const uint64_t last = lastk[t];   // read into the pool above: its head reached the bound
      if (last != 0ull && last > kth) {
        const int q = before + atomicAdd(&nnew, 1);
        if (q < LM_REDO_CAP) redo_l[q] = t;
      }
    }
    __syncthreads();
    if (nnew == 0) break;
    if (before + nnew > LM_REDO_CAP) {
      // cannot happen: at most ceil(M / LM_KT) lists hold LM_KT keys above the
      // M-th, and recomputing them lowers the M-th only by rounding
      if (tid == 0) atomicOr(err, 16);
      break;
    }
    // 5. recompute those lists' logits of the row (fp32 dot products, k in
    //    order) and their statistics
    if (before == 0)
      for (int k = tid; k < K; k += 256) hrow[k] = bf16_to_f32(hidden[(size_t)row * K + k]);
    __syncthreads();
    const int nk = K / BK;
    for (int i = tid; i < nnew * LM_COLS; i += 256) {
      const int q = before + i / LM_COLS, j = i % LM_COLS, col = redo_l[q] * LM_COLS + j;
      const float v = col < N ? wlm_dot(Bt, nk, col, hrow) : -INFINITY;
      redo_v[q][j] = v;
      if (user_logits && col < N) user_logits[(size_t)row * N + col] = v;
    }
    __syncthreads();
    for (int q = before + wv; q < before + nnew; q += 4) {
      const int t = redo_l[q];
      float m = -INFINITY;
      for (int j = lane; j < LM_COLS; j += 64)
        if (t * LM_COLS + j < N) m = fmaxf(m, redo_v[q][j]);
      m = wave_max(m);
      float s = 0.f;
      if (m > -INFINITY)
        for (int j = lane; j < LM_COLS; j += 64)
          if (t * LM_COLS + j < N) s += __builtin_amdgcn_exp2f(__builtin_fmaf(redo_v[q][j], l2t, -m * l2t));
      s = wave_sum(s);
      if (lane == 0) {
        sst[t] = make_float2(m, s);
        hk[t] = m > -INFINITY ? f32_key(m) : 0u;   // the recomputed list's head
      }
    }
    if (tid == 0) nredo = before + nnew;
    __syncthreads();
  }

  // 6. the LSE over the row and over the tokens left out
  float mloc = -INFINITY;
  for (int i = tid; i < nl; i += 256) mloc = fmaxf(mloc, sst[i].x);
  const float mstar = block_max<256>(mloc, red);
  float s_all = 0.f;
  if (mstar > -INFINITY)
    for (int i = tid; i < nl; i += 256)
      if (sst[i].x > -INFINITY) s_all += sst[i].y * __builtin_amdgcn_exp2f((sst[i].x - mstar) * l2t);
  float s_sel = 0.f;
  const int nb = nbest;
  if (mstar > -INFINITY && tid < nb) {
    const uint64_t k = best[tid];
    const float x = key_f32(cand_key(k));
    const float mt = sst[(int)cand_id(k) / LM_COLS].x;
    s_sel = __builtin_amdgcn_exp2f(__builtin_fmaf(x, l2t, -mt * l2t)) * __builtin_amdgcn_exp2f((mt - mstar) * l2t);
  }
  s_all = block_sum<256>(s_all, red);
  s_sel = block_sum<256>(s_sel, red);
  if (tid == 0) {
    const float lse = (mstar > -INFINITY && s_all > 0.f) ? mstar / T + __logf(s_all) : -INFINITY;
    const float st = fmaxf(s_all - s_sel, 0.f);
    lse_out[row] = lse;
    tail_out[row] = (mstar > -INFINITY && st > 0.f) ? mstar / T + __logf(st) : -INFINITY;
    if (user_lse) user_lse[row] = lse;
  }
  // 7. the candidates and the rank of each one's token id among them
  if (tid < M) {
    const uint64_t k = tid < nb ? best[tid] : 0ull;
    const int id = tid < nb ? (int)cand_id(k) : 0;
    const float v = tid < nb ? key_f32(cand_key(k)) : -INFINITY;
    ids_out[(size_t)row * M + tid] = id;
    vals_out[(size_t)row * M + tid] = v;
    if (user_ids) user_ids[(size_t)row * M + tid] = id;
    if (user_vals) user_vals[(size_t)row * M + tid] = v;
    int r = 0;
#pragma unroll 8
    for (int j = 0; j < nb; ++j) r += (int)cand_id(best[j]) < id;
    tokrank_out[(size_t)row * M + tid] = r;
  }
}

int lm_lists_per_row(int N) { return 2 * ((N + BT - 1) / BT); }

bool lm_topm_ok(int M, int N, int K, int topM) {
  return gemm_b_tiles_ok(N, K) && K <= 8192 && M > 0 && topM >= 1 && topM <= DT_TOPM_MAX &&
         (size_t)lm_lists_per_row(N) * (sizeof(float2) + 8 + 4) <= 96 * 1024;
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

hipError_t launch_lm_topm_gemm(const uint16_t* A, const uint16_t* Btiled, int M, int N, int K, uint16_t* a_tiles,
                               float T, uint64_t* lists, float2* stats, float* user_logits, hipStream_t stream) {
  if (!gemm_b_tiles_ok(N, K) || M <= 0 || !a_tiles || !lists || !stats) return hipErrorInvalidValue;
  const int nk = K / BK;
  const size_t n = (size_t)((M + BT - 1) / BT) * BT * nk;
  hipLaunchKernelGGL(pack_a_tiles_kernel, dim3((unsigned)std::min<size_t>((n + 255) / 256, 4096)), dim3(256), 0,
                     stream, A, a_tiles, M, K);
  const int tm = (M + HM - 1) / HM, tiles = tm * ((N + BT - 1) / BT), per_xcd = (tiles + 7) / 8;
  hipError_t e = hipFuncSetAttribute((const void*)gemm_lm_topk_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)HALF_LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gemm_lm_topk_kernel, dim3(8 * per_xcd), dim3(256), HALF_LDS, stream, a_tiles, Btiled, M, N, K,
                     tm, tiles, per_xcd, 1.4426950408889634f / T, lm_lists_per_row(N), lists, stats, user_logits, N);
  return hipGetLastError();
}

hipError_t launch_lm_select(const uint64_t* lists, const float2* stats, int rows, int N, int K, int topM, float T,
                            const uint16_t* hidden, const uint16_t* Btiled, int32_t* ids, float* vals, float* lse,
                            float* tail, int32_t* tokrank, int32_t* user_ids, float* user_vals, float* user_lse,
                            float* user_logits, int* err, hipStream_t stream) {
  if (!lm_topm_ok(rows, N, K, topM)) return hipErrorInvalidValue;
  const int nl = lm_lists_per_row(N);
  hipLaunchKernelGGL(lm_select_kernel, dim3(rows), dim3(256), (size_t)nl * (sizeof(float2) + 8 + 4), stream, lists, stats, nl,
                     topM, T, 1.4426950408889634f / T, hidden, Btiled, K, N, ids, vals, lse, tail, tokrank, user_ids,
                     user_vals, user_lse, user_logits, err);
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

