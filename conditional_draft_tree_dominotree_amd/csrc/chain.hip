// Domino chain head over the whole vocabulary: for each draft position
// d = 1..D, dL = W2 SiLU(W1 [H_d; S]) on every token, the pick
// x_d = argmax(base_d + dL) (ties to the lowest id), then S <- GRU(S, E[x_d])
// ("Domino：在投机解码中将因果建模与自回归草稿解耦", 核心方法 and 方法步骤详情:
// the head corrects each position's block-parallel base logits with a GRU
// state advanced from the previously drafted token, each token sampled from
// the refined logits).  Sampled chains rank (base + dL) / T + g instead, g a
// standard Gumbel variate per (request, position, token) from a seeded
// Philox4x32-10 stream: the Gumbel-max rule draws x_d from
// softmax((base + dL) / T).
//
// Per position, three launches on the caller's stream:
//   1. [W_hh S~ | W1_S^T S~] for the batch (the dense-product kernels), S~ the
//      state as a matrix operand;
//   2. the correction of every token and, per block and request, the best
//      (corrected logit, token) composite: with bf16 weights on the matrix
//      cores (chain_correct_mfma_kernel, W2^T in fragment order, `a` split
//      into two bf16 terms); with fp32 weights one thread per vocabulary row
//      (chain_correct_kernel: a = SiLU(P_d + W1_S^T S~) for every request in
//      LDS as [j][b], one 16-byte broadcast read serving four requests, the
//      thread's W2^T row requested at once, one accumulator per request);
//   3. chain_pick: one block per request reduces the block composites to the
//      pick and advances the GRU state with G[pick] = E W_ih^T + b_ih (the
//      handle's table) and the product of step 1.
#include "common.h"
#include "kernels.h"

namespace dt {

constexpr int CT = 256;  // threads per block (one vocabulary row each)

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds, each multiplying words 0 and 2 by
// the two round constants and forming (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2),
// hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key advances by the two Weyl
// increments between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    if (i) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
    const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

// The noise of token v at position d of request row b is word v % 4 of
// Philox4x32-10 at counter (v / 4, d, b, 0); u = (w / 2^9 + 1/2) / 2^23 (an
// odd multiple of 2^-24 in (0, 1), exact in fp32) and g = -ln(-ln u).
__device__ __forceinline__ uint4 chain_noise_words(int v4, int d, int b, uint32_t k0, uint32_t k1) {
  return philox4x32_10(make_uint4((uint32_t)v4, (uint32_t)d, (uint32_t)b, 0u), k0, k1);
}
__device__ __forceinline__ float gumbel_of(uint32_t w) {
  const float u = (float)(w >> 9) * 0x1p-23f + 0x1p-24f;
  return -logf(-logf(u));
}
__device__ __forceinline__ uint32_t word_of(const uint4& w, int i) {
  return i == 0 ? w.x : i == 1 ? w.y : i == 2 ? w.z : w.w;
}

// Row pieces of 8 elements held in registers at once: a whole bf16 row of
// rank <= 256 (32 x 16 bytes; half of it with 32 requests), an fp32 row 64
// elements at a time.
template <typename T>
struct RowPiece;
template <>
struct RowPiece<uint16_t> {
  typedef uint4 type;
  static constexpr int CHUNK = 256;
  static __device__ __forceinline__ void unpack(const uint4& q, float (&w)[8]) {
    const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[2 * i] = __uint_as_float(u[i] << 16);
      w[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  }
};
struct F8 {
  float4 a, b;
};
template <>
struct RowPiece<float> {
  typedef F8 type;
  static constexpr int CHUNK = 64;
  static __device__ __forceinline__ void unpack(const F8& q, float (&w)[8]) {
    w[0] = q.a.x; w[1] = q.a.y; w[2] = q.a.z; w[3] = q.a.w;
    w[4] = q.b.x; w[5] = q.b.y; w[6] = q.b.z; w[7] = q.b.w;
  }
};

// One vocabulary row per thread (the grid covers V).  NB: requests handled,
// a multiple of 4 and >= B.  The row's W2^T pieces are all requested before
// the first is used, so a thread waits for memory once per chunk.
template <typename T, int NB, bool SAMPLE>
__global__ __launch_bounds__(CT) void chain_correct_kernel(const T* __restrict__ w2t, const float* __restrict__ base,
                                                           const float* __restrict__ P,
                                                           const float* __restrict__ gu, int B, int D, int d,
                                                           int V, int r, int gstride, int goff,
                                                           uint64_t* __restrict__ part, float temp, uint32_t k0,
                                                           uint32_t k1) {
  typedef typename RowPiece<T>::type Piece;
  // 32 accumulators leave room for half a bf16 row at a time
  constexpr int CH = (NB >= 32 && RowPiece<T>::CHUNK > 128) ? 128 : RowPiece<T>::CHUNK;
  __shared__ __attribute__((aligned(16))) float a[CHAIN_MAX_RANK * NB];
  __shared__ uint64_t wbest[CT / 64][NB];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int t = tid; t < r * NB; t += CT) {
    const int j = t / NB, b = t - j * NB;
    float v = 0.f;
    if (b < B) {
      const float u = P[((size_t)b * D + d) * r + j] + gu[(size_t)b * gstride + goff + j];
      v = u / (1.f + expf(-u));  // SiLU
    }
    a[t] = v;
  }
  __syncthreads();
  const int v = blockIdx.x * CT + tid;
  const int vr = min(v, V - 1);  // rows past V compute on the last row and are not kept
  float acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = 0.f;
  const Piece* row = reinterpret_cast<const Piece*>(w2t + (size_t)vr * r);
  for (int c0 = 0; c0 < r; c0 += CH) {
    Piece q[CH / 8];
#pragma unroll
    for (int i = 0; i < CH / 8; ++i)
      if (c0 + 8 * i < r) q[i] = row[c0 / 8 + i];
#pragma unroll
    for (int i = 0; i < CH / 8; ++i) {
      if (c0 + 8 * i < r) {
        float w[8];
        RowPiece<T>::unpack(q[i], w);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float4* aj = reinterpret_cast<const float4*>(&a[(c0 + 8 * i + jj) * NB]);
#pragma unroll
          for (int g = 0; g < NB / 4; ++g) {
            const float4 av = aj[g];
            acc[4 * g] = fmaf(w[jj], av.x, acc[4 * g]);
            acc[4 * g + 1] = fmaf(w[jj], av.y, acc[4 * g + 1]);
            acc[4 * g + 2] = fmaf(w[jj], av.z, acc[4 * g + 2]);
            acc[4 * g + 3] = fmaf(w[jj], av.w, acc[4 * g + 3]);
          }
        }
      }
    }
  }
  // per request: the block's best (corrected logit desc, token asc; when
  // sampling, the perturbed score)
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b < B) {
      float z = base[((size_t)b * D + d) * V + vr] + acc[b];
      if constexpr (SAMPLE) z = z / temp + gumbel_of(word_of(chain_noise_words(vr >> 2, d, b, k0, k1), vr & 3));
      const uint64_t m = wave_max_u64(v < V ? cand_pack(f32_key(z), (uint32_t)v) : 0ull);
      if (lane == 0) wbest[wv][b] = m;
    }
  }
  __syncthreads();
  if (tid < B) {
    uint64_t m = wbest[0][tid];
#pragma unroll
    for (int w = 1; w < CT / 64; ++w) m = wbest[w][tid] > m ? wbest[w][tid] : m;
    part[(size_t)tid * gridDim.x + blockIdx.x] = m;
  }
}

// bf16 weights: the product W2^T a on the matrix cores.  a (fp32) is split
// into a_hi = bf16(a) and a_lo = bf16(a - a_hi), and dL = W2^T a_hi +
// W2^T a_lo is two v_mfma_f32_32x32x16_bf16 per 16 k with fp32
// accumulation: each product is exact, and what a_hi + a_lo leaves out of a
// is below 2^-16 of it.  A wave takes 32-row tiles of W2^T (the MFMA A
// operand, read straight from memory, a tile's sixteen 16-byte loads per lane
// issued together and the next tile's before this tile's MFMAs) against the
// 32 request columns of a (the B operand, bf16 rows padded in LDS); the
// accumulator lane holds request (lane & 31) for 16 rows, so the best
// (corrected logit, token) per request is kept per lane.
typedef __bf16 chain_bf16x8 __attribute__((ext_vector_type(8)));
typedef float chain_floatx16 __attribute__((ext_vector_type(16)));
constexpr int MT = 2;                 // 32-row tiles per wave
constexpr int MROWS = 4 * MT * 32;    // rows per block
constexpr int AROW = CHAIN_MAX_RANK + 8;  // bf16 per LDS row of a_hi / a_lo (padded)

template <bool SAMPLE>
__global__ __launch_bounds__(CT) void chain_correct_mfma_kernel(const uint16_t* __restrict__ w2f,
                                                                const float* __restrict__ base,
                                                                const float* __restrict__ P,
                                                                const float* __restrict__ gu, int B, int D, int d,
                                                                int V, int r, int gstride, int goff,
                                                                uint64_t* __restrict__ part, float temp,
                                                                uint32_t k0, uint32_t k1) {
  __shared__ __attribute__((aligned(16))) uint16_t ahi[32 * AROW];
  __shared__ __attribute__((aligned(16))) uint16_t alo[32 * AROW];
  __shared__ uint64_t wbest[CT / 64][32];
  // per wave, the base logits of its current 32-row tile for every request,
  // [b][v] with rows padded to 36 floats (16-byte reads of 32 requests at one
  // v offset spread over the banks)
  __shared__ __attribute__((aligned(16))) float bstage[CT / 64][32 * 36];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int fr = lane & 31, fk = 8 * (lane >> 5);
  const int ks = r / 16;  // 16-k steps
  const int vbase = blockIdx.x * MROWS + wv * MT * 32;
  uint64_t best = 0ull;
  uint4 q[2][CHAIN_MAX_RANK / 16];
  // w2f: W2^T in fragment order (launch_pack_w2_frags): the 16-byte operand
  // pieces of the 64 lanes for (32-row tile, 16-k step) are one contiguous
  // 1 KB, so each load instruction moves eight whole 128-byte lines
  const int ntile = (V + 31) / 32;
  auto load_tile = [&](int tile, uint4 (&dst)[CHAIN_MAX_RANK / 16]) {
    const int tg = min((vbase >> 5) + tile, ntile - 1);
    const uint4* src = reinterpret_cast<const uint4*>(w2f) + (size_t)tg * ks * 64 + lane;
#pragma unroll
    for (int s = 0; s < CHAIN_MAX_RANK / 16; ++s)
      if (s < ks) dst[s] = src[s * 64];
  };
  // the first tile's W2^T loads go out before `a` is built (they do not need it)
  load_tile(0, q[0]);
  for (int t = tid; t < 32 * r; t += CT) {
    const int b = t / r, j = t - b * r;
    float v = 0.f;
    if (b < B) {
      const float u = P[((size_t)b * D + d) * r + j] + gu[(size_t)b * gstride + goff + j];
      v = u / (1.f + expf(-u));  // SiLU
    }
    const uint16_t hi = f32_to_bf16(v);
    ahi[b * AROW + j] = hi;
    alo[b * AROW + j] = f32_to_bf16(v - bf16_to_f32(hi));
  }
  __syncthreads();
#pragma unroll
  for (int tile = 0; tile < MT; ++tile) {
    if (tile + 1 < MT) load_tile(tile + 1, q[(tile + 1) & 1]);
    chain_floatx16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
    for (int s = 0; s < CHAIN_MAX_RANK / 16; ++s) {
      if (s < ks) {
        const chain_bf16x8 av = *reinterpret_cast<const chain_bf16x8*>(&q[tile & 1][s]);
        const chain_bf16x8 bh = *reinterpret_cast<const chain_bf16x8*>(&ahi[fr * AROW + 16 * s + fk]);
        const chain_bf16x8 bl = *reinterpret_cast<const chain_bf16x8*>(&alo[fr * AROW + 16 * s + fk]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bl, acc, 0, 0, 0);
      }
    }
    // the tile's base logits, read row by row (128 contiguous bytes per
    // request): load i brings requests 8 i .. 8 i + 7, lane l request
    // 8 i + l / 8, rows 4 (l % 8) .. + 3
    const int v0 = vbase + tile * 32;
    float* bs = bstage[wv];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = 8 * i + (lane >> 3), vv = v0 + 4 * (lane & 7);
      if (8 * i < B) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (b < B) {
          const float* brow = base + ((size_t)b * D + d) * V;
          if ((V & 3) == 0 && vv + 3 < V) {
            x = *reinterpret_cast<const float4*>(brow + vv);  // 16-byte aligned: V % 4 == 0
          } else {
            x.x = vv < V ? brow[vv] : 0.f;
            x.y = vv + 1 < V ? brow[vv + 1] : 0.f;
            x.z = vv + 2 < V ? brow[vv + 2] : 0.f;
            x.w = vv + 3 < V ? brow[vv + 3] : 0.f;
          }
        }
        *reinterpret_cast<float4*>(&bs[b * 36 + 4 * (lane & 7)]) = x;
      }
    }
    // lane: request fr, rows 8 (e / 4) + 4 (lane >> 5) + (e % 4) of the tile
    // (the stage is this wave's own: its writes are visible to its reads)
    if (fr < B) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 bv = *reinterpret_cast<const float4*>(&bs[fr * 36 + 8 * g + 4 * (lane >> 5)]);
        const float bb[4] = {bv.x, bv.y, bv.z, bv.w};
        // the four rows are the tokens of one noise counter
        uint4 nw = make_uint4(0u, 0u, 0u, 0u);
        if constexpr (SAMPLE) nw = chain_noise_words((v0 + 8 * g + 4 * (lane >> 5)) >> 2, d, fr, k0, k1);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int e = 4 * g + q;
          const int v = v0 + 8 * g + 4 * (lane >> 5) + q;
          if (v < V) {
            float z = bb[q] + acc[e];
            if constexpr (SAMPLE) z = z / temp + gumbel_of(word_of(nw, q));
            const uint64_t c = cand_pack(f32_key(z), (uint32_t)v);
            best = c > best ? c : best;
          }
        }
      }
    }
  }
  // lanes l and l + 32 hold the same request
  const uint64_t o = shfl_xor_u64(best, 32);
  best = o > best ? o : best;
  if (lane < 32) wbest[wv][lane] = best;
  __syncthreads();
  if (tid < B) {
    uint64_t m = wbest[0][tid];
#pragma unroll
    for (int w = 1; w < CT / 64; ++w) m = wbest[w][tid] > m ? wbest[w][tid] : m;
    part[(size_t)tid * gridDim.x + blockIdx.x] = m;
  }
}

// S <- GRU(S, x) for one request, the input term gi = W_ih x + b_ih given
// (a row of G): gate rows (r, z, n), the reset gate on (W_hn S + b_hn),
// S' = (1 - z) n + z S; S' also goes to s_op (bf16, nearest-even, or fp32)
// and, when given, to out.  One block; gh = W_hh S~ (no bias).
template <typename T>
__device__ __forceinline__ void gru_advance(const float* __restrict__ gi, const float* __restrict__ gh,
                                            const float* __restrict__ b_hh, int ds, float* __restrict__ s,
                                            T* __restrict__ s_op, float* __restrict__ out) {
  for (int i = threadIdx.x; i < ds; i += blockDim.x) {
    const float hr = gh[i] + (b_hh ? b_hh[i] : 0.f);
    const float hz = gh[ds + i] + (b_hh ? b_hh[ds + i] : 0.f);
    const float hn = gh[2 * ds + i] + (b_hh ? b_hh[2 * ds + i] : 0.f);
    const float rg = 1.f / (1.f + expf(-(gi[i] + hr)));
    const float zg = 1.f / (1.f + expf(-(gi[ds + i] + hz)));
    const float ng = tanhf(gi[2 * ds + i] + rg * hn);
    const float sn = (1.f - zg) * ng + zg * s[i];
    s[i] = sn;
    if constexpr (sizeof(T) == 2) s_op[i] = f32_to_bf16(sn);  // bf16 operand, nearest-even
    else s_op[i] = sn;
    if (out) out[i] = sn;
  }
}

// The pick of request b (one block each): the largest block composite; then,
// for a sampled chain, the pick's corrected logit base + W2[:, x] . a
// recomputed (the composite holds its perturbed score); then the state.
template <typename T>
__global__ __launch_bounds__(CT) void chain_pick_kernel(const uint64_t* __restrict__ part, int nblk, int V,
                                                        const float* __restrict__ G, const float* __restrict__ gu,
                                                        const float* __restrict__ b_hh, int gstride, int ds,
                                                        int D, int d, int advance, float* __restrict__ s,
                                                        T* __restrict__ s_op, int32_t* __restrict__ tokens,
                                                        float* __restrict__ logits, int sample,
                                                        const T* __restrict__ w2t, const float* __restrict__ base,
                                                        const float* __restrict__ P, int r, int goff) {
  __shared__ uint64_t wm[CT / 64];
  __shared__ uint64_t pick;
  __shared__ float wsum[CT / 64];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint64_t m = 0ull;
  for (int i = tid; i < nblk; i += CT) {
    const uint64_t c = part[(size_t)b * nblk + i];
    m = c > m ? c : m;
  }
  m = wave_max_u64(m);
  if (lane == 0) wm[wv] = m;
  __syncthreads();
  if (tid == 0) {
    uint64_t x = wm[0];
    for (int w = 1; w < CT / 64; ++w) x = wm[w] > x ? wm[w] : x;
    pick = x;
    tokens[(size_t)b * D + d] = (int32_t)cand_id(x);
    if (logits && !sample) logits[(size_t)b * D + d] = key_f32(cand_key(x));
  }
  __syncthreads();
  if (sample && logits) {
    const size_t x = min(cand_id(pick), (uint32_t)(V - 1));
    float acc = 0.f;
    for (int j = tid; j < r; j += CT) {
      const float u = P[((size_t)b * D + d) * r + j] + gu[(size_t)b * gstride + goff + j];
      float w;
      if constexpr (sizeof(T) == 2) w = bf16_to_f32(w2t[x * r + j]);
      else w = w2t[x * r + j];
      acc = fmaf(w, u / (1.f + expf(-u)), acc);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) wsum[wv] = acc;
    __syncthreads();
    if (tid == 0) logits[(size_t)b * D + d] = base[((size_t)b * D + d) * V + x] + ((wsum[0] + wsum[1]) + (wsum[2] + wsum[3]));
  }
  if (!advance) return;
  gru_advance<T>(G + (size_t)min(cand_id(pick), (uint32_t)(V - 1)) * 3 * ds, gu + (size_t)b * gstride, b_hh, ds,
                 s + (size_t)b * ds, s_op + (size_t)b * ds, nullptr);
}

// Fold one committed token per request into the state: S <- GRU(S, E[token])
// (token ids clamped to 0..V-1); `out`, when given, also receives S.
template <typename T>
__global__ __launch_bounds__(CT) void fold_step_kernel(const int32_t* __restrict__ tokens, int L, int t, int V,
                                                       const float* __restrict__ G, const float* __restrict__ gu,
                                                       const float* __restrict__ b_hh, int gstride, int ds,
                                                       float* __restrict__ s, T* __restrict__ s_op,
                                                       float* __restrict__ out) {
  const int b = blockIdx.x;
  const int tok = min(max(tokens[(size_t)b * L + t], 0), V - 1);
  gru_advance<T>(G + (size_t)tok * 3 * ds, gu + (size_t)b * gstride, b_hh, ds, s + (size_t)b * ds,
                 s_op + (size_t)b * ds, out ? out + (size_t)b * ds : nullptr);
}

template <typename T>
__global__ void chain_init_kernel(const float* __restrict__ root, int n, float* __restrict__ s, T* __restrict__ s_op) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const float v = root ? root[i] : 0.f;
    s[i] = v;
    if constexpr (sizeof(T) == 2) s_op[i] = f32_to_bf16(v);
    else s_op[i] = v;
  }
}

// W2^T [V, r] bf16 -> fragment order [ceil(V / 32)][r / 16][64 lanes][8]:
// lane l of (tile t, step s) holds row 32 t + (l & 31), k 16 s + 8 (l >> 5)
// .. + 7 (the v_mfma_f32_32x32x16_bf16 A-operand piece); rows past V zero.
__global__ void pack_w2_frags_kernel(const uint16_t* __restrict__ w2t, uint16_t* __restrict__ out, int V, int r) {
  const int ks = r / 16;
  const size_t n = (size_t)((V + 31) / 32) * ks * 64;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const int l = (int)(i & 63);
    const size_t ts = i >> 6;
    const int st = (int)(ts % ks);
    const size_t t = ts / ks;
    const size_t row = t * 32 + (l & 31);
    uint4 q = make_uint4(0, 0, 0, 0);
    if (row < (size_t)V) q = *reinterpret_cast<const uint4*>(w2t + row * r + 16 * st + 8 * (l >> 5));
    reinterpret_cast<uint4*>(out)[i] = q;
  }
}

size_t chain_w2_frags_elems(int V, int r) { return (size_t)((V + 31) / 32) * 32 * r; }

hipError_t launch_pack_w2_frags(const uint16_t* w2t, uint16_t* out, int V, int r, hipStream_t stream) {
  if (r % 16 || r > CHAIN_MAX_RANK) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_w2_frags_kernel, dim3(2048), dim3(256), 0, stream, w2t, out, V, r);
  return hipGetLastError();
}

int chain_blocks(int V) { return (V + CT - 1) / CT; }
int chain_mfma_blocks(int V) { return (V + MROWS - 1) / MROWS; }

hipError_t launch_fold(const ChainArgs& c, const int32_t* tokens, int L, float* out, hipStream_t stream) {
  if (c.B < 1 || L < 1) return hipErrorInvalidValue;
  const int gstride = 3 * c.ds + c.r, n = c.B * c.ds;
  if (c.bf16)
    hipLaunchKernelGGL(chain_init_kernel<uint16_t>, dim3((n + 255) / 256), dim3(256), 0, stream, c.root, n, c.s,
                       (uint16_t*)c.s_op);
  else
    hipLaunchKernelGGL(chain_init_kernel<float>, dim3((n + 255) / 256), dim3(256), 0, stream, c.root, n, c.s,
                       (float*)c.s_op);
  hipError_t e = hipGetLastError();
  for (int t = 0; t < L && e == hipSuccess; ++t) {
    // W_hh S~ (the first 3 ds rows of the row-major [W_hh ; W1_S^T])
    e = c.bf16 ? launch_gemm_bf16((const uint16_t*)c.s_op, nullptr, (const uint16_t*)c.wc, nullptr, c.gu, c.B,
                                  3 * c.ds, c.ds, gstride, stream)
               : launch_gemm_f32((const float*)c.s_op, nullptr, (const float*)c.wc, nullptr, c.gu, c.B, 3 * c.ds,
                                 c.ds, gstride, stream);
    if (e != hipSuccess) return e;
    float* o = t + 1 == L ? out : nullptr;
    if (c.bf16)
      hipLaunchKernelGGL(fold_step_kernel<uint16_t>, dim3(c.B), dim3(CT), 0, stream, tokens, L, t, c.V, c.G, c.gu,
                         c.b_hh, gstride, c.ds, c.s, (uint16_t*)c.s_op, o);
    else
      hipLaunchKernelGGL(fold_step_kernel<float>, dim3(c.B), dim3(CT), 0, stream, tokens, L, t, c.V, c.G, c.gu,
                         c.b_hh, gstride, c.ds, c.s, (float*)c.s_op, o);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_chain(const ChainArgs& c, hipStream_t stream) {
  if (c.B < 1 || c.B > 32 || c.r < 8 || c.r > CHAIN_MAX_RANK || c.r % 8) return hipErrorInvalidValue;
  const int nblk = chain_blocks(c.V), gstride = 3 * c.ds + c.r, goff = 3 * c.ds;
  const int n = c.B * c.ds;
  if (c.bf16)
    hipLaunchKernelGGL(chain_init_kernel<uint16_t>, dim3((n + 255) / 256), dim3(256), 0, stream, c.root, n, c.s,
                       (uint16_t*)c.s_op);
  else
    hipLaunchKernelGGL(chain_init_kernel<float>, dim3((n + 255) / 256), dim3(256), 0, stream, c.root, n, c.s,
                       (float*)c.s_op);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int d = 0; d < c.D; ++d) {
    // 1. [W_hh S~ | W1_S^T S~]
    e = c.bf16 ? launch_gemm_bf16((const uint16_t*)c.s_op, nullptr, (const uint16_t*)c.wc, nullptr, c.gu, c.B,
                                  gstride, c.ds, gstride, stream)
               : launch_gemm_f32((const float*)c.s_op, nullptr, (const float*)c.wc, nullptr, c.gu, c.B, gstride,
                                 c.ds, gstride, stream);
    if (e != hipSuccess) return e;
    // 2. corrected logits of every token, block-wise best per request
#define CHAIN_CORRECT(T, NB)                                                                                   \
  do {                                                                                                         \
    if (c.sample)                                                                                              \
      hipLaunchKernelGGL((chain_correct_kernel<T, NB, true>), dim3(nblk), dim3(CT), 0, stream, (const T*)c.w2t, \
                         c.base, c.P, c.gu, c.B, c.D, d, c.V, c.r, gstride, goff, c.part, c.temperature, c.key0, \
                         c.key1);                                                                              \
    else                                                                                                       \
      hipLaunchKernelGGL((chain_correct_kernel<T, NB, false>), dim3(nblk), dim3(CT), 0, stream,                 \
                         (const T*)c.w2t, c.base, c.P, c.gu, c.B, c.D, d, c.V, c.r, gstride, goff, c.part, 1.f, \
                         0u, 0u);                                                                              \
  } while (0)
    if (c.w2f) {
      if (c.sample)
        hipLaunchKernelGGL(chain_correct_mfma_kernel<true>, dim3(chain_mfma_blocks(c.V)), dim3(CT), 0, stream,
                           (const uint16_t*)c.w2f, c.base, c.P, c.gu, c.B, c.D, d, c.V, c.r, gstride, goff, c.part,
                           c.temperature, c.key0, c.key1);
      else
        hipLaunchKernelGGL(chain_correct_mfma_kernel<false>, dim3(chain_mfma_blocks(c.V)), dim3(CT), 0, stream,
                           (const uint16_t*)c.w2f, c.base, c.P, c.gu, c.B, c.D, d, c.V, c.r, gstride, goff, c.part,
                           1.f, 0u, 0u);
    } else if (c.bf16) {
      if (c.B <= 4) CHAIN_CORRECT(uint16_t, 4);
      else if (c.B <= 8) CHAIN_CORRECT(uint16_t, 8);
      else if (c.B <= 16) CHAIN_CORRECT(uint16_t, 16);
      else CHAIN_CORRECT(uint16_t, 32);
    } else {
      if (c.B <= 4) CHAIN_CORRECT(float, 4);
      else if (c.B <= 8) CHAIN_CORRECT(float, 8);
      else if (c.B <= 16) CHAIN_CORRECT(float, 16);
      else CHAIN_CORRECT(float, 32);
    }
#undef CHAIN_CORRECT
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // 3. the pick, then the state for the next position
    const int adv = d + 1 < c.D;
    const int np = c.w2f ? chain_mfma_blocks(c.V) : nblk;
    if (c.bf16)
      hipLaunchKernelGGL(chain_pick_kernel<uint16_t>, dim3(c.B), dim3(CT), 0, stream, c.part, np, c.V, c.G, c.gu,
                         c.b_hh, gstride, c.ds, c.D, d, adv, c.s, (uint16_t*)c.s_op, c.tokens, c.logits, c.sample,
                         (const uint16_t*)c.w2t, c.base, c.P, c.r, goff);
    else
      hipLaunchKernelGGL(chain_pick_kernel<float>, dim3(c.B), dim3(CT), 0, stream, c.part, np, c.V, c.G, c.gu,
                         c.b_hh, gstride, c.ds, c.D, d, adv, c.s, (float*)c.s_op, c.tokens, c.logits, c.sample,
                         (const float*)c.w2t, c.base, c.P, c.r, goff);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dt
