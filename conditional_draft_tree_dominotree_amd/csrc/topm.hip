// Per-depth candidate selection: the M largest base logits of each
// (request, depth) row, ties to the lowest token id, plus the log-sum-exp of
// base/T over the whole vocabulary and over the tokens left out ("tail").
//
// DominoTree technical summary, Componenti Core 2: the correction is applied
// only to each depth's top-M marginal candidates.  The selection is pure
// comparison on the fp32 inputs, so it is exact; only the two LSE values are
// rounded.
//
// Kernels.  topm_chunk: one 256-thread block per (row, chunk of 8192 tokens)
// item; the block reads its item once from HBM into registers (32 values per
// thread, 16-byte loads), and the several blocks resident on a CU overlap one
// block's loads with another's selection.  Each wave bounds the ceil(M/4)-th
// largest of its 64 per-thread maxima from below (a bit search over ballots,
// to 16 key bits); the smallest of the four wave values bounds the
// chunk's M-th largest value from below (at least M threads reach it), so the
// keys at or above it -- typically a few more than M -- hold the chunk's
// top-M; they are ranked exactly as (value desc, id asc) composites.  When
// more than 512 keys reach that bound (many equal values), an exact radix
// select over the same registers (four 8-bit passes, ties at the threshold
// taken in id order) replaces the ranking.  The chunk's LSE statistics come
// from the same registers.  topm_merge: one block per row bounds the row's
// M-th key from below by the M-th largest of the first few entries of every
// chunk list, ranks the keys at or above the bound against each other and
// keeps the M best; the LSE statistics combine exactly (a token left out of
// its chunk's list is left out of the row's).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dt {

constexpr int TOPM_THREADS = 256;

// A block barrier for LDS only: the block's LDS operations complete, then
// s_barrier.  __syncthreads also waits for the block's outstanding global
// memory operations (one counter covers loads and stores), which would wait
// for loads meant to stay in flight across the barrier; the barriers here
// order LDS accesses only (global results are read by later launches).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

constexpr int PER_THREAD = TOPM_CHUNK / TOPM_THREADS;  // 32 values per thread
constexpr int FAST_CAP = 512;                          // candidates the fast path ranks
constexpr int MERGE_SUB = 320;   // merge: subset keys for the bound (S (M / S + 2) <= M + 2 S)
constexpr int MERGE_CAP = 1024;  // merge: candidates ranked pairwise

// Inclusive add-scan over the lanes of a wave: doubling shifts within each
// row of 16, then each row adds the totals of the rows before it.
__device__ __forceinline__ int wave_add_scan_incl(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 to rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 to rows 2, 3
  return v;
}

// Largest key of the wave (every lane gets it).
__device__ __forceinline__ uint32_t wave_max_key(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));
  const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 15), (uint32_t)__builtin_amdgcn_readlane((int)v, 31));
  const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 47), (uint32_t)__builtin_amdgcn_readlane((int)v, 63));
  return max(a, b);
}

// A lower bound of the m-th largest of the wave's 64 keys (1 <= m <= 64):
// the largest c whose low LOW bits are zero with at least m keys >= c, built
// bit by bit from the top (LOW = 0: the m-th largest itself).
template <int LOW>
__device__ __forceinline__ uint32_t wave_kth_largest(uint32_t v, int m) {
  uint32_t p = 0;
#pragma unroll
  for (int b = 31; b >= LOW; --b) {
    const uint32_t c = p | (1u << b);
    if ((int)__popcll(__ballot(v >= c)) >= m) p = c;
  }
  return p;
}

// Exclusive prefix sum over the threads of the block in thread order, and
// the block total.  `red` holds 4 ints.
__device__ __forceinline__ int block_prefix_excl(int v, int* red, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = wave_add_scan_incl(v);
  lds_barrier();
  if (lane == 63) red[w] = incl;
  lds_barrier();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < TOPM_THREADS / 64; ++i) {
    before += i < w ? red[i] : 0;
    tot += red[i];
  }
  *total = tot;
  return before + incl - v;
}

struct ChunkLds {
  uint64_t sel[FAST_CAP];        // keys at or above the threshold; radix histogram of the exact path
  uint64_t list[DT_TOPM_MAX];    // the chunk's Mc best, sorted
  uint32_t wb[4], wm[4];         // per wave: threshold bound, largest key
  float ws[4];                   // per wave: sum of exp
  int wi[4];                     // scan totals
  int sel_count, digit, above;
};

// Item = (row, chunk): element tid*4 + 1024 j + e of the chunk goes to
// x[4 j + e] of thread tid (coalesced float4 pieces when VEC4).  Loads past
// the chunk's end are clamped to its last element (every load stays in
// bounds) and the values are then replaced by -inf.  The logits are read
// once per round: non-temporal loads (nt) keep them from evicting what the
// tree build reads from the caches (measured: candidates 68 -> 60 us, tree
// kernel 262 -> 258 us, and a round after a 512 MB write 0.378 -> 0.327 ms at
// the Qwen3-8B shape with 32 requests).
template <bool VEC4>
__device__ __forceinline__ void chunk_load(const float* __restrict__ src, int len, float (&x)[PER_THREAD]) {
  const int tid = threadIdx.x;
  if (VEC4) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4* s4 = reinterpret_cast<const f32x4*>(src);
    const int n4 = len >> 2;  // V is a multiple of 4
#pragma unroll
    for (int j = 0; j < PER_THREAD / 4; ++j) {
      const f32x4 v = __builtin_nontemporal_load(s4 + min(j * TOPM_THREADS + tid, n4 - 1));
      x[4 * j] = v.x;
      x[4 * j + 1] = v.y;
      x[4 * j + 2] = v.z;
      x[4 * j + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < PER_THREAD / 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        x[4 * j + e] = __builtin_nontemporal_load(src + min((j * TOPM_THREADS + tid) * 4 + e, len - 1));
  }
  if (len < TOPM_CHUNK) {
    const int lim = len - 4 * tid;
#pragma unroll
    for (int q = 0; q < PER_THREAD; ++q)
      if (!(((q >> 2) * (4 * TOPM_THREADS) + (q & 3)) < lim)) x[q] = -INFINITY;
  }
}

// The per-round product P = H W1_H (the path-independent half of the
// correction's first projection: H_d is shared by every path, DominoTree
// summary, Componenti Core 1), launched as extra blocks behind the rows of
// the candidate merge, whose latency-bound blocks leave the CUs room (in the
// chunk kernel its registers would cut that kernel's occupancy).  K is split
// P_KSPLIT ways over blocks: a block computes one 32 x 32 output tile over
// its K share, its four waves splitting the share again (512 k each at
// h = 4096 with two shares), so that a wave issues the loads of 256 k at once
// (16 bytes a lane, straight from memory, 16 rows x 64 bytes per load
// instruction) and waits for memory about once per 256 k: with only a 64-k
// step's products (about 128 cycles) to cover each load, a wave walking its
// share 64 k at a time would pay one memory latency per step.  The four
// waves' tiles are summed in LDS in a fixed order and the block writes
// partial kz of P; the consumer adds the P_KSPLIT partials in a fixed order.
// Two shares rather than four or eight: the tree kernel's prefetch adds
// fewer partials, and the launch stays as short (measured by the round: one
// share 0.325, two 0.318, four 0.320, eight 0.336 ms at the Qwen3-8B shape
// with 32 requests).
typedef float floatx16 __attribute__((ext_vector_type(16)));

struct PArgs {
  const uint16_t* A;   // H [M, K] bf16
  const uint16_t* Bt;  // W1_H^T [N, K] bf16
  float* C;            // P partials [P_KSPLIT][M, N] fp32
  int M, N, K;
  int blocks;          // output tiles x P_KSPLIT (0: no P blocks)
};

// 8 bf16 of a row at k0, or zeros past the rows or past kend (K and kend
// multiples of 8).  The load itself is unconditional, from a clamped address
// that is always in bounds, so that the loads of a step carry no branch and
// stay in flight together.
__device__ __forceinline__ uint4 p_load8(const uint16_t* base, int row, int rows, int k0, int kend, int K) {
  const uint32_t m = (row < rows && k0 < kend) ? 0xFFFFFFFFu : 0u;  // a mask, not a branch around the load
  const uint4 v = *reinterpret_cast<const uint4*>(base + (size_t)min(row, rows - 1) * K + min(k0, kend - 8));
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

__device__ __forceinline__ void p_tile(const PArgs& pa, int blk, float* part /* [4][1024] */) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int tile = blk / P_KSPLIT, kz = blk - tile * P_KSPLIT;
  const int tn = (pa.N + 31) / 32;
  const int m0 = (tile / tn) * 32, n0 = (tile % tn) * 32;
  const int K = pa.K;
  constexpr int NS = 4;                                       // 64-k steps whose loads go out together
  const int kblk = ((K + P_KSPLIT - 1) / P_KSPLIT + 255) / 256 * 256;  // k per block, a multiple of 4 x 64
  const int kw = kblk / 4;                                    // k per wave, a multiple of 64
  const int kb = min(K, kz * kblk + w * kw), ke = min(K, kb + kw);
  // v_mfma_f32_16x16x32_bf16 on the four 16 x 16 quarters of the tile: lane
  // l holds row (l & 15) at k 8 (l >> 4) of each 32-k half step
  const int r16 = lane & 15, ko = 8 * (lane >> 4);
  floatx4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int k = kb; k < ke; k += 64 * NS) {
    uint4 ra[NS][2][2], rb[NS][2][2];  // [step][row or column half][32-k half]
#pragma unroll
    for (int d = 0; d < NS; ++d)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          ra[d][h][q] = p_load8(pa.A, m0 + 16 * h + r16, pa.M, k + 64 * d + 32 * q + ko, ke, K);
          rb[d][h][q] = p_load8(pa.Bt, n0 + 16 * h + r16, pa.N, k + 64 * d + 32 * q + ko, ke, K);
        }
#pragma unroll
    for (int d = 0; d < NS; ++d)
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(&ra[d][i][q]),
                                                                *reinterpret_cast<const bf16x8*>(&rb[d][j][q]),
                                                                acc[i][j], 0, 0, 0);
  }
  // lane: column (lane & 15), rows 4 (lane >> 4) + e of each quarter
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        part[w * 1024 + (16 * i + 4 * (lane >> 4) + e) * 32 + 16 * j + r16] = acc[i][j][e];
  __syncthreads();
  float* C = pa.C + (size_t)kz * pa.M * pa.N;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = tid + 256 * u;
    const float v = (part[i] + part[1024 + i]) + (part[2048 + i] + part[3072 + i]);
    const int row = m0 + i / 32, col = n0 + i % 32;
    if (row < pa.M && col < pa.N) C[(size_t)row * pa.N + col] = v;
  }
}

// One block per item.  The selection works on the fp32 values with float
// compares (a key per element only for the few candidates): per element a
// max, a compare with the threshold and one exp.
// One item's selection from its values in registers (x, loaded by
// chunk_load); uses L and ends with the block's LDS reads done.
template <bool VEC4>
__device__ __forceinline__ void chunk_select(ChunkLds& L, const float* __restrict__ logits, int V, int S, int M,
                                             float T, int item, float (&x)[PER_THREAD],
                                             uint64_t* __restrict__ out_cand, float4* __restrict__ out_stat) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int row = item / S, c = item - row * S;
  const int c0 = c * TOPM_CHUNK, len = min(TOPM_CHUNK, V - c0), Mc = min(M, len);
  const float* src = logits + (size_t)row * (size_t)V + c0;
  // element q of this thread is chunk element 4 tid + off(q)
  auto off = [](int q) { return (q >> 2) * (4 * TOPM_THREADS) + (q & 3); };
  const uint32_t id0 = (uint32_t)(c0 + 4 * tid);
  // 1. threshold: in each wave a lower bound of the ceil(Mc/4)-th largest
  //    lane maximum, to 16 bits of its key (the sign, the exponent and the top
  //    7 mantissa bits: half the search steps, a few more candidates); the
  //    smallest of the four bounds the chunk's Mc-th largest value from below
  //    (at least 4 ceil(Mc/4) >= Mc threads have a maximum at or above it)
  float vmax = x[0];
#pragma unroll
  for (int q = 1; q < PER_THREAD; ++q) vmax = fmaxf(vmax, x[q]);  // NaN is dropped
  const uint32_t kmax = f32_key(vmax);
  const uint32_t wbound = wave_kth_largest<16>(kmax, (Mc + 3) >> 2);
  const uint32_t wtop = wave_max_key(kmax);
  if (lane == 0) {
    L.wb[wv] = wbound;
    L.wm[wv] = wtop;
  }
  if (tid == 0) L.sel_count = 0;
  lds_barrier();
  const uint32_t tau = min(min(L.wb[0], L.wb[1]), min(L.wb[2], L.wb[3]));
  const uint32_t ktop = max(max(L.wm[0], L.wm[1]), max(L.wm[2], L.wm[3]));
  const float vm = ktop > 0x007FFFFFu ? key_f32(ktop) : -INFINITY;  // the chunk's largest value
  // a bound above -inf: the candidates are the values >= tau_f (no -inf, no
  // NaN, no padding); else the exact path
  const bool fast = tau > 0x007FFFFFu;
  const float tau_f = fast ? key_f32(tau) : INFINITY;
  // 2. compaction of the candidates: the wave's count from ballots, one LDS
  //    atomic per wave, then each element q's candidates written at the
  //    wave's running position plus their rank among the lanes (the order in
  //    sel does not matter: the keys are ranked by value below)
  // (the wave's count: each lane counts its own hits, one DPP scan adds them)
  int hits = 0;
#pragma unroll
  for (int q = 0; q < PER_THREAD; ++q) hits += x[q] >= tau_f;
  const int wtot = __builtin_amdgcn_readlane(wave_add_scan_incl(hits), 63);
  int base = 0;
  if (lane == 0 && wtot > 0) base = atomicAdd(&L.sel_count, wtot);
  int pos = __builtin_amdgcn_readfirstlane(base);
  if (wtot > 0) {
#pragma unroll
    for (int q = 0; q < PER_THREAD; ++q) {
      const bool h = x[q] >= tau_f;
      const unsigned long long hm = __ballot(h);
      if (hm) {  // wave-uniform: most elements of a wave have no candidate
        const int p = pos + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(hm >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((unsigned)hm, 0u));
        if (h && p < FAST_CAP) L.sel[p] = cand_pack(f32_key(x[q]), id0 + (uint32_t)off(q));
        pos += (int)__popcll(hm);
      }
    }
  }
  // 3. the chunk's sum of exp(x/T - m) (-inf adds 0); each term is
  //    exp2(fma(x, log2(e)/T, -mb)), the same expression as the listed terms'
  //    below, so that the tail (chunk sum minus listed terms) cancels them
  //    term for term
  const float l2t = 1.4426950408889634f / T;  // exp(y / T) = exp2(y * log2(e) / T)
  const float mb = vm * l2t;
  float s_all = 0.f;
  if (vm > -INFINITY) {
#pragma unroll
    for (int q = 0; q < PER_THREAD; ++q) s_all += __builtin_amdgcn_exp2f(__builtin_fmaf(x[q], l2t, -mb));
  }
  s_all = wave_sum_dpp(s_all);
  if (lane == 0) L.ws[wv] = s_all;
  lds_barrier();
  const int cnt = L.sel_count;
  if (fast && cnt <= FAST_CAP) {
    // 4. rank the candidates exactly (composite keys are unique)
    uint64_t mine[FAST_CAP / TOPM_THREADS];
    int rk[FAST_CAP / TOPM_THREADS];
#pragma unroll
    for (int u = 0; u < FAST_CAP / TOPM_THREADS; ++u) {
      const int e = tid + u * TOPM_THREADS;
      mine[u] = e < cnt ? L.sel[e] : ~0ull;
      rk[u] = 0;
    }
    const ulonglong2* s2 = reinterpret_cast<const ulonglong2*>(L.sel);
    const int pairs = cnt >> 1;
    if (cnt <= TOPM_THREADS) {
      // only the waves that hold candidates rank (typically just the first)
      if (wv * 64 < cnt) {
        for (int i = 0; i < pairs; ++i) {
          const ulonglong2 o = s2[i];
          rk[0] += (o.x > mine[0]) + (o.y > mine[0]);
        }
        if (cnt & 1) rk[0] += L.sel[cnt - 1] > mine[0];
      }
    } else {
      for (int i = 0; i < pairs; ++i) {
        const ulonglong2 o = s2[i];
#pragma unroll
        for (int u = 0; u < FAST_CAP / TOPM_THREADS; ++u) rk[u] += (o.x > mine[u]) + (o.y > mine[u]);
      }
      if (cnt & 1) {
        const uint64_t o = L.sel[cnt - 1];
#pragma unroll
        for (int u = 0; u < FAST_CAP / TOPM_THREADS; ++u) rk[u] += o > mine[u];
      }
    }
#pragma unroll
    for (int u = 0; u < FAST_CAP / TOPM_THREADS; ++u) {
      const int e = tid + u * TOPM_THREADS;
      if (e < cnt && rk[u] < Mc) L.list[rk[u]] = mine[u];  // ranks < Mc are distinct
    }
  } else {
    // 4'. exact select (many equal values, or fewer than Mc finite ones):
    //     radix passes of 8 bits over the chunk, read again from memory, find
    //     the Mc-th largest key kstar; the keys above it and the first `need`
    //     keys equal to it (lowest ids) form the list
    uint32_t* hist = reinterpret_cast<uint32_t*>(L.sel);
    uint32_t prefix = 0, pmask = 0;
    int need = Mc;
    for (int sh = 24; sh >= 0; sh -= 8) {
      hist[tid] = 0;
      lds_barrier();
      for (int i = tid; i < len; i += TOPM_THREADS) {
        const uint32_t k = f32_key(src[i]);
        if ((k & pmask) == prefix) atomicAdd(&hist[(k >> sh) & 255u], 1u);
      }
      lds_barrier();
      const int h = (int)hist[tid];
      const int above = block_suffix_excl<TOPM_THREADS>(h, L.wi);  // keys with a larger digit
      if (above < need && above + h >= need) {
        L.digit = tid;
        L.above = above;
      }
      lds_barrier();
      need -= L.above;
      prefix |= (uint32_t)L.digit << sh;
      pmask |= 255u << sh;
    }
    const uint32_t kstar = prefix;
    if (tid == 0) L.sel_count = 0;
    lds_barrier();
    for (int i = tid; i < len; i += TOPM_THREADS) {
      const uint32_t k = f32_key(src[i]);
      if (k > kstar) L.list[atomicAdd(&L.sel_count, 1)] = cand_pack(k, (uint32_t)(c0 + i));
    }
    int slot = Mc - need, left = need;  // Mc - need keys are above kstar
    for (int b0 = 0; b0 < len && left > 0; b0 += TOPM_THREADS) {
      const int i = b0 + tid;
      const bool f = i < len && f32_key(src[min(i, len - 1)]) == kstar;
      int tot;
      const int r = block_prefix_excl(f ? 1 : 0, L.wi, &tot);
      if (f && r < left) L.list[slot + r] = cand_pack(kstar, (uint32_t)(c0 + i));
      const int took = min(tot, left);
      slot += took;
      left -= took;
    }
    lds_barrier();
    if (wv == 0) {
      uint64_t v = lane < Mc ? L.list[lane] : 0ull;
      v = wave_sort_desc_u64(v);
      L.list[lane] = v;
    }
  }
  lds_barrier();
  // 5. the list, zero padded to M, and the statistics (m = max / T, the
  //    chunk's sum of exp(x/T - m), the same sum over its tokens left out of
  //    the list as the chunk sum minus the listed terms -- the listed values
  //    are the largest, so the difference keeps the tail to within rounding
  //    of the chunk sum -- and Mc)
  uint64_t* out_list = out_cand + (size_t)item * M;
  if (tid < M) out_list[tid] = tid < Mc ? L.list[tid] : 0ull;
  if (wv == 0) {
    const float e = (lane < Mc && vm > -INFINITY)
                        ? __builtin_amdgcn_exp2f(__builtin_fmaf(key_f32(cand_key(L.list[lane])), l2t, -mb)) : 0.f;
    const float s_sel = wave_sum_dpp(e);
    if (lane == 0) {
      const float tot = (L.ws[0] + L.ws[1]) + (L.ws[2] + L.ws[3]);
      out_stat[item] = make_float4(vm / T, tot, fmaxf(tot - s_sel, 0.f), __int_as_float(Mc));
    }
  }
}


__device__ __forceinline__ const float* chunk_src(const float* logits, int V, int S, int item, int* len) {
  const int row = item / S, c = item - row * S;
  *len = min(TOPM_CHUNK, V - c * TOPM_CHUNK);
  return logits + (size_t)row * (size_t)V + (size_t)c * TOPM_CHUNK;
}

// One block per item.
template <bool VEC4>
__global__ __launch_bounds__(TOPM_THREADS) void topm_chunk_kernel(
    const float* __restrict__ logits, int V, int S, int M, float T,
    uint64_t* __restrict__ out_cand, float4* __restrict__ out_stat) {
  __shared__ ChunkLds L;
  int len;
  const float* src = chunk_src(logits, V, S, blockIdx.x, &len);
  float x[PER_THREAD];
  chunk_load<VEC4>(src, len, x);
  chunk_select<VEC4>(L, logits, V, S, M, T, blockIdx.x, x, out_cand, out_stat);
}

// Number of entries of a descending list greater than `key`.
__device__ __forceinline__ int count_greater(const uint64_t* list, int n, uint64_t key) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (list[mid] > key) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(TOPM_THREADS) void topm_merge_kernel(
    const uint64_t* __restrict__ cand, const float4* __restrict__ stat, int S, int M, float T,
    int32_t* __restrict__ ids_out, float* __restrict__ vals_out, float* __restrict__ lse_out,
    float* __restrict__ tail_out, int32_t* __restrict__ tokrank_out, int32_t* __restrict__ user_ids,
    float* __restrict__ user_vals, float* __restrict__ user_lse, PArgs pa) {
  extern __shared__ uint64_t lists[];  // [S][M], then [MERGE_CAP] candidates (P tiles: [4][1024] floats)
  const int nrows = (int)gridDim.x - pa.blocks;  // the rows' blocks first, then P's
  if ((int)blockIdx.x >= nrows) {
    p_tile(pa, (int)blockIdx.x - nrows, reinterpret_cast<float*>(lists));
    return;
  }
  __shared__ int cnt[DT_TOPM_MAX_CHUNKS];
  __shared__ float mc[DT_TOPM_MAX_CHUNKS], sc[DT_TOPM_MAX_CHUNKS], tc[DT_TOPM_MAX_CHUNKS];
  __shared__ int out_ids[DT_TOPM_MAX];
  __shared__ float red[4];
  __shared__ uint64_t sub[MERGE_SUB];
  __shared__ int nsub, ncand;
  __shared__ uint64_t lbound, kth;

  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  uint64_t* cands = lists + (size_t)S * M;
  const uint64_t* src = cand + (size_t)row * S * M;
  for (int i = tid; i < S * M; i += TOPM_THREADS) lists[i] = src[i];
  for (int i = tid; i < S; i += TOPM_THREADS) {
    const float4 st = stat[(size_t)row * S + i];
    mc[i] = st.x;
    sc[i] = st.y;
    tc[i] = st.z;
    cnt[i] = __float_as_int(st.w);
  }
  if (tid == 0) {
    nsub = 0;
    ncand = 0;
    lbound = 0ull;
    kth = 0ull;
  }
  __syncthreads();
  float mloc = -INFINITY;
  for (int i = tid; i < S; i += TOPM_THREADS) mloc = fmaxf(mloc, mc[i]);
  const float mstar = block_max<TOPM_THREADS>(mloc, red);

  // 1. a lower bound for the row's M-th largest key: the M-th largest of the
  //    first tn entries of every (sorted) chunk list, a subset with at least M
  //    keys whenever the lists hold tn each (else the bound is 0: every key)
  const int tn = M / S + 2;
  for (int e = tid; e < S * tn; e += TOPM_THREADS) {
    const int c = e / tn, i = e - c * tn;
    if (i < cnt[c]) {
      const int slot = atomicAdd(&nsub, 1);
      if (slot < MERGE_SUB) sub[slot] = lists[c * M + i];
    }
  }
  __syncthreads();
  const int U = min(nsub, MERGE_SUB);
  for (int i = tid; i < U; i += TOPM_THREADS) {
    const uint64_t key = sub[i];
    int r = 0;
#pragma unroll 8
    for (int j = 0; j < U; ++j) r += sub[j] > key;
    if (r == M - 1) lbound = key;  // keys are unique: one thread at most
  }
  __syncthreads();
  // 2. the candidates: every key at or above the bound (a prefix of each list)
  const uint64_t lb = lbound;
  for (int e = tid; e < S * M; e += TOPM_THREADS) {
    const int c = e / M, i = e - c * M;
    const uint64_t key = lists[e];
    if (i < cnt[c] && key >= lb) {
      const int slot = atomicAdd(&ncand, 1);
      if (slot < MERGE_CAP) cands[slot] = key;
    }
  }
  __syncthreads();
  const int C = ncand;
  if (C <= MERGE_CAP) {
    // 3. exact ranks among the candidates; the M best are the row's list
    for (int i = tid; i < C; i += TOPM_THREADS) {
      const uint64_t key = cands[i];
      int rank = 0;
#pragma unroll 8
      for (int j = 0; j < C; ++j) rank += cands[j] > key;
      if (rank < M) {
        const int id = (int)cand_id(key);
        const float v = key_f32(cand_key(key));
        out_ids[rank] = id;
        ids_out[(size_t)row * M + rank] = id;
        vals_out[(size_t)row * M + rank] = v;
        if (user_ids) user_ids[(size_t)row * M + rank] = id;
        if (user_vals) user_vals[(size_t)row * M + rank] = v;
        if (rank == M - 1) kth = key;
      }
    }
  } else {
    // many keys at the bound: rank every list entry against the other lists
    for (int e = tid; e < S * M; e += TOPM_THREADS) {
      const int c = e / M, i = e - c * M;
      if (i >= cnt[c]) continue;
      const uint64_t key = lists[e];
      int rank = i;
      for (int c2 = 0; c2 < S; ++c2)
        if (c2 != c) rank += count_greater(lists + c2 * M, cnt[c2], key);
      if (rank < M) {
        const int id = (int)cand_id(key);
        const float v = key_f32(cand_key(key));
        out_ids[rank] = id;
        ids_out[(size_t)row * M + rank] = id;
        vals_out[(size_t)row * M + rank] = v;
        if (user_ids) user_ids[(size_t)row * M + rank] = id;
        if (user_vals) user_vals[(size_t)row * M + rank] = v;
        if (rank == M - 1) kth = key;
      }
    }
  }
  __syncthreads();
  // 4. the list entries left out of the row's M (keys below the M-th) join the tail
  const uint64_t km = kth;
  float extra = 0.f;
  if (mstar > -INFINITY) {
    for (int e = tid; e < S * M; e += TOPM_THREADS) {
      const int c = e / M, i = e - c * M;
      const uint64_t key = lists[e];
      if (i < cnt[c] && key < km) extra += __expf(key_f32(cand_key(key)) / T - mstar);
    }
  }
  float s_all = 0.f, s_tail = 0.f;
  if (mstar > -INFINITY) {
    for (int i = tid; i < S; i += TOPM_THREADS) {
      if (mc[i] > -INFINITY) {
        const float f = __expf(mc[i] - mstar);
        s_all += sc[i] * f;
        s_tail += tc[i] * f;
      }
    }
  }
  s_all = block_sum<TOPM_THREADS>(s_all, red);
  s_tail = block_sum<TOPM_THREADS>(s_tail + extra, red);
  if (tid == 0) {
    const float lse = (mstar > -INFINITY && s_all > 0.f) ? mstar + __logf(s_all) : -INFINITY;
    const float tail = (mstar > -INFINITY && s_tail > 0.f) ? mstar + __logf(s_tail) : -INFINITY;
    lse_out[row] = lse;
    tail_out[row] = tail;
    if (user_lse) user_lse[row] = lse;
  }
  __syncthreads();
  // rank of each candidate's token id among the row's candidates (heap tie order)
  for (int i = tid; i < M; i += TOPM_THREADS) {
    int r = 0;
    for (int j = 0; j < M; ++j) r += out_ids[j] < out_ids[i];
    tokrank_out[(size_t)row * M + i] = r;
  }
}

// NaN scan for DT_VALIDATE: sets *flag when any value is NaN.
__global__ void nan_scan_kernel(const float* __restrict__ x, size_t n, int* __restrict__ flag) {
  bool bad = false;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    bad |= x[i] != x[i];
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flag, 1);
}

hipError_t launch_topm(const float* logits, int rows, int V, int M, float T, uint64_t* chunk_cand,
                       float4* chunk_stat, int32_t* ids, float* vals, float* lse, float* tail,
                       int32_t* tokrank, int32_t* user_ids, float* user_vals, float* user_lse,
                       hipStream_t stream, const uint16_t* pA, const uint16_t* pBt, float* pC, int pN, int pK) {
  const int S = topm_chunks(V);
  const int items = rows * S;
  if (items == 0) return hipSuccess;
  PArgs pa{pA, pBt, pC, rows, pN, pK, 0};
  if (pA) {
    if (!pBt || !pC || pN < 1 || pK < 8 || pK % 8) return hipErrorInvalidValue;
    pa.blocks = ((rows + 31) / 32) * ((pN + 31) / 32) * P_KSPLIT;
  }
  const bool vec4 = (V % 4 == 0) && (reinterpret_cast<uintptr_t>(logits) % 16 == 0);
  if (vec4)
    hipLaunchKernelGGL(topm_chunk_kernel<true>, dim3(items), dim3(TOPM_THREADS), 0, stream, logits, V, S, M, T,
                       chunk_cand, chunk_stat);
  else
    hipLaunchKernelGGL(topm_chunk_kernel<false>, dim3(items), dim3(TOPM_THREADS), 0, stream, logits, V, S, M, T,
                       chunk_cand, chunk_stat);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = std::max(((size_t)S * M + MERGE_CAP) * sizeof(uint64_t), pa.blocks ? 4 * 1024 * sizeof(float) : 0);
  hipLaunchKernelGGL(topm_merge_kernel, dim3(pa.blocks + rows), dim3(TOPM_THREADS), lds, stream, chunk_cand,
                     chunk_stat, S, M, T, ids, vals, lse, tail, tokrank, user_ids, user_vals, user_lse, pa);
  return hipGetLastError();
}

hipError_t launch_topm_merge(const uint64_t* chunk_cand, const float4* chunk_stat, int rows, int S,
                             int M, float T, int32_t* ids, float* vals, float* lse, float* tail,
                             int32_t* tokrank, int32_t* user_ids, float* user_vals, float* user_lse,
                             hipStream_t stream) {
  const size_t lds = ((size_t)S * M + MERGE_CAP) * sizeof(uint64_t);
  hipLaunchKernelGGL(topm_merge_kernel, dim3(rows), dim3(TOPM_THREADS), lds, stream, chunk_cand,
                     chunk_stat, S, M, T, ids, vals, lse, tail, tokrank, user_ids, user_vals, user_lse, PArgs{});
  return hipGetLastError();
}

hipError_t launch_nan_scan(const float* x, size_t n, int* flag, hipStream_t stream) {
  hipLaunchKernelGGL(nan_scan_kernel, dim3(1024), dim3(256), 0, stream, x, n, flag);
  return hipGetLastError();
}

}  // namespace dt
