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
// reads its chunk once from HBM into registers (32 values per thread).  Each
// wave sorts its 64 per-thread maxima and takes the ceil(M/4)-th largest; the
// smallest of the four wave values bounds the chunk's M-th largest value from
// below (at least M threads reach it), so the keys at or above it -- typically
// a few more than M -- hold the chunk's top-M; they are ranked exactly as
// (value desc, id asc) composites.  The chunk's LSE statistics come from the
// same registers.  topm_fallback: when more than 512 keys reach that bound
// (many equal values), an exact 3-pass radix select over the chunk in LDS
// redoes that chunk.  topm_merge: one block per row bounds the row's M-th key
// from below by the M-th largest of the first few entries of every chunk list,
// ranks the keys at or above the bound against each other and keeps the M
// best; the LSE statistics combine exactly (a token left out of its chunk's
// list is left out of the row's).
#include "common.h"
#include "kernels.h"

namespace dt {

constexpr int TOPM_THREADS = 256;
constexpr int HBINS = 4096;

constexpr int PER_THREAD = TOPM_CHUNK / TOPM_THREADS;  // 32 values per thread
constexpr int FAST_CAP = 512;                          // candidates the fast path ranks
constexpr int MERGE_SUB = 320;   // merge: subset keys for the bound (S (M / S + 2) <= M + 2 S)
constexpr int MERGE_CAP = 1024;  // merge: candidates ranked pairwise

// Bitonic sort of one 32-bit value per lane of a wave, descending.
__device__ __forceinline__ uint32_t wave_sort_desc_u32(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j >= 1; j >>= 1) {
      const uint32_t o = (uint32_t)__shfl_xor((int)v, j);
      const bool lower = (lane & j) == 0;
      const bool desc_block = (lane & k) == 0;  // the last (k = 64) block is descending
      v = (lower == desc_block) ? max(v, o) : min(v, o);
    }
  }
  return v;
}

template <bool FULL>
__device__ __forceinline__ void topm_chunk_body(const float* __restrict__ src, int len, int c0, int Mc, int M,
                                                float T, uint64_t* __restrict__ out_list,
                                                float4* __restrict__ out_stat_p, uint64_t* sel, uint32_t* wb,
                                                float* red, int* sel_count) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // 1. read the chunk once into registers: element tid*4 + 1024 j + e holds
  //    float4 piece j of thread tid (coalesced); missing elements are -inf.
  float x[PER_THREAD];
  if (FULL) {
    const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll
    for (int j = 0; j < PER_THREAD / 4; ++j) {
      const float4 v = s4[j * TOPM_THREADS + tid];
      x[4 * j] = v.x;
      x[4 * j + 1] = v.y;
      x[4 * j + 2] = v.z;
      x[4 * j + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < PER_THREAD / 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = (j * TOPM_THREADS + tid) * 4 + e;
        x[4 * j + e] = i < len ? src[i] : -INFINITY;
      }
  }
  auto idx_of = [&](int q) { return ((q >> 2) * TOPM_THREADS + tid) * 4 + (q & 3); };
  float vmax = -INFINITY;
  uint32_t kmax = 0;
#pragma unroll
  for (int q = 0; q < PER_THREAD; ++q) {
    vmax = fmaxf(vmax, x[q]);
    if (FULL || idx_of(q) < len) kmax = max(kmax, f32_key(x[q]));
  }
  // 2. threshold: in each wave the ceil(Mc/4)-th largest lane maximum; the
  //    smallest of the four bounds the chunk's Mc-th largest key from below
  //    (at least 4 ceil(Mc/4) >= Mc threads have a maximum at or above it)
  const int m4 = (Mc + 3) >> 2;
  const uint32_t sorted = wave_sort_desc_u32(kmax);
  const uint32_t wbound = (uint32_t)__builtin_amdgcn_readlane((int)sorted, m4 - 1);
  const float wmax = wave_max_dpp(vmax);
  if (lane == 0) {
    wb[wv] = wbound;
    red[wv] = wmax;
  }
  if (tid == 0) *sel_count = 0;
  __syncthreads();
  const uint32_t tau = min(min(wb[0], wb[1]), min(wb[2], wb[3]));
  const float vm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));  // the chunk's max value
#pragma unroll
  for (int q = 0; q < PER_THREAD; ++q) {
    const uint32_t k = f32_key(x[q]);
    if ((FULL || idx_of(q) < len) && k >= tau) {
      const int slot = atomicAdd(sel_count, 1);
      if (slot < FAST_CAP) sel[slot] = cand_pack(k, (uint32_t)(c0 + idx_of(q)));
    }
  }
  __syncthreads();
  const int cnt = *sel_count;
  if (cnt > FAST_CAP) {
    // too many keys at the threshold (equal values): topm_fallback_kernel
    // redoes this chunk exactly
    if (tid == 0) *out_stat_p = make_float4(0.f, 0.f, 0.f, __int_as_float(-1));
    return;
  }
  // 3. rank the candidates exactly (composite keys are unique)
  uint64_t mine[FAST_CAP / TOPM_THREADS];
  int rk[FAST_CAP / TOPM_THREADS];
#pragma unroll
  for (int u = 0; u < FAST_CAP / TOPM_THREADS; ++u) {
    const int e = tid + u * TOPM_THREADS;
    mine[u] = e < cnt ? sel[e] : 0ull;
    rk[u] = 0;
  }
  if (tid == 0 && (cnt & 1)) sel[cnt] = 0ull;  // pad to pairs (0 ranks below every key)
  __syncthreads();
  const ulonglong2* s2 = reinterpret_cast<const ulonglong2*>(sel);
  if (cnt <= TOPM_THREADS) {
    for (int i = 0; i < (cnt + 1) / 2; ++i) {
      const ulonglong2 o = s2[i];
      rk[0] += (o.x > mine[0]) + (o.y > mine[0]);
    }
  } else {
    for (int i = 0; i < (cnt + 1) / 2; ++i) {
      const ulonglong2 o = s2[i];
#pragma unroll
      for (int u = 0; u < FAST_CAP / TOPM_THREADS; ++u) rk[u] += (o.x > mine[u]) + (o.y > mine[u]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < FAST_CAP / TOPM_THREADS; ++u) {
    const int e = tid + u * TOPM_THREADS;
    if (e < cnt && rk[u] < Mc) sel[rk[u]] = mine[u];  // ranks < Mc are distinct
  }
  __syncthreads();
  // 4. the chunk's list, sorted (value desc, id asc), zero padded to M
  if (tid < M) out_list[tid] = tid < Mc ? sel[tid] : 0ull;

  // 5. LSE statistics: the chunk's sum of exp(x/T - m), and the same sum over
  //    its left-out tokens as the chunk sum minus the selected terms (the
  //    selected values are the largest, so the difference keeps the tail to
  //    within rounding of the chunk sum)
  const float m = vm / T;
  const float l2t = 1.4426950408889634f / T;  // exp(y / T) = exp2(y * log2(e) / T)
  float s_all = 0.f;
  if (vm > -INFINITY) {
#pragma unroll
    for (int q = 0; q < PER_THREAD; ++q) s_all += __builtin_amdgcn_exp2f((x[q] - vm) * l2t);  // -inf adds 0
  }
  s_all = wave_sum_dpp(s_all);
  float s_sel = 0.f;
  if (wv == 0) {
    const float e = (lane < Mc && vm > -INFINITY) ? __builtin_amdgcn_exp2f((key_f32(cand_key(sel[lane])) - vm) * l2t)
                                                  : 0.f;
    s_sel = wave_sum_dpp(e);
  }
  __syncthreads();
  if (lane == 0) red[wv] = s_all;
  __syncthreads();
  if (tid == 0) {
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    *out_stat_p = make_float4(m, tot, fmaxf(tot - s_sel, 0.f), __int_as_float(Mc));
  }
}

__global__ __launch_bounds__(TOPM_THREADS) void topm_chunk_kernel(
    const float* __restrict__ logits, int V, int S, int M, float T,
    uint64_t* __restrict__ out_cand, float4* __restrict__ out_stat) {
  __shared__ __attribute__((aligned(16))) uint64_t sel[FAST_CAP + 2];
  __shared__ uint32_t wb[4];
  __shared__ float red[4];
  __shared__ int sel_count;
  const int c = blockIdx.x;
  const int row = blockIdx.y;
  const int c0 = c * TOPM_CHUNK;
  const int len = min(TOPM_CHUNK, V - c0);
  const int Mc = min(M, len);
  const float* src = logits + (size_t)row * (size_t)V + c0;
  uint64_t* list = out_cand + ((size_t)row * S + c) * M;
  float4* stat = out_stat + (size_t)row * S + c;
  if ((V & 3) == 0 && len == TOPM_CHUNK)
    topm_chunk_body<true>(src, len, c0, Mc, M, T, list, stat, sel, wb, red, &sel_count);
  else
    topm_chunk_body<false>(src, len, c0, Mc, M, T, list, stat, sel, wb, red, &sel_count);
}

// Exact per-chunk selection for the chunks the fast path could not rank
// (more than FAST_CAP keys at or above its threshold: many equal values).
// Every other block returns at once.  3-pass radix select (12, 12, 8 bits) of
// the Mc-th largest key over the chunk in LDS, ties at the threshold taken in
// id order.
__global__ __launch_bounds__(TOPM_THREADS) void topm_fallback_kernel(
    const float* __restrict__ logits, int V, int S, int M, float T,
    uint64_t* __restrict__ out_cand, float4* __restrict__ out_stat) {
  const int c = blockIdx.x, row = blockIdx.y;
  if (__float_as_int(out_stat[(size_t)row * S + c].w) != -1) return;
  __shared__ uint32_t keys[TOPM_CHUNK];
  __shared__ uint32_t hist[HBINS];
  __shared__ uint64_t sel[DT_TOPM_MAX];
  __shared__ float red[4];
  __shared__ int ired[4];
  __shared__ int found_digit, found_above, sel_count, tie_last_s;
  const int tid = threadIdx.x;
  const int c0 = c * TOPM_CHUNK;
  const int len = min(TOPM_CHUNK, V - c0);
  const int Mc = min(M, len);
  const float* src = logits + (size_t)row * (size_t)V + c0;
  float vmax = -INFINITY;
  for (int i = tid; i < len; i += TOPM_THREADS) {
    const float x = src[i];
    keys[i] = f32_key(x);
    vmax = fmaxf(vmax, x);
  }
  const float m = block_max<TOPM_THREADS>(vmax, red) / T;
  uint32_t prefix = 0, pmask = 0;
  int need = Mc;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
    const int width = pass == 2 ? 8 : 12;
    const uint32_t dmask = (1u << width) - 1u;
    const int nb = 1 << width;
    for (int i = tid; i < nb; i += TOPM_THREADS) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < len; i += TOPM_THREADS) {
      const uint32_t k = keys[i];
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> sh) & dmask], 1u);
    }
    __syncthreads();
    const int per = nb / TOPM_THREADS;
    int mine = 0;
    for (int b = 0; b < per; ++b) mine += (int)hist[tid * per + b];
    int above = block_suffix_excl<TOPM_THREADS>(mine, ired);
    for (int b = per - 1; b >= 0; --b) {
      const int h = (int)hist[tid * per + b];
      if (above < need && above + h >= need) {
        found_digit = tid * per + b;
        found_above = above;
      }
      above += h;
    }
    __syncthreads();
    need -= found_above;
    prefix |= (uint32_t)found_digit << sh;
    pmask |= dmask << sh;
    __syncthreads();
  }
  const uint32_t kstar = prefix;
  if (tid == 0) {
    sel_count = 0;
    tie_last_s = -1;
  }
  __syncthreads();
  for (int i = tid; i < len; i += TOPM_THREADS) {
    const uint32_t k = keys[i];
    if (k > kstar) sel[atomicAdd(&sel_count, 1)] = cand_pack(k, (uint32_t)(c0 + i));
  }
  __syncthreads();
  int slot = Mc - need;
  for (int b0 = 0; b0 < len && need > 0; b0 += TOPM_THREADS) {
    const int i = b0 + tid;
    const bool f = i < len && keys[i] == kstar;
    int total;
    const int r = block_rank_flag<TOPM_THREADS>(f, ired, &total);
    if (f && r < need) {
      sel[slot + r] = cand_pack(kstar, (uint32_t)(c0 + i));
      if (r == need - 1) tie_last_s = i;
    }
    const int took = min(total, need);
    slot += took;
    need -= took;
    __syncthreads();
  }
  const int tie_last = tie_last_s;
  if (tid < 64) {
    uint64_t v = tid < Mc ? sel[tid] : 0ull;
    v = wave_sort_desc_u64(v);
    if (tid < M) out_cand[((size_t)row * S + c) * M + tid] = v;
  }
  float s_all = 0.f, s_tail = 0.f;
  if (m > -INFINITY) {
    for (int i = tid; i < len; i += TOPM_THREADS) {
      const uint32_t k = keys[i];
      const float e = __expf(key_f32(k) / T - m);
      s_all += e;
      if (!(k > kstar || (k == kstar && i <= tie_last))) s_tail += e;
    }
  }
  s_all = block_sum<TOPM_THREADS>(s_all, red);
  s_tail = block_sum<TOPM_THREADS>(s_tail, red);
  if (tid == 0) out_stat[(size_t)row * S + c] = make_float4(m, s_all, s_tail, __int_as_float(Mc));
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
    float* __restrict__ user_vals, float* __restrict__ user_lse) {
  extern __shared__ uint64_t lists[];  // [S][M], then [MERGE_CAP] candidates
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
                       hipStream_t stream) {
  const int S = topm_chunks(V);
  hipLaunchKernelGGL(topm_chunk_kernel, dim3(S, rows), dim3(TOPM_THREADS), 0, stream, logits, V, S, M,
                     T, chunk_cand, chunk_stat);
  hipLaunchKernelGGL(topm_fallback_kernel, dim3(S, rows), dim3(TOPM_THREADS), 0, stream, logits, V, S, M,
                     T, chunk_cand, chunk_stat);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topm_merge(chunk_cand, chunk_stat, rows, S, M, T, ids, vals, lse, tail, tokrank,
                           user_ids, user_vals, user_lse, stream);
}

hipError_t launch_topm_merge(const uint64_t* chunk_cand, const float4* chunk_stat, int rows, int S,
                             int M, float T, int32_t* ids, float* vals, float* lse, float* tail,
                             int32_t* tokrank, int32_t* user_ids, float* user_vals, float* user_lse,
                             hipStream_t stream) {
  const size_t lds = ((size_t)S * M + MERGE_CAP) * sizeof(uint64_t);
  hipLaunchKernelGGL(topm_merge_kernel, dim3(rows), dim3(TOPM_THREADS), lds, stream, chunk_cand,
                     chunk_stat, S, M, T, ids, vals, lse, tail, tokrank, user_ids, user_vals, user_lse);
  return hipGetLastError();
}

hipError_t launch_nan_scan(const float* x, size_t n, int* flag, hipStream_t stream) {
  hipLaunchKernelGGL(nan_scan_kernel, dim3(1024), dim3(256), 0, stream, x, n, flag);
  return hipGetLastError();
}

}  // namespace dt
