// The conditional best-first tree builder: one persistent cooperative kernel.
//
// Method (DominoTree technical summary, Componenti Core 1, 2 and 4; Domino
// summary, 核心方法): per request, pop the frontier node with the highest
// cumulative log-prob, advance the GRU causal state along that node's path,
// correct the next depth's M candidate logits with W2[:, cand] SiLU(W1 [H; S]),
// log-softmax them, push the k best children; stop after N pops.
//
// Roles (blocks of 256 threads, one per CU, launched cooperatively so that all
// are resident):
//   * worker blocks [0, n_workers): each keeps `tiles_per_worker` 16-row tiles
//     of the per-node product Wc = [W_hh ; W1_S^T] ((3 d_s + r) x d_s) in LDS
//     for the whole launch.  Each step it multiplies its rows by the GEMM
//     operand copy of the states of the nodes being expanded (one column per
//     request) with MFMA, and publishes gh = W_hh S~ + b_hh and u = W1_S^T S~.
//   * controller blocks [n_workers, n_workers + B): one per request.  It keeps
//     the request's candidates, node records and frontier in LDS; scores the
//     children of the node just expanded (a = SiLU(u + P_d), dL on the M
//     candidate columns of W2, log-softmax, top-k), pushes them, pops the next
//     node, and advances the GRU state for it elementwise from
//     G[token] = W_ih E[token] + b_ih (a table folded once per handle) and its
//     parent's gh.
// The GRU input product never runs per node, and the per-node weights never
// leave LDS; each step moves only states (d_s), gh (3 d_s) and u (r) per request.
//
// Exchange between blocks: every published value is written once per launch
// to its own 128-byte-aligned slot with device-scope (sc1) stores; after the
// stores complete the producer raises a flag word in each consumer's mailbox
// line (sc1 store); a consumer polls only its own mailbox line (sc1 loads)
// and then reads the published slots.  Slots are never read before they are
// published, so no cache holds a stale copy.  Every wait is bounded: when it
// runs out the block sets the error word and leaves its loop.
#include "common.h"
#include "kernels.h"

namespace dt {

constexpr uint32_t MBOX_DONE = 0xFFFFFFFFu;

// ---------------------------------------------------------------------------
// device-scope memory operations

__device__ __forceinline__ void st_dev_u32(void* p, uint32_t v) {
  asm volatile("global_store_dword %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void st_dev_u16(void* p, uint32_t v) {
  asm volatile("global_store_short %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void st_dev_f32x4(void* p, floatx4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ uint32_t ld_dev_u32(const void* p) {
  uint32_t v;
  asm volatile("global_load_dword %0, %1, off sc1\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
  return v;
}
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void st_dev_f32(float* p, float v) { st_dev_u32(p, __float_as_uint(v)); }

template <typename W>
__device__ __forceinline__ void st_dev_act(W* p, float v, int act_bf16);
template <>
__device__ __forceinline__ void st_dev_act<uint16_t>(uint16_t* p, float v, int) {
  st_dev_u16(p, f32_to_bf16(v));
}
template <>
__device__ __forceinline__ void st_dev_act<float>(float* p, float v, int act_bf16) {
  st_dev_f32(p, act_bf16 ? bf16_to_f32(f32_to_bf16(v)) : v);
}

template <typename W>
__device__ __forceinline__ float w_to_f32(W v);
template <>
__device__ __forceinline__ float w_to_f32<uint16_t>(uint16_t v) { return bf16_to_f32(v); }
template <>
__device__ __forceinline__ float w_to_f32<float>(float v) { return v; }

// ---------------------------------------------------------------------------
// layout helpers

__host__ __device__ inline int round_up(int x, int m) { return (x + m - 1) / m * m; }
__host__ __device__ inline int act_stride(int ds) { return round_up(ds, 64); }     // elements
__host__ __device__ inline int k_padded(int ds) { return round_up(ds, 32); }
__host__ __device__ inline int st_stride(int ds) { return round_up(ds, 32); }      // floats
__host__ __device__ inline int gh_stride(int ds) { return round_up(3 * ds, 32); }  // floats
__host__ __device__ inline int u_stride(int r) { return round_up(r, 32); }         // floats
constexpr int STAGE_PAD = 8;  // extra elements per staged column (LDS bank spread)

// frontier key: score | 31-depth | 63-tokrank | 1023-parent | slot
__device__ __forceinline__ uint64_t make_key(float score, int depth, int tokrank, int parent, int slot) {
  return ((uint64_t)f32_key(score) << 32) | ((uint64_t)(31 - depth) << 27) |
         ((uint64_t)(63 - tokrank) << 21) | ((uint64_t)(1023 - parent) << 11) | ((uint64_t)slot << 5);
}
__device__ __forceinline__ float key_score(uint64_t k) { return key_f32((uint32_t)(k >> 32)); }
__device__ __forceinline__ int key_depth(uint64_t k) { return 31 - (int)((k >> 27) & 31); }
__device__ __forceinline__ int key_parent(uint64_t k) { return 1023 - (int)((k >> 11) & 1023); }
__device__ __forceinline__ int key_slot(uint64_t k) { return (int)((k >> 5) & 63); }

// bounded wait on the words of one mailbox line; wave-uniform
__device__ bool wait_mbox(const uint32_t* box, int nwords, uint32_t epoch, const int* err,
                          unsigned limit) {
  const int lane = threadIdx.x & 63;
  unsigned it = 0;
  while (true) {
    bool ok = true;
    for (int i = lane; i < nwords; i += 64) ok &= ld_dev_u32(box + i) >= epoch;
    if (__all(ok)) return true;
    if ((++it & 255) == 0) {
      if (ld_dev_u32(err) != 0) return false;
      if (it > limit) {
        if (lane == 0) atomicOr((int*)err, 1);
        return false;
      }
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// ---------------------------------------------------------------------------
// worker: per-step product of its Wc tiles with the expanded nodes' states

template <typename W>
struct WorkerLds {
  // tiles [tpw][kp/32][4][16][8] elements, then the staged columns [32][kp + STAGE_PAD]
  static size_t bytes(int tpw, int kp) {
    return (size_t)tpw * 16 * kp * sizeof(W) + (size_t)32 * (kp + STAGE_PAD) * sizeof(W) + 1024;
  }
};

__device__ __forceinline__ void worker_store_out(const TreeArgs& a, int b, int node, int row, float v) {
  const int ds3 = 3 * a.ds;
  if (row < ds3) {
    st_dev_f32(a.gh + ((size_t)b * (a.N + 1) + node) * gh_stride(a.ds) + row, v + (a.b_hh ? a.b_hh[row] : 0.f));
  } else if (row < ds3 + a.r) {
    st_dev_f32(a.u + ((size_t)b * (a.N + 1) + node) * u_stride(a.r) + (row - ds3), v);
  }
}

template <typename W>
__device__ void worker_compute(const TreeArgs& a, const W* tiles_lds, const W* stage, int ncols,
                               const int* colb, const int* coln, int my_tile0, int my_ntiles, int kp);

// bf16: MFMA 16x16x32; wave w takes (tile, column block) pairs w, w+4, ...
template <>
__device__ void worker_compute<uint16_t>(const TreeArgs& a, const uint16_t* tiles_lds, const uint16_t* stage,
                                         int ncols, const int* colb, const int* coln, int my_tile0,
                                         int my_ntiles, int kp) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nkb = kp / 32;
  const int ncb = (ncols + 15) / 16;
  const int kps = kp + STAGE_PAD;
  for (int pair = wv; pair < my_ntiles * ncb; pair += 4) {
    const int tt = pair / ncb, cb = pair % ncb;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* wt = tiles_lds + (size_t)tt * 16 * kp;
    const int col = cb * 16 + (lane & 15);
    const uint16_t* sc = stage + (size_t)col * kps + 8 * (lane >> 4);
    for (int kb = 0; kb < nkb; ++kb) {
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(wt + ((size_t)kb * 64 + lane) * 8);
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(sc + kb * 32);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
    }
    // lane holds column (lane & 15), rows 4 (lane >> 4) + i of the tile
    if (col < ncols) {
      const int b = colb[col], node = coln[col];
      const int row0 = (my_tile0 + tt) * 16 + 4 * (lane >> 4);
      const int ds3 = 3 * a.ds;
      if (row0 + 3 < ds3 && (ds3 & 3) == 0) {
        const float* bh = a.b_hh;
        floatx4 v = acc;
        if (bh) {
          v[0] += bh[row0];
          v[1] += bh[row0 + 1];
          v[2] += bh[row0 + 2];
          v[3] += bh[row0 + 3];
        }
        st_dev_f32x4(a.gh + ((size_t)b * (a.N + 1) + node) * gh_stride(a.ds) + row0, v);
      } else {
        for (int i = 0; i < 4; ++i) worker_store_out(a, b, node, row0 + i, acc[i]);
      }
    }
  }
}

// fp32: one (row, column) dot product per thread over the padded k
template <>
__device__ void worker_compute<float>(const TreeArgs& a, const float* tiles_lds, const float* stage, int ncols,
                                      const int* colb, const int* coln, int my_tile0, int my_ntiles,
                                      int kp) {
  const int kps = kp + STAGE_PAD;
  const int total = my_ntiles * 16 * ncols;
  for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
    const int col = idx % ncols;
    const int rr = (idx / ncols) % 16;
    const int tt = idx / (ncols * 16);
    const float* wt = tiles_lds + (size_t)tt * 16 * kp;
    const float* sc = stage + (size_t)col * kps;
    float s = 0.f;
    for (int k = 0; k < kp; ++k) {
      const int kb = k >> 5, kg = (k >> 3) & 3, e = k & 7;
      s = fmaf(wt[(((size_t)kb * 4 + kg) * 16 + rr) * 8 + e], sc[k], s);
    }
    worker_store_out(a, colb[col], coln[col], (my_tile0 + tt) * 16 + rr, s);
  }
}

template <typename W>
__device__ void worker_main(const TreeArgs& a, unsigned char* lds) {
  const int w = blockIdx.x;
  const int tid = threadIdx.x;
  const int kp = k_padded(a.ds);
  const int tile0 = w * a.tiles_per_worker;
  const int ntiles = max(0, min(a.tiles_per_worker, a.n_tiles - tile0));
  W* tiles_lds = reinterpret_cast<W*>(lds);
  W* stage = tiles_lds + (size_t)a.tiles_per_worker * 16 * kp;
  int* colb = reinterpret_cast<int*>(stage + (size_t)32 * (kp + STAGE_PAD));
  int* coln = colb + 32;
  int* ncols_s = coln + 32;

  // the block's Wc tiles stay in LDS for the whole launch
  {
    const W* src = reinterpret_cast<const W*>(a.tiles) + (size_t)tile0 * 16 * kp;
    const size_t n16 = (size_t)ntiles * 16 * kp * sizeof(W) / 16;
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
    uint4* d4 = reinterpret_cast<uint4*>(tiles_lds);
    for (size_t i = tid; i < n16; i += blockDim.x) d4[i] = s4[i];
  }
  __syncthreads();

  const uint32_t* mybox = a.mbox_w + (size_t)w * 32;
  const int as = act_stride(a.ds);
  const int kps = kp + STAGE_PAD;
  for (int t = 0;; ++t) {
    const uint32_t epoch = (uint32_t)t + 1u;
    if (tid < 64) {
      bool ok = wait_mbox(mybox, a.B, epoch, a.err, a.spin_limit);
      if (tid == 0) *ncols_s = ok ? 0 : -1;
    }
    __syncthreads();
    if (*ncols_s < 0) return;
    // active columns: requests whose controller has not finished
    if (tid < 64) {
      const int b = tid;
      bool act = false;
      int node = -1;
      if (b < a.B && ld_dev_u32(mybox + b) != MBOX_DONE) {
        node = (int)ld_dev_u32(a.rec + (size_t)b * (a.N + 2) + t);
        act = node >= 0;
      }
      const unsigned long long m = __ballot(act);
      if (act) {
        const int slot = __popcll(m & ((1ull << tid) - 1ull));
        colb[slot] = b;
        coln[slot] = node;
      }
      if (tid == 0) *ncols_s = __popcll(m);
    }
    __syncthreads();
    const int ncols = *ncols_s;
    if (ncols == 0) return;  // every request is finished
    // stage the GEMM operand copies of the expanded states (published, read once)
    {
      const int per = kp * (int)sizeof(W) / 16;  // 16-byte pieces per column
      for (int i = tid; i < ncols * per; i += blockDim.x) {
        const int c = i / per, p = i % per;
        const W* src = reinterpret_cast<const W*>(a.act) + ((size_t)colb[c] * (a.N + 1) + coln[c]) * as;
        *reinterpret_cast<uint4*>(stage + (size_t)c * kps + p * (16 / sizeof(W))) =
            reinterpret_cast<const uint4*>(src)[p];
      }
    }
    __syncthreads();
    if (ntiles > 0) worker_compute<W>(a, tiles_lds, stage, ncols, colb, coln, tile0, ntiles, kp);
    stores_done();
    __syncthreads();
    // tell each active request's controller that this worker's rows are out
    if (tid < ncols) st_dev_u32(a.mbox_c + (size_t)colb[tid] * 256 + w, epoch);
    stores_done();
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// controller: one request's candidates, frontier, node records and GRU states

struct CtlLds {
  int* cid;        // [D*M]
  float* cval;     // [D*M]
  int* crank;      // [D*M]
  float* tailv;    // [D]
  uint64_t* front; // [fcap]
  int* ntok;       // [N+1]
  int* npar;
  int* ndep;
  float* nscore;
  float* av;       // [r]
  float* z;        // [64]
  float* logp;     // [64]
  int* okf;        // [64]
  int* misc;       // [16]
  uint64_t* red64; // [4]
  int* redpos;     // [4]
  float* redf;     // [4]
};

__host__ __device__ inline size_t ctl_lds_bytes(int D, int M, int N, int r, int fcap) {
  size_t s = 0;
  s += (size_t)fcap * 8;              // front (first: 8-byte aligned)
  s += (size_t)D * M * 4 * 3 + D * 4; // cid, cval, crank, tailv
  s += (size_t)(N + 1) * 4 * 4;       // node records
  s += (size_t)r * 4 + 64 * 4 * 3;    // av, z, logp, okf
  s += 16 * 4 + 4 * 8 + 4 * 4 + 4 * 4 + 64;
  return s;
}

__device__ CtlLds ctl_carve(unsigned char* lds, int D, int M, int N, int r, int fcap) {
  CtlLds c;
  unsigned char* p = lds;
  c.front = reinterpret_cast<uint64_t*>(p); p += (size_t)fcap * 8;
  c.red64 = reinterpret_cast<uint64_t*>(p); p += 4 * 8;
  c.cid = reinterpret_cast<int*>(p); p += (size_t)D * M * 4;
  c.cval = reinterpret_cast<float*>(p); p += (size_t)D * M * 4;
  c.crank = reinterpret_cast<int*>(p); p += (size_t)D * M * 4;
  c.tailv = reinterpret_cast<float*>(p); p += (size_t)D * 4;
  c.ntok = reinterpret_cast<int*>(p); p += (size_t)(N + 1) * 4;
  c.npar = reinterpret_cast<int*>(p); p += (size_t)(N + 1) * 4;
  c.ndep = reinterpret_cast<int*>(p); p += (size_t)(N + 1) * 4;
  c.nscore = reinterpret_cast<float*>(p); p += (size_t)(N + 1) * 4;
  c.av = reinterpret_cast<float*>(p); p += (size_t)r * 4;
  c.z = reinterpret_cast<float*>(p); p += 64 * 4;
  c.logp = reinterpret_cast<float*>(p); p += 64 * 4;
  c.okf = reinterpret_cast<int*>(p); p += 64 * 4;
  c.misc = reinterpret_cast<int*>(p); p += 16 * 4;
  c.redpos = reinterpret_cast<int*>(p); p += 4 * 4;
  c.redf = reinterpret_cast<float*>(p); p += 4 * 4;
  return c;
}

__device__ __forceinline__ float sigm(float x) { return 1.0f / (1.0f + expf(-x)); }

// score the children of node y (depth dy < D) and push the k best
template <typename W>
__device__ void ctl_expand(const TreeArgs& a, const CtlLds& c, int b, int y) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int M = a.M, r = a.r;
  const int dy = c.ndep[y];        // children are at depth dy + 1; row dy of the tables
  const float* urow = a.u + ((size_t)b * (a.N + 1) + y) * u_stride(r);
  const float* prow = a.P + ((size_t)b * a.D + dy) * r;
  for (int j = tid; j < r; j += blockDim.x) {
    const float x = urow[j] + prow[j];
    c.av[j] = x * sigm(x);  // SiLU
  }
  __syncthreads();
  // dL_m = W2[:, cand_m] . a  (thread group per candidate, fixed order)
  int tpc = 1;
  while (tpc * 2 * M <= (int)blockDim.x && tpc < 64) tpc *= 2;  // threads per candidate
  const int m = tid / tpc, part = tid % tpc;
  float dl = 0.f;
  if (m < M) {
    const int id = c.cid[dy * M + m];
    const W* wrow = reinterpret_cast<const W*>(a.w2t) + (size_t)id * r;
    for (int j = part; j < r; j += tpc) dl = fmaf(w_to_f32<W>(wrow[j]), c.av[j], dl);
  }
  for (int s = 1; s < tpc; s <<= 1) dl += __shfl_xor(dl, s);
  if (m < M && part == 0) c.z[m] = (c.cval[dy * M + m] + dl) / a.T + 0.0f;
  __syncthreads();
  // log-softmax over the candidates (plus the base tail under fullv), wave 0
  if (tid < 64) {
    const float zv = lane < M ? c.z[lane] : -INFINITY;
    float mx = wave_max(zv);
    if (a.fullv) mx = fmaxf(mx, c.tailv[dy]);
    float se = 0.f;
    if (mx > -INFINITY) {
      se = wave_sum(lane < M ? expf(zv - mx) : 0.f);
      if (a.fullv && c.tailv[dy] > -INFINITY) se += expf(c.tailv[dy] - mx);
    }
    const float lz = mx > -INFINITY ? mx + logf(se) : -INFINITY;
    if (lane < M) c.logp[lane] = zv - lz;
  }
  __syncthreads();
  // rank by (z desc, token asc); the k best with a finite log-prob are pushed.
  // -inf log-probs rank after every finite one, so the children take ranks 0..n-1.
  if (tid < M) {
    const float zm = c.z[tid];
    const int idm = c.cid[dy * M + tid];
    int rank = 0;
    for (int q = 0; q < M; ++q) {
      const float zq = c.z[q];
      rank += (zq > zm) || (zq == zm && c.cid[dy * M + q] < idm);
    }
    const float lp = c.logp[tid];
    const bool ok = rank < a.k && isfinite(lp);
    c.okf[tid] = ok;
    if (ok) c.front[c.misc[0] + rank] = make_key(c.nscore[y] + lp, dy + 1, c.crank[dy * M + tid], y, tid);
  }
  __syncthreads();
  if (tid == 0) {
    int nch = 0;
    for (int q = 0; q < M; ++q) nch += c.okf[q];
    c.misc[0] += nch;
  }
  __syncthreads();
}

// pop the best frontier entry; returns false when the frontier is empty
__device__ bool ctl_pop(const CtlLds& c, uint64_t* key_out) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = c.misc[0];
  if (n == 0) return false;
  uint64_t best = 0;
  int pos = -1;
  for (int i = tid; i < n; i += blockDim.x) {
    const uint64_t k = c.front[i];
    if (pos < 0 || k > best) {
      best = k;
      pos = i;
    }
  }
  const uint64_t wbest = wave_max_u64(pos < 0 ? 0ull : best);
  if (lane == 0) c.red64[wv] = wbest;
  __syncthreads();
  uint64_t gbest = c.red64[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) gbest = c.red64[i] > gbest ? c.red64[i] : gbest;
  if (pos >= 0 && best == gbest) c.misc[1] = pos;  // keys are unique
  __syncthreads();
  if (tid == 0) {
    const int p = c.misc[1];
    c.front[p] = c.front[n - 1];
    c.misc[0] = n - 1;
  }
  __syncthreads();
  *key_out = gbest;
  return true;
}

template <typename W>
__device__ void ctl_advance_state(const TreeArgs& a, int b, int y, int x, int tok) {
  // S_y = GRU(S_x, E[tok]) with W_ih E[tok] + b_ih = G[tok] and gh_x = W_hh S~_x + b_hh
  const int ds = a.ds;
  const float* gi = a.G + (size_t)tok * 3 * ds;
  const float* gh = a.gh + ((size_t)b * (a.N + 1) + x) * gh_stride(ds);
  const float* sx = a.state + ((size_t)b * (a.N + 1) + x) * st_stride(ds);
  float* sy = a.state + ((size_t)b * (a.N + 1) + y) * st_stride(ds);
  W* ay = reinterpret_cast<W*>(a.act) + ((size_t)b * (a.N + 1) + y) * act_stride(ds);
  for (int j = threadIdx.x; j < ds; j += blockDim.x) {
    const float rg = sigm(gi[j] + gh[j]);
    const float zg = sigm(gi[ds + j] + gh[ds + j]);
    const float ng = tanhf(gi[2 * ds + j] + rg * gh[2 * ds + j]);
    const float s = (1.0f - zg) * ng + zg * sx[j];
    st_dev_f32(sy + j, s);
    st_dev_act<W>(ay + j, s, a.act_bf16);
  }
  for (int j = ds + threadIdx.x; j < k_padded(ds); j += blockDim.x) st_dev_act<W>(ay + j, 0.f, 0);
}

template <typename W>
__device__ void controller_main(const TreeArgs& a, unsigned char* lds) {
  const int b = blockIdx.x - a.n_workers;
  const int tid = threadIdx.x;
  const int D = a.D, M = a.M, N = a.N;
  const int fcap = a.N * (a.k - 1) + 1;
  CtlLds c = ctl_carve(lds, D, M, N, a.r, fcap);

  for (int i = tid; i < D * M; i += blockDim.x) {
    c.cid[i] = a.cand_ids[(size_t)b * D * M + i];
    c.cval[i] = a.cand_vals[(size_t)b * D * M + i];
    c.crank[i] = a.tokrank[(size_t)b * D * M + i];
  }
  for (int i = tid; i < D; i += blockDim.x) c.tailv[i] = a.tail[(size_t)b * D + i];
  if (tid == 0) {
    c.misc[0] = 0;  // frontier size
    c.ntok[0] = -1;
    c.npar[0] = -1;
    c.ndep[0] = 0;
    c.nscore[0] = 0.f;
  }
  // root state and its GEMM operand copy
  {
    const int ds = a.ds;
    float* s0 = a.state + (size_t)b * (N + 1) * st_stride(ds);
    W* a0 = reinterpret_cast<W*>(a.act) + (size_t)b * (N + 1) * act_stride(ds);
    for (int j = tid; j < ds; j += blockDim.x) {
      const float v = a.root ? a.root[(size_t)b * ds + j] : 0.f;
      st_dev_f32(s0 + j, v);
      st_dev_act<W>(a0 + j, v, a.act_bf16);
    }
    for (int j = ds + tid; j < k_padded(ds); j += blockDim.x) st_dev_act<W>(a0 + j, 0.f, 0);
  }
  if (tid == 0) st_dev_u32(a.rec + (size_t)b * (N + 2), 0u);
  stores_done();
  __syncthreads();
  if (tid < a.n_workers) st_dev_u32(a.mbox_w + (size_t)tid * 32 + b, 1u);  // step 0 posted
  for (int w = tid + 256; w < a.n_workers; w += 256) st_dev_u32(a.mbox_w + (size_t)w * 32 + b, 1u);
  stores_done();
  __syncthreads();

  int y = 0;  // node expanded at this step
  int n = 0;  // non-root nodes popped (same value in every thread)
  bool failed = false;
  for (int t = 0;; ++t) {
    const uint32_t epoch = (uint32_t)t + 1u;
    if (tid < 64) {
      const bool ok = wait_mbox(a.mbox_c + (size_t)b * 256, a.n_workers, epoch, a.err, a.spin_limit);
      if (tid == 0) c.misc[3] = ok;
    }
    __syncthreads();
    if (!c.misc[3]) {
      failed = true;
      break;
    }
    ctl_expand<W>(a, c, b, y);
    // pop until a node to expand is found, the budget is met or the frontier is empty
    int next = -1;
    while (n < N) {
      uint64_t key;
      if (!ctl_pop(c, &key)) break;
      const int i = n + 1;
      const int d = key_depth(key), slot = key_slot(key);
      if (tid == 0) {
        c.ntok[i] = c.cid[(d - 1) * M + slot];
        c.npar[i] = key_parent(key);
        c.ndep[i] = d;
        c.nscore[i] = key_score(key);
      }
      n = i;
      if (d < D && i < N) {
        next = i;
        break;
      }
    }
    __syncthreads();
    if (next < 0) break;
    ctl_advance_state<W>(a, b, next, c.npar[next], c.ntok[next]);
    if (tid == 0) st_dev_u32(a.rec + (size_t)b * (N + 2) + t + 1, (uint32_t)next);
    stores_done();
    __syncthreads();
    for (int w = tid; w < a.n_workers; w += blockDim.x)
      st_dev_u32(a.mbox_w + (size_t)w * 32 + b, epoch + 1u);
    stores_done();
    __syncthreads();
    y = next;
  }
  // release the workers from this request
  for (int w = tid; w < a.n_workers; w += blockDim.x) st_dev_u32(a.mbox_w + (size_t)w * 32 + b, MBOX_DONE);
  stores_done();
  // outputs, padded past n
  for (int i = tid; i <= N; i += blockDim.x) {
    const bool in = i <= n;
    a.tokens[(size_t)b * (N + 1) + i] = in ? c.ntok[i] : -1;
    a.parents[(size_t)b * (N + 1) + i] = in ? c.npar[i] : -1;
    a.depths[(size_t)b * (N + 1) + i] = in ? c.ndep[i] : -1;
    a.scores[(size_t)b * (N + 1) + i] = in ? c.nscore[i] : -INFINITY;
  }
  if (tid == 0) a.n_nodes[b] = failed ? -1 : n;
}

template <typename W>
__global__ __launch_bounds__(256) void tree_kernel(TreeArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  // no cache line of an exchange slot may survive from an earlier launch
  __threadfence();
  if ((int)blockIdx.x < a.n_workers) worker_main<W>(a, lds);
  else controller_main<W>(a, lds);
}

size_t tree_lds_bytes(const TreeArgs& a, int wdtype_bf16) {
  const int kp = k_padded(a.ds);
  const size_t w = wdtype_bf16 ? WorkerLds<uint16_t>::bytes(a.tiles_per_worker, kp)
                               : WorkerLds<float>::bytes(a.tiles_per_worker, kp);
  const size_t c = ctl_lds_bytes(a.D, a.M, a.N, a.r, a.N * (a.k - 1) + 1);
  return w > c ? w : c;
}

hipError_t launch_tree(const TreeArgs& a, int wdtype_bf16, size_t lds_bytes, hipStream_t stream) {
  void* args[] = {const_cast<TreeArgs*>(&a)};
  const dim3 grid(a.n_workers + a.B), block(256);
  const void* fn = wdtype_bf16 ? (const void*)tree_kernel<uint16_t> : (const void*)tree_kernel<float>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
  if (e != hipSuccess) return e;
  return hipLaunchCooperativeKernel(fn, grid, block, args, (unsigned)lds_bytes, stream);
}

}  // namespace dt
