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

__device__ __forceinline__ void st_dev_u32x2(void* p, uint32_t lo, uint32_t hi) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  u32x2 v = {lo, hi};
  asm volatile("global_store_dwordx2 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}

// four consecutive operand values (the address is 8- or 16-byte aligned)
template <typename W>
__device__ __forceinline__ void st_dev_act4(W* p, floatx4 v, int act_bf16);
template <>
__device__ __forceinline__ void st_dev_act4<uint16_t>(uint16_t* p, floatx4 v, int) {
  const uint32_t lo = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
  st_dev_u32x2(p, lo, hi);
}
template <>
__device__ __forceinline__ void st_dev_act4<float>(float* p, floatx4 v, int act_bf16) {
  if (act_bf16)
    for (int q = 0; q < 4; ++q) v[q] = bf16_to_f32(f32_to_bf16(v[q]));
  st_dev_f32x4(p, v);
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
__device__ __forceinline__ bool wait_mbox(const uint32_t* box, int nwords, uint32_t epoch, const int* err,
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

// Exchange slots are step-major: the column request b publishes at step t
// lives in slot t * B + b of act, gh and u.
__device__ __forceinline__ size_t slot_of(const TreeArgs& a, int t, int b) { return (size_t)t * a.B + b; }

__device__ __forceinline__ void worker_store_out(const TreeArgs& a, size_t slot, int row, float v) {
  const int ds3 = 3 * a.ds;
  if (row < ds3) {
    st_dev_f32(a.gh + slot * gh_stride(a.ds) + row, v + (a.b_hh ? a.b_hh[row] : 0.f));
  } else if (row < ds3 + a.r) {
    st_dev_f32(a.u + slot * u_stride(a.r) + (row - ds3), v);
  }
}

template <typename W>
__device__ __forceinline__ void worker_compute(const TreeArgs& a, const W* tiles_lds, const W* stage, int ncols,
                               const int* colb, const int* coln, int my_tile0, int my_ntiles, int kp);

// bf16: MFMA 16x16x32; wave w takes (tile, column block) pairs w, w+4, ...
template <>
__device__ __forceinline__ void worker_compute<uint16_t>(const TreeArgs& a, const uint16_t* tiles_lds, const uint16_t* stage,
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
    // two independent accumulation chains, 4 k blocks in flight
    floatx4 acc2 = {0.f, 0.f, 0.f, 0.f};
    int kb = 0;
    for (; kb + 4 <= nkb; kb += 4) {
      bf16x8 av[4], bv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        av[q] = *reinterpret_cast<const bf16x8*>(wt + ((size_t)(kb + q) * 64 + lane) * 8);
        bv[q] = *reinterpret_cast<const bf16x8*>(sc + (kb + q) * 32);
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[0], bv[0], acc, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[1], bv[1], acc2, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[2], bv[2], acc, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[3], bv[3], acc2, 0, 0, 0);
    }
    for (; kb < nkb; ++kb) {
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(wt + ((size_t)kb * 64 + lane) * 8);
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(sc + kb * 32);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
    }
    acc += acc2;
    // lane holds column (lane & 15), rows 4 (lane >> 4) + i of the tile
    if (col < ncols) {
      const size_t slot = (size_t)coln[col];
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
        st_dev_f32x4(a.gh + slot * gh_stride(a.ds) + row0, v);
      } else {
        for (int i = 0; i < 4; ++i) worker_store_out(a, slot, row0 + i, acc[i]);
      }
    }
  }
}

// fp32: one (row, column) dot product per thread over the padded k
template <>
__device__ __forceinline__ void worker_compute<float>(const TreeArgs& a, const float* tiles_lds, const float* stage, int ncols,
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
    worker_store_out(a, (size_t)coln[col], (my_tile0 + tt) * 16 + rr, s);
  }
}

template <typename W>
__device__ __forceinline__ void worker_main(const TreeArgs& a, unsigned char* lds) {
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
      const bool act = b < a.B && ld_dev_u32(mybox + b) != MBOX_DONE;
      const unsigned long long m = __ballot(act);
      if (act) {
        const int c = __popcll(m & ((1ull << tid) - 1ull));
        colb[c] = b;
        coln[c] = (int)slot_of(a, t, b);  // exchange slot of this column
      }
      if (tid == 0) *ncols_s = __popcll(m);
    }
    __syncthreads();
    const int ncols = *ncols_s;
    if (ncols == 0) return;  // every request is finished
    // stage the GEMM operand copies of the expanded states (published, read
    // once).  Thread tid owns piece tid % per of columns tid / per + j * cpt;
    // every load of a round is issued before any LDS store.
    {
      const int per = kp * (int)sizeof(W) / 16;  // 16-byte pieces per column
      if (per <= 256 && 256 % per == 0) {
        const int cpt = 256 / per;                 // columns per pass
        const int pc = tid % per, c0 = tid / per;
        constexpr int U = 16;
        for (int cb = 0; cb < ncols; cb += U * cpt) {
          uint4 v[U];
#pragma unroll
          for (int q = 0; q < U; ++q) {  // clamped: every lane loads a valid piece
            const int c = min(cb + c0 + q * cpt, ncols - 1);
            v[q] = reinterpret_cast<const uint4*>(reinterpret_cast<const W*>(a.act) + (size_t)coln[c] * as)[pc];
          }
          // unconditional stores (a clamped duplicate rewrites identical data),
          // so that no load is sunk into a guarded block and serialised
#pragma unroll
          for (int q = 0; q < U; ++q) {
            const int c = min(cb + c0 + q * cpt, ncols - 1);
            *reinterpret_cast<uint4*>(stage + (size_t)c * kps + pc * (16 / sizeof(W))) = v[q];
          }
        }
      } else {
        for (int i = tid; i < ncols * per; i += blockDim.x) {
          const int c = i / per, pc = i % per;
          *reinterpret_cast<uint4*>(stage + (size_t)c * kps + pc * (16 / sizeof(W))) =
              reinterpret_cast<const uint4*>(reinterpret_cast<const W*>(a.act) + (size_t)coln[c] * as)[pc];
        }
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
  int* nstep;      // [N+1] step at which a node was expanded
  float* nscore;
  float* av;       // [r]
  void* w2s;       // [M][r] candidate rows of W2 for the next expansion (wdtype)
  float* ps;       // [r] P row of the next expansion
  float* z;        // [64]
  float* logp;     // [64]
  int* okf;        // [64]
  int* misc;       // [16]
  uint64_t* red64; // [4]
  int* redpos;     // [4]
  float* redf;     // [4]
};

__host__ __device__ inline size_t ctl_lds_bytes(int D, int M, int N, int r, int fcap, int esz) {
  size_t s = (size_t)M * r * esz + (size_t)r * 4 + 32;  // w2s, ps
  s += (size_t)fcap * 8;              // front (first: 8-byte aligned)
  s += (size_t)D * M * 4 * 3 + D * 4; // cid, cval, crank, tailv
  s += (size_t)(N + 1) * 4 * 5;       // node records
  s += (size_t)r * 4 + 64 * 4 * 3;    // av, z, logp, okf
  s += 16 * 4 + 4 * 8 + 4 * 4 + 4 * 4 + 64;
  return s;
}

__device__ __forceinline__ CtlLds ctl_carve(unsigned char* lds, int D, int M, int N, int r, int fcap, int esz) {
  CtlLds c;
  unsigned char* p = lds;
  c.w2s = p; p += ((size_t)M * r * esz + 15) / 16 * 16;
  c.front = reinterpret_cast<uint64_t*>(p); p += (size_t)fcap * 8;
  c.red64 = reinterpret_cast<uint64_t*>(p); p += 4 * 8;
  c.cid = reinterpret_cast<int*>(p); p += (size_t)D * M * 4;
  c.cval = reinterpret_cast<float*>(p); p += (size_t)D * M * 4;
  c.crank = reinterpret_cast<int*>(p); p += (size_t)D * M * 4;
  c.tailv = reinterpret_cast<float*>(p); p += (size_t)D * 4;
  c.ntok = reinterpret_cast<int*>(p); p += (size_t)(N + 1) * 4;
  c.npar = reinterpret_cast<int*>(p); p += (size_t)(N + 1) * 4;
  c.ndep = reinterpret_cast<int*>(p); p += (size_t)(N + 1) * 4;
  c.nstep = reinterpret_cast<int*>(p); p += (size_t)(N + 1) * 4;
  c.nscore = reinterpret_cast<float*>(p); p += (size_t)(N + 1) * 4;
  c.av = reinterpret_cast<float*>(p); p += (size_t)r * 4;
  c.ps = reinterpret_cast<float*>(p); p += (size_t)r * 4;
  c.z = reinterpret_cast<float*>(p); p += 64 * 4;
  c.logp = reinterpret_cast<float*>(p); p += 64 * 4;
  c.okf = reinterpret_cast<int*>(p); p += 64 * 4;
  c.misc = reinterpret_cast<int*>(p); p += 16 * 4;
  c.redpos = reinterpret_cast<int*>(p); p += 4 * 4;
  c.redf = reinterpret_cast<float*>(p); p += 4 * 4;
  return c;
}

__device__ __forceinline__ float sigm(float x) { return 1.0f / (1.0f + expf(-x)); }

// Load the W2 rows of depth row dy's candidates and its P row into LDS.
// Issued while the controller waits for the workers, so the expansion that
// follows reads only LDS and the published u.
template <typename W>
__device__ __forceinline__ void ctl_prefetch(const TreeArgs& a, const CtlLds& c, int b, int dy) {
  const int tid = threadIdx.x, M = a.M, r = a.r;
  W* dst = reinterpret_cast<W*>(c.w2s);
  const W* w2t = reinterpret_cast<const W*>(a.w2t);
  const int per = r * (int)sizeof(W) / 16;   // 16-byte pieces per row
  if ((r * (int)sizeof(W)) % 16 == 0 && per <= 256 && 256 % per == 0) {
    const int rpt = 256 / per;                 // rows per pass
    const int pc = tid % per, m0 = tid / per;
    constexpr int U = 8;
    for (int mb = 0; mb < M; mb += U * rpt) {
      uint4 v[U];
#pragma unroll
      for (int q = 0; q < U; ++q) {  // clamped: every lane loads a valid piece
        const int m = min(mb + m0 + q * rpt, M - 1);
        v[q] = reinterpret_cast<const uint4*>(w2t + (size_t)c.cid[dy * M + m] * r)[pc];
      }
#pragma unroll
      for (int q = 0; q < U; ++q) {  // unconditional: see the worker's staging
        const int m = min(mb + m0 + q * rpt, M - 1);
        reinterpret_cast<uint4*>(dst)[m * per + pc] = v[q];
      }
    }
  } else {
    for (int i = tid; i < M * r; i += blockDim.x) dst[i] = w2t[(size_t)c.cid[dy * M + i / r] * r + i % r];
  }
  const float* prow = a.P + ((size_t)b * a.D + dy) * r;
  for (int j = tid; j < r; j += blockDim.x) c.ps[j] = prow[j];
}

// score the children of node y (depth dy < D) and push the k best
template <typename W>
__device__ __forceinline__ void ctl_expand(const TreeArgs& a, const CtlLds& c, int b, int y, int t) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int M = a.M, r = a.r;
  const int dy = c.ndep[y];        // children are at depth dy + 1; row dy of the tables
  const float* urow = a.u + slot_of(a, t, b) * u_stride(r);
  for (int j = tid; j < r; j += blockDim.x) {
    const float x = urow[j] + c.ps[j];
    c.av[j] = x * sigm(x);  // SiLU
  }
  __syncthreads();
  // dL_m = W2[:, cand_m] . a: tpc threads per candidate, each a contiguous
  // slice of the rank, combined in a fixed order
  int tpc = 1;
  while (tpc * 2 * M <= (int)blockDim.x && tpc < 64) tpc *= 2;
  const int m = tid / tpc, part = tid % tpc;
  const int len = (r + tpc - 1) / tpc;
  float dl = 0.f;
  if (m < M) {
    const W* wrow = reinterpret_cast<const W*>(c.w2s) + (size_t)m * r;
    const int j0 = part * len, j1 = min(r, j0 + len);
    constexpr int VE = 16 / sizeof(W);  // elements per 16-byte piece
    if (j1 - j0 == len && len % VE == 0 && (r * (int)sizeof(W)) % 16 == 0) {
      for (int j = j0; j < j1; j += VE) {
        const uint4 wv = *reinterpret_cast<const uint4*>(wrow + j);
        const W* we = reinterpret_cast<const W*>(&wv);
#pragma unroll
        for (int q = 0; q < VE; q += 4) {
          const float4 av = *reinterpret_cast<const float4*>(c.av + j + q);
          dl = fmaf(w_to_f32<W>(we[q]), av.x, dl);
          dl = fmaf(w_to_f32<W>(we[q + 1]), av.y, dl);
          dl = fmaf(w_to_f32<W>(we[q + 2]), av.z, dl);
          dl = fmaf(w_to_f32<W>(we[q + 3]), av.w, dl);
        }
      }
    } else {
      for (int j = j0; j < j1; ++j) dl = fmaf(w_to_f32<W>(wrow[j]), c.av[j], dl);
    }
  }
  for (int s = 1; s < tpc; s <<= 1) dl += __shfl_xor(dl, s);
  if (m < M && part == 0) c.z[m] = (c.cval[dy * M + m] + dl) / a.T + 0.0f;
  __syncthreads();
  // wave 0, one candidate per lane: log-softmax over the candidates (plus the
  // base tail under fullv), rank by (z desc, token asc), push the k best with
  // a finite log-prob.  -inf log-probs rank after every finite one, so the
  // children take ranks 0..n-1.
  if (tid < 64) {
    const bool has = lane < M;
    const float zv = has ? c.z[lane] : -INFINITY;
    const int idv = has ? c.cid[dy * M + lane] : 0x7FFFFFFF;
    float mx = wave_max(zv);
    const float tl = a.fullv ? c.tailv[dy] : -INFINITY;
    mx = fmaxf(mx, tl);
    float lz = -INFINITY;
    if (mx > -INFINITY) {
      float se = wave_sum(has ? expf(zv - mx) : 0.f);
      if (tl > -INFINITY) se += expf(tl - mx);
      lz = mx + logf(se);
    }
    const float lp = zv - lz;
    int rank = 0;
    for (int q = 0; q < M; ++q) {
      const float zq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(zv), q));
      const int iq = __builtin_amdgcn_readlane(idv, q);
      rank += (zq > zv) || (zq == zv && iq < idv);
    }
    const bool ok = has && rank < a.k && isfinite(lp);
    const int base = c.misc[0];
    if (ok) c.front[base + rank] = make_key(c.nscore[y] + lp, dy + 1, c.crank[dy * M + lane], y, lane);
    const unsigned long long bal = __ballot(ok);
    if (lane == 0) c.misc[0] = base + __popcll(bal);
  }
  __syncthreads();
}

// Wave 0 pops frontier entries in order, recording each as the next node,
// until it finds one to expand (depth < D and index < N), the budget is met
// or the frontier is empty.  Returns the node to expand or -1; updates *n.
// Called by all threads; only wave 0 works, then one barrier.
__device__ __forceinline__ int ctl_pop_until_expandable(const CtlLds& c, int D, int M, int N, int* n) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < 64) {
    int cnt = c.misc[0];
    int nn = *n;
    int next = -1;
    while (nn < N && cnt > 0) {
      uint64_t best = 0;
      int pos = -1;
      for (int i = lane; i < cnt; i += 64) {
        const uint64_t k = c.front[i];
        if (pos < 0 || k > best) {
          best = k;
          pos = i;
        }
      }
      const uint64_t g = wave_max_u64(pos < 0 ? 0ull : best);
      const unsigned long long hit = __ballot(pos >= 0 && best == g);  // keys are unique
      const int src = __ffsll((long long)hit) - 1;
      const int gpos = __shfl(pos, src);
      const int i = nn + 1;
      const int d = key_depth(g);
      if (lane == 0) {
        c.front[gpos] = c.front[cnt - 1];
        c.ntok[i] = c.cid[(d - 1) * M + key_slot(g)];
        c.npar[i] = key_parent(g);
        c.ndep[i] = d;
        c.nscore[i] = key_score(g);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      --cnt;
      nn = i;
      if (d < D && i < N) {
        next = i;
        break;
      }
    }
    if (lane == 0) {
      c.misc[0] = cnt;
      c.misc[4] = nn;
      c.misc[5] = next;
    }
  }
  __syncthreads();
  *n = c.misc[4];
  return c.misc[5];
}

template <typename W>
__device__ __forceinline__ void ctl_advance_state(const TreeArgs& a, int b, int y, int x, int tok, int tx,
                                                  int ty) {
  // x was expanded at step tx; y is published for step ty
  // S_y = GRU(S_x, E[tok]) with W_ih E[tok] + b_ih = G[tok] and gh_x = W_hh S~_x + b_hh
  const int ds = a.ds;
  const float* gi = a.G + (size_t)tok * 3 * ds;
  const float* gh = a.gh + slot_of(a, tx, b) * gh_stride(ds);
  const float* sx = a.state + ((size_t)b * (a.N + 1) + x) * st_stride(ds);
  float* sy = a.state + ((size_t)b * (a.N + 1) + y) * st_stride(ds);
  W* ay = reinterpret_cast<W*>(a.act) + slot_of(a, ty, b) * act_stride(ds);
  if ((ds & 3) == 0) {
    for (int j = 4 * threadIdx.x; j < ds; j += 4 * blockDim.x) {
      const float4 ir = *reinterpret_cast<const float4*>(gi + j);
      const float4 iz = *reinterpret_cast<const float4*>(gi + ds + j);
      const float4 in = *reinterpret_cast<const float4*>(gi + 2 * ds + j);
      const float4 hr = *reinterpret_cast<const float4*>(gh + j);
      const float4 hz = *reinterpret_cast<const float4*>(gh + ds + j);
      const float4 hn = *reinterpret_cast<const float4*>(gh + 2 * ds + j);
      const float4 sp = *reinterpret_cast<const float4*>(sx + j);
      const float a0[4] = {ir.x, ir.y, ir.z, ir.w}, b0[4] = {hr.x, hr.y, hr.z, hr.w};
      const float a1[4] = {iz.x, iz.y, iz.z, iz.w}, b1[4] = {hz.x, hz.y, hz.z, hz.w};
      const float a2[4] = {in.x, in.y, in.z, in.w}, b2[4] = {hn.x, hn.y, hn.z, hn.w};
      const float s0[4] = {sp.x, sp.y, sp.z, sp.w};
      floatx4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float rg = sigm(a0[q] + b0[q]);
        const float zg = sigm(a1[q] + b1[q]);
        const float ng = tanhf(a2[q] + rg * b2[q]);
        o[q] = (1.0f - zg) * ng + zg * s0[q];
      }
      st_dev_f32x4(sy + j, o);
      st_dev_act4<W>(ay + j, o, a.act_bf16);
    }
  } else {
    for (int j = threadIdx.x; j < ds; j += blockDim.x) {
      const float rg = sigm(gi[j] + gh[j]);
      const float zg = sigm(gi[ds + j] + gh[ds + j]);
      const float ng = tanhf(gi[2 * ds + j] + rg * gh[2 * ds + j]);
      const float s = (1.0f - zg) * ng + zg * sx[j];
      st_dev_f32(sy + j, s);
      st_dev_act<W>(ay + j, s, a.act_bf16);
    }
  }
  for (int j = ds + threadIdx.x; j < k_padded(ds); j += blockDim.x) st_dev_act<W>(ay + j, 0.f, 0);
}

template <typename W>
__device__ __forceinline__ void controller_main(const TreeArgs& a, unsigned char* lds) {
  const int b = blockIdx.x - a.n_workers;
  const int tid = threadIdx.x;
  const int D = a.D, M = a.M, N = a.N;
  const int fcap = a.N * (a.k - 1) + 1;
  CtlLds c = ctl_carve(lds, D, M, N, a.r, fcap, (int)sizeof(W));

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
    W* a0 = reinterpret_cast<W*>(a.act) + slot_of(a, 0, b) * act_stride(ds);
    for (int j = tid; j < ds; j += blockDim.x) {
      const float v = a.root ? a.root[(size_t)b * ds + j] : 0.f;
      st_dev_f32(s0 + j, v);
      st_dev_act<W>(a0 + j, v, a.act_bf16);
    }
    for (int j = ds + tid; j < k_padded(ds); j += blockDim.x) st_dev_act<W>(a0 + j, 0.f, 0);
  }
  if (tid == 0) c.nstep[0] = 0;
  stores_done();
  __syncthreads();
  if (tid < a.n_workers) st_dev_u32(a.mbox_w + (size_t)tid * 32 + b, 1u);  // step 0 posted
  for (int w = tid + 256; w < a.n_workers; w += 256) st_dev_u32(a.mbox_w + (size_t)w * 32 + b, 1u);
  stores_done();
  __syncthreads();

  ctl_prefetch<W>(a, c, b, 0);  // the root's children are at depth 1
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
    ctl_expand<W>(a, c, b, y, t);
    // pop until a node to expand is found, the budget is met or the frontier is empty
    const int next = ctl_pop_until_expandable(c, D, M, N, &n);
    if (next < 0) break;
    ctl_advance_state<W>(a, b, next, c.npar[next], c.ntok[next], c.nstep[c.npar[next]], t + 1);
    if (tid == 0) c.nstep[next] = t + 1;
    stores_done();
    __syncthreads();
    for (int w = tid; w < a.n_workers; w += blockDim.x)
      st_dev_u32(a.mbox_w + (size_t)w * 32 + b, epoch + 1u);
    stores_done();
    ctl_prefetch<W>(a, c, b, c.ndep[next]);  // overlaps the workers' step
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
  const size_t c = ctl_lds_bytes(a.D, a.M, a.N, a.r, a.N * (a.k - 1) + 1, wdtype_bf16 ? 2 : 4);
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
