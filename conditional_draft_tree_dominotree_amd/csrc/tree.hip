// The conditional best-first tree builder: one persistent kernel.
//
// Method (DominoTree technical summary, Componenti Core 1, 2 and 4; Domino
// summary, 核心方法): per request, repeatedly take the frontier node with the
// highest cumulative log-prob, advance the GRU causal state along that node's
// path, correct the next depth's M candidate logits with
// W2[:, cand] SiLU(W1 [H; S]), log-softmax them and push the k best children,
// until N nodes have been taken.
//
// The tree this returns is the one the one-node-at-a-time loop returns: its N
// nodes are the N best nodes of the whole k-restricted tree under the total
// order (score desc, depth asc, token asc, parent's order asc), because a
// child always comes after its parent in that order.  The kernel uses this to
// expand up to p frontier nodes of a request per step instead of one:
//   * a frontier entry f is taken into the request's record set X only if
//     fewer than N + 1 records of X (the root included) precede it in the
//     total order (otherwise it, and everything after it, can never be among
//     the N best: X only grows);
//   * the first node taken in a step is always one of the N best (every node
//     that precedes it is already in X); the others are speculative and may
//     later be pushed out by descendants of earlier ones;
//   * the build ends when the frontier holds no entry that passes the test;
//     the output is X ranked by the total order, cut after N + 1 records.
// Speculation changes how much work is done, never the result.
//
// Roles (blocks of 256 threads, one per CU, all resident at once: they wait
// on each other, so the grid never exceeds the GPU's CUs; a plain launch by
// default, a cooperative one on request):
//   * worker blocks [0, n_workers) keep tiles of the per-node product
//     Wc = [W_hh ; W1_S^T] ((3 d_s + r) x d_s) for the whole launch: at
//     d_s = 1024 in bf16 as MFMA operands in registers ("register workers"),
//     otherwise `tiles_per_worker` 16-row tiles in LDS.  Each step they
//     multiply their rows by the GEMM operand copies of the states expanded in
//     that step (one column per expanded node) and publish
//     gh = W_hh S~ + b_hh and u = W1_S^T S~.  Register workers own fixed
//     columns (node c % p of a request of their column group), read each
//     column's node (token, parent slot) from a node entry its controller
//     writes, and advance those nodes' GRU states themselves from
//     G[token] = W_ih E[token] + b_ih (a table folded once per handle) and the
//     parents' gh before the product.
//   * controller blocks [n_workers, n_workers + B): one per request.  It keeps
//     the request's candidates, node records and sorted frontier in LDS;
//     scores the children of the nodes expanded in the step
//     (a = SiLU(u + P_d), dL on the M candidate columns of W2, log-softmax,
//     top-k), merges them into the frontier, takes the next nodes and
//     publishes them (node entries for register workers; beside LDS workers
//     it advances their states itself and raises mailbox words).
//
// Exchange between blocks: every published value is written once per launch
// to its own 128-byte-aligned slot with device-scope (sc1) stores; after the
// stores complete the producer raises a word its consumers poll with sc1
// loads (a node entry carrying the step's epoch, an acknowledgement, a group
// flag, or a mailbox word in eight copies of one line), and the consumer then
// reads the published slots.  Slots are never read before they are
// published, so no cache holds a stale copy.  The blocks of a register-worker
// column group that run on one XCD raise their group flags in that XCD's L2
// (sc0 stores).  Every wait is bounded: when it runs out the block sets the
// error word and leaves its loop.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "tree.h"

namespace dt {

constexpr uint32_t MBOX_DONE_E = 31u;  // node count field of a request's last word (no more steps)
constexpr int NT = 256;      // threads per block (every block of the builder)
constexpr int PMAX = 16;     // nodes per request per step
constexpr int QCAP = 32;     // frontier entries tested per pop round
constexpr int FCAPMAX = 6144;  // frontier entries per request
constexpr int XMAX = 2047;   // records per request (11-bit parent field)
constexpr int PPW = 2;       // (tile, column block) pairs per worker wave
constexpr int GA = 8;        // states advanced together per controller thread

// ---------------------------------------------------------------------------
// device-scope memory operations

__device__ __forceinline__ void st_dev_u32(void* p, uint32_t v) {
  asm volatile("global_store_dword %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void st_dev_u16(void* p, uint32_t v) {
  asm volatile("global_store_short %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
// A store of more than 8 bytes reads its data registers after it issues; the
// compiler does not see into the asm, so the asm itself waits out that window
// before any following instruction may overwrite them.
__device__ __forceinline__ void st_dev_f32x4(void* p, floatx4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ uint32_t ld_dev_u32(const void* p) {
  uint32_t v;
  asm volatile("global_load_dword %0, %1, off sc1\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
  return v;
}
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// A block barrier that waits only for this wave's LDS operations (a
// __syncthreads also waits for its outstanding global loads and stores).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Keeps the instruction scheduler from moving anything across this point.  Put
// between the loads of a batch and their uses, so that every load of the
// batch is in flight at once instead of being sunk next to its use (which
// the scheduler does under register pressure, one memory round trip each).
__device__ __forceinline__ void keep_batch() { __builtin_amdgcn_sched_barrier(0); }

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

__device__ __forceinline__ void st_dev_u64(void* p, uint64_t v) {
  asm volatile("global_store_dwordx2 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void st_dev_u32x2(void* p, uint32_t lo, uint32_t hi) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  u32x2 v = {lo, hi};
  asm volatile("global_store_dwordx2 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
// Stores that stop at the XCD's L2 (sc0; no write-through), for exchanges
// between blocks known to run on one XCD: such a block sees them with the
// device-coherent loads (sc1) that bypass its L1, and with plain loads of lines
// it has not read before.  Measured between two CUs of one XCD, a flag stored
// this way is seen about 0.2 us sooner than one stored with sc1.
__device__ __forceinline__ void st_l2_u32(void* p, uint32_t v) {
  asm volatile("global_store_dword %0, %1, off sc0" ::"v"(p), "v"(v) : "memory");
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

// Logistic function and tanh from the hardware exp2 and reciprocal (about
// 1e-7 relative error; a tanh near 0 is accurate to about 1e-7 absolute).
__device__ __forceinline__ float sigm(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}
__device__ __forceinline__ float tanh_(float x) { return 2.0f * sigm(2.0f * x) - 1.0f; }

// ---------------------------------------------------------------------------
// layout helpers

__host__ __device__ constexpr int round_up(int x, int m) { return (x + m - 1) / m * m; }
__host__ __device__ inline int act_stride(int ds) { return round_up(ds, 64); }     // elements
__host__ __device__ inline int k_padded(int ds) { return round_up(ds, 32); }
__host__ __device__ inline int st_stride(int ds) { return round_up(ds, 32); }      // floats
__host__ __device__ inline int gh_stride(int ds) { return round_up(3 * ds, 32); }  // floats
__host__ __device__ inline int u_stride(int r) { return round_up(r, 32); }         // floats
constexpr int STAGE_PAD = 8;  // extra elements per staged column (bank spread)

// exchange slot of the j-th node a request expands at step t
__device__ __forceinline__ size_t slot_of(const TreeArgs& a, int t, int b, int j) {
  return ((size_t)t * a.B + b) * a.p + j;
}

// Frontier entry / record key, larger = earlier in the total order:
//   [63:32] score | [31:27] 31 - depth | [26:21] 63 - token rank |
//   [20:10] parent record | [9:4] candidate slot m
// The upper 43 bits (score, depth, token) decide the order except between
// nodes of equal score at the same depth with the same token, which the
// parents' order decides (rec_better).  The parent field of a record's own key
// goes stale when records are renumbered; rpar holds the current one.
__device__ __forceinline__ uint64_t make_key(float score, int depth, int tokrank, int parent, int m) {
  return ((uint64_t)f32_key(score) << 32) | ((uint64_t)(31 - depth) << 27) | ((uint64_t)(63 - tokrank) << 21) |
         ((uint64_t)parent << 10) | ((uint64_t)m << 4);
}
__device__ __forceinline__ uint64_t key_u(uint64_t k) { return k >> 21; }
__device__ __forceinline__ float key_score(uint64_t k) { return key_f32((uint32_t)(k >> 32)); }
__device__ __forceinline__ int key_depth(uint64_t k) { return 31 - (int)((k >> 27) & 31); }
__device__ __forceinline__ int key_parent(uint64_t k) { return (int)((k >> 10) & 2047); }
__device__ __forceinline__ int key_m(uint64_t k) { return (int)((k >> 4) & 63); }
__device__ __forceinline__ uint64_t key_with_parent(uint64_t k, int parent) {
  return (k & ~(2047ull << 10)) | ((uint64_t)parent << 10);
}

// Bounded wait, wave-uniform: poll the words at p[0..Q) of every lane until
// all are >= need.  Two polls are in flight at a time: the next one is issued
// before the previous one is examined, so a word that lands is seen about half
// a load latency sooner than with polls issued one after the other.  The loads
// are device-coherent (relaxed, agent scope).  On success *word0, when given,
// receives what the deciding poll read at p[0].
template <int Q>
__device__ __forceinline__ bool wait_ptrs(const uint32_t* const (&p)[Q], uint32_t need, const int* err,
                                          unsigned limit, uint32_t* word0) {
  const int lane = threadIdx.x & 63;
  uint32_t x[Q], y[Q];
  auto issue = [&](uint32_t (&v)[Q]) {
#pragma unroll
    for (int q = 0; q < Q; ++q) v[q] = __hip_atomic_load(p[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  auto all_in = [&](const uint32_t (&v)[Q]) {
    bool ok = true;
#pragma unroll
    for (int q = 0; q < Q; ++q) ok &= v[q] >= need;
    return __all(ok);
  };
  issue(x);
  unsigned it = 0;
  while (true) {
    __builtin_amdgcn_s_sleep(1);
    issue(y);
    if (all_in(x)) {
      if (word0) *word0 = x[0];
      break;
    }
    __builtin_amdgcn_s_sleep(1);
    issue(x);
    if (all_in(y)) {
      if (word0) *word0 = y[0];
      break;
    }
    if ((++it & 127) == 0) {
      if (ld_dev_u32(err) != 0) return false;
      if (2 * it > limit) {
        if (lane == 0) atomicOr((int*)err, 1);
        return false;
      }
    }
  }
  asm volatile("" ::: "memory");  // what the caller reads next stays after the poll that saw the words
  return true;
}
// The words box[0..nwords) (nwords <= 64 Q); lanes past nwords re-read the
// last word; *word0 receives box[min(lane, nwords - 1)].
template <int Q>
__device__ __forceinline__ bool wait_words(const uint32_t* box, int nwords, uint32_t need, const int* err,
                                           unsigned limit, uint32_t* word0) {
  const int lane = threadIdx.x & 63;
  const uint32_t* p[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) p[q] = box + min(lane + 64 * q, nwords - 1);
  return wait_ptrs<Q>(p, need, err, limit, word0);
}

__device__ __forceinline__ bool wait_mbox(const uint32_t* box, int nwords, uint32_t need, const int* err,
                                          unsigned limit, uint32_t* word0 = nullptr) {
  if (nwords <= 0) return true;
  if (nwords <= 64) return wait_words<1>(box, nwords, need, err, limit, word0);
  if (nwords <= 256) return wait_words<4>(box, nwords, need, err, limit, word0);
  const int lane = threadIdx.x & 63;
  unsigned it = 0;
  while (true) {
    bool ok = true;
    for (int i = lane; i < nwords; i += 64) ok &= ld_dev_u32(box + i) >= need;
    if (__all(ok)) {
      if (word0) *word0 = ld_dev_u32(box + min(lane, nwords - 1));
      return true;
    }
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

// controller -> worker mailbox word: step epoch in the high bits, nodes expanded
// by the request in that step in the low 5 (MBOX_DONE_E: the request is done).
// Epochs run from ebase + 1 within a launch and only grow across launches, so
// no mailbox needs clearing between builds.
__device__ __forceinline__ uint32_t mbox_word(uint32_t epoch, uint32_t e) { return (epoch << 5) | e; }

// ---------------------------------------------------------------------------
// worker: per-step product of its Wc tiles with the expanded nodes' states

// LDS: tiles [tpw][kp/32][4][16][8] elements, staged columns
// [round_up(cols, 16)][kc + STAGE_PAD], then the column tables
__host__ __device__ inline size_t worker_stage_offset(int tpw, int kp, int esz) {
  return (size_t)tpw * 16 * kp * esz;
}
__host__ __device__ inline size_t worker_lds_bytes(int tpw, int kp, int kc, int cols, int esz) {
  return worker_stage_offset(tpw, kp, esz) + (size_t)round_up(cols, 16) * (kc + STAGE_PAD) * esz +
         (size_t)(2 * TREE_MAX_COLS + 64) * 4;
}

__device__ __forceinline__ void worker_store_out(const TreeArgs& a, size_t slot, int row, float v) {
  const int ds3 = 3 * a.ds;
  if (row < ds3) {
    st_dev_f32(a.gh + slot * gh_stride(a.ds) + row, v + (a.b_hh ? a.b_hh[row] : 0.f));
  } else if (row < ds3 + a.r) {
    st_dev_f32(a.u + slot * u_stride(a.r) + (row - ds3), v);
  }
}

// A uniform address as a scalar register pair (the base operand of the
// batched loads): the compiler may keep uniform values in vector registers
// where scalar registers are short.  The batches begin with s_nop 4: a vector
// instruction that writes a scalar register (v_readfirstlane here, v_readlane
// for a spilled one) needs five wait states before a memory instruction reads
// that register as its address, and the compiler does not look inside asm.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const void*>((uintptr_t)(((uint64_t)hi << 32) | lo));
}

// Sixteen 16-byte loads from base + off[q] (byte offsets), issued back to back
// and completed together.  One asm block, so that register pressure elsewhere
// in the kernel cannot make the compiler wait after each load.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void load16_batch(const void* base, const unsigned (&off)[16], u32x4 (&v)[16]) {
  asm volatile(
      "s_nop 4\n\t"  // the base may have been written by a vector instruction just before
      "global_load_dwordx4 %0, %16, %32\n\t"
      "global_load_dwordx4 %1, %17, %32\n\t"
      "global_load_dwordx4 %2, %18, %32\n\t"
      "global_load_dwordx4 %3, %19, %32\n\t"
      "global_load_dwordx4 %4, %20, %32\n\t"
      "global_load_dwordx4 %5, %21, %32\n\t"
      "global_load_dwordx4 %6, %22, %32\n\t"
      "global_load_dwordx4 %7, %23, %32\n\t"
      "global_load_dwordx4 %8, %24, %32\n\t"
      "global_load_dwordx4 %9, %25, %32\n\t"
      "global_load_dwordx4 %10, %26, %32\n\t"
      "global_load_dwordx4 %11, %27, %32\n\t"
      "global_load_dwordx4 %12, %28, %32\n\t"
      "global_load_dwordx4 %13, %29, %32\n\t"
      "global_load_dwordx4 %14, %30, %32\n\t"
      "global_load_dwordx4 %15, %31, %32\n\t"
      "s_waitcnt vmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7]),
        "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]), "=&v"(v[12]), "=&v"(v[13]), "=&v"(v[14]), "=&v"(v[15])
      : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "v"(off[4]), "v"(off[5]), "v"(off[6]), "v"(off[7]),
        "v"(off[8]), "v"(off[9]), "v"(off[10]), "v"(off[11]), "v"(off[12]), "v"(off[13]), "v"(off[14]), "v"(off[15]),
        "s"(uniform_ptr(base))
      : "memory");
}

// Copy elements [k0, k0 + kc) of each active column's operand into the stage.
// Thread tid owns 16-byte piece tid % per of columns tid / per + j * cpt;
// every load of a batch is issued before any store.  slot0 is the first
// exchange slot of the step (its columns lie in the next TREE_MAX_COLS slots,
// so byte offsets from it fit 32 bits).
template <typename W>
__device__ __forceinline__ void worker_stage(const TreeArgs& a, W* stage, const int* coln, int ncols, int k0,
                                             int kc, int slot0) {
  const int tid = threadIdx.x;
  const int as = act_stride(a.ds);
  const int kcs = kc + STAGE_PAD;
  const int per = kc * (int)sizeof(W) / 16;  // 16-byte pieces per column
  const W* act = reinterpret_cast<const W*>(a.act);
  if (per <= 256 && 256 % per == 0) {
    const int cpt = 256 / per;  // columns per pass
    const int pc = tid % per, c0 = tid / per;
    constexpr int U = 16;
    const W* base = act + (size_t)slot0 * as + k0;
    for (int cb = 0; cb < ncols; cb += U * cpt) {
      unsigned off[U];
      u32x4 v[U];
#pragma unroll
      for (int q = 0; q < U; ++q) {  // clamped: every lane loads a valid piece
        const int c = min(cb + c0 + q * cpt, ncols - 1);
        off[q] = (unsigned)(((coln[c] - slot0) * as + pc * (16 / (int)sizeof(W))) * (int)sizeof(W));
      }
      load16_batch(base, off, v);
      // unconditional stores (a clamped duplicate rewrites identical data)
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const int c = min(cb + c0 + q * cpt, ncols - 1);
        *reinterpret_cast<u32x4*>(stage + (size_t)c * kcs + pc * (16 / sizeof(W))) = v[q];
      }
    }
  } else {
    for (int i = tid; i < ncols * per; i += NT) {
      const int c = i / per, pc = i % per;
      *reinterpret_cast<uint4*>(stage + (size_t)c * kcs + pc * (16 / sizeof(W))) =
          reinterpret_cast<const uint4*>(act + (size_t)coln[c] * as + k0)[pc];
    }
  }
}

// bf16: MFMA 16x16x32 over the k blocks [kb0, kb0 + nkb) staged in this phase;
// wave w owns (tile, column block) pairs w, w + 4, ... (at most PPW)
__device__ __forceinline__ void worker_mfma_phase(const uint16_t* tiles_lds, const uint16_t* stage, int kp,
                                                  int kb0, int nkb, int kcs, int ncb, int pairs,
                                                  floatx4 (&acc)[PPW][2]) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    const int pair = wv + 4 * i;
    if (pair < pairs) {
      const int tt = pair / ncb, cb = pair - tt * ncb;
      const uint16_t* wt = tiles_lds + (size_t)tt * 16 * kp + (size_t)kb0 * 512;
      const uint16_t* sc = stage + (size_t)(cb * 16 + (lane & 15)) * kcs + 8 * (lane >> 4);
      int kb = 0;
      for (; kb + 4 <= nkb; kb += 4) {
        bf16x8 av[4], bv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          av[q] = *reinterpret_cast<const bf16x8*>(wt + ((size_t)(kb + q) * 64 + lane) * 8);
          bv[q] = *reinterpret_cast<const bf16x8*>(sc + (kb + q) * 32);
        }
        acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[0], bv[0], acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[1], bv[1], acc[i][1], 0, 0, 0);
        acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[2], bv[2], acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[3], bv[3], acc[i][1], 0, 0, 0);
      }
      for (; kb < nkb; ++kb) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(wt + ((size_t)kb * 64 + lane) * 8);
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(sc + kb * 32);
        acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[i][0], 0, 0, 0);
      }
    }
  }
}

__device__ __forceinline__ void worker_epilogue_bf16(const TreeArgs& a, const int* coln, int ncols, int tile0,
                                                     int ncb, int pairs, floatx4 (&acc)[PPW][2]) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ds3 = 3 * a.ds;
#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    const int pair = wv + 4 * i;
    if (pair < pairs) {
      const int tt = pair / ncb, cb = pair - tt * ncb;
      const int col = cb * 16 + (lane & 15);
      // lane holds column (lane & 15), rows 4 (lane >> 4) + q of the tile
      if (col < ncols) {
        const floatx4 s = acc[i][0] + acc[i][1];
        const size_t slot = (size_t)coln[col];
        const int row0 = (tile0 + tt) * 16 + 4 * (lane >> 4);
        if (row0 + 3 < ds3 && (ds3 & 3) == 0) {
          const float* bh = a.b_hh;
          floatx4 v = s;
          if (bh) {
            v[0] += bh[row0];
            v[1] += bh[row0 + 1];
            v[2] += bh[row0 + 2];
            v[3] += bh[row0 + 3];
          }
          st_dev_f32x4(a.gh + slot * gh_stride(a.ds) + row0, v);
        } else if (row0 >= ds3 && row0 + 3 < ds3 + a.r && (ds3 & 3) == 0 && (a.r & 3) == 0) {
          st_dev_f32x4(a.u + slot * u_stride(a.r) + (row0 - ds3), s);
        } else {
          for (int q = 0; q < 4; ++q) worker_store_out(a, slot, row0 + q, s[q]);
        }
      }
    }
  }
}

// fp32: one (row, column) dot product per thread over the staged k (one phase)
__device__ __forceinline__ void worker_compute_f32(const TreeArgs& a, const float* tiles_lds, const float* stage,
                                                   int ncols, const int* coln, int tile0, int ntiles, int kp,
                                                   int kcs) {
  const int total = ntiles * 16 * ncols;
  for (int idx = threadIdx.x; idx < total; idx += NT) {
    const int col = idx % ncols;
    const int rr = (idx / ncols) % 16;
    const int tt = idx / (ncols * 16);
    const float* wt = tiles_lds + (size_t)tt * 16 * kp;
    const float* sc = stage + (size_t)col * kcs;
    float s = 0.f;
    for (int k = 0; k < kp; ++k) {
      const int kb = k >> 5, kg = (k >> 3) & 3, e = k & 7;
      s = fmaf(wt[(((size_t)kb * 4 + kg) * 16 + rr) * 8 + e], sc[k], s);
    }
    worker_store_out(a, (size_t)coln[col], (tile0 + tt) * 16 + rr, s);
  }
}

// Wave 0 waits for every request's word of step t in worker w's mailbox, then
// lists the step's columns (exchange slots, request-major) in coln and the
// requests with work in reqs; misc[0] = columns (-1: a wait ran out),
// misc[1] = requests.  Ends with a block barrier.
// The columns of the nodes that the requests [b0, b0 + nb) expand at step t:
// waits for those requests' mailbox words, then lists their exchange slots in
// coln and the requests with nodes in reqs; misc[0] = column count (-1: a wait
// ran out; 0: every one of these requests is finished), misc[1] = request count.
__device__ __forceinline__ void worker_columns(const TreeArgs& a, int w, int t, int b0, int nb, int* coln, int* reqs,
                                               int* misc) {
  const int tid = threadIdx.x, lane = tid & 63;
  const uint32_t epoch = a.ebase + (uint32_t)t + 1u;
  if (tid < 64) {
    const uint32_t* mybox = a.mbox_w + (size_t)(w % MBOX_REPL) * 32 + b0;
    uint32_t word = 0;
    const bool ok = wait_mbox(mybox, nb, epoch << 5, a.err, a.spin_limit, &word);
    const int b = b0 + lane;
    const int e = (ok && lane < nb && (word & 31u) != MBOX_DONE_E) ? (int)(word & 31u) : 0;
    // exclusive prefix of e over the lanes
    int incl = e;
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    const int base = incl - e;
    for (int j = 0; j < e; ++j) coln[base + j] = (int)slot_of(a, t, b, j);
    const unsigned long long has = __ballot(e > 0);
    if (e > 0) reqs[__popcll(has & ((1ull << lane) - 1ull))] = b;
    if (lane == 63) misc[0] = ok ? incl : -1;
    if (lane == 0) misc[1] = __popcll(has);
  }
  __syncthreads();
}

// Poll, per lane, the node entry at p (lanes with poll false: none) until
// every polled entry carries the step's 24-bit epoch ep; two polls in flight,
// as in wait_ptrs.  False if the wait ran out or the error word is set.
__device__ __forceinline__ bool wait_entries(const uint64_t* p, bool poll, uint32_t ep, const int* err,
                                             unsigned limit, uint64_t& out) {
  const int lane = threadIdx.x & 63;
  auto in = [&](uint64_t v) { return !poll || (uint32_t)(v >> 40) == ep; };
  uint64_t x = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), y;
  unsigned it = 0;
  while (true) {
    __builtin_amdgcn_s_sleep(1);
    y = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__all(in(x))) {
      out = x;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
    x = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__all(in(y))) {
      out = y;
      break;
    }
    if ((++it & 127) == 0) {
      if (ld_dev_u32(err) != 0) return false;
      if (2 * it > limit) {
        if (lane == 0) atomicOr((int*)err, 1);
        return false;
      }
    }
  }
  asm volatile("" ::: "memory");
  return true;
}

// Register workers: the columns of block w's group at step t for the requests
// [hb0, hb0 + hn) of a half.  Column c of the half is node c % p of request
// hb0 + c / p; the block polls the node entries of its columns [col0, col0 +
// nc) (nc <= 64) directly (no mailbox word first), except those of requests
// it has seen finish (the lanes in fin, updated here).  It writes coln[i]
// (i < nc): the slot staged for column col0 + i (a present column's slot where
// there is no node), and for the k-th present column coln[64 + k] its slot,
// coln[128 + k] its token, coln[192 + k] its parent's slot; reqs: the running
// requests among these columns'.  misc[0] = present columns (-1: a wait ran
// out), misc[1] = running requests, misc[4] = 1 when none is running,
// misc[6], misc[7] = the mask of present columns.
__device__ __forceinline__ void worker_columns_fixed(const TreeArgs& a, int t, int hb0, int hn, int col0, int nc,
                                                     unsigned long long& fin, int* coln, int* reqs, int* misc) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int p = a.p;
  const int c1 = min(col0 + nc, hn * p);
  if (tid < 64) {
    int nval = 0, nact = 0, none = 1;
    unsigned long long vm = 0;
    bool ok = true;
    if (col0 < c1) {
      const uint32_t ep = (a.ebase + (uint32_t)t + 1u) & 0xFFFFFFu;
      const int rb0 = col0 / p;  // the first request (within the half) of these columns
      const int c = col0 + lane;
      const bool col = lane < nc && c < c1;
      const bool poll = col && !((fin >> lane) & 1ull);
      const uint64_t* ptr = a.ninfo + (poll ? (size_t)t * TREE_MAX_COLS + (size_t)(hb0 + c / p) * p + c % p : 0);
      uint64_t en = 0;
      ok = wait_entries(ptr, poll, ep, a.err, a.spin_limit, en);
      const uint32_t tok = (uint32_t)(en >> 20) & 0xFFFFFu, src = (uint32_t)en & 0xFFFFFu;
      const bool done = col && (!poll || tok == NINFO_DONE);
      fin |= __ballot(done);
      const bool v = ok && poll && tok != NINFO_DONE && tok != NINFO_NONE;
      // a request's first column among these: it lists the request if running
      const bool first = col && (c % p == 0 || lane == 0);
      const unsigned long long act = __ballot(ok && first && !done);
      nact = __popcll(act);
      none = act == 0ull;
      if (ok && first && !done) reqs[__popcll(act & ((1ull << lane) - 1ull))] = hb0 + rb0 + (c / p - rb0);
      const int s = v ? (int)slot_of(a, t, hb0 + c / p, c % p) : -1;
      vm = __ballot(v);
      nval = __popcll(vm);
      const int s0 = __shfl(s, vm ? __ffsll((long long)vm) - 1 : 0);
      if (lane < nc) coln[lane] = v ? s : s0;
      if (v) {
        const int k = __popcll(vm & ((1ull << lane) - 1ull));
        coln[64 + k] = s;
        coln[128 + k] = (int)tok;
        coln[192 + k] = (int)src;
      }
    }
    if (lane == 0) {
      misc[0] = ok ? nval : -1;
      misc[1] = nact;
      misc[4] = none;
      misc[6] = (int)(uint32_t)vm;
      misc[7] = (int)(uint32_t)(vm >> 32);
    }
  }
  __syncthreads();
}

// Workers load their weights only once every controller has its start-up
// loads (candidates, first W2 rows): at launch the weight loads would
// otherwise queue ahead of them.  Returns false if the wait ran out.
__device__ __forceinline__ bool worker_wait_ready(const TreeArgs& a, int* misc) {
  if (threadIdx.x < 64) {
    const bool ok = wait_mbox(a.ready, a.B, a.ebase + 1, a.err, a.spin_limit);
    if (threadIdx.x == 0) misc[2] = ok;
  }
  __syncthreads();
  return misc[2] != 0;
}

// Once this block's rows of the step are stored, tell each active request's
// controller.
__device__ __forceinline__ void worker_ack(const TreeArgs& a, int w, const int* reqs, int nreq, uint32_t epoch) {
  const int tid = threadIdx.x;
  stores_done();
  __syncthreads();
  // wave 0 only (nreq <= 64); the ack drains while it polls the next step
  if (tid < nreq) st_dev_u32(a.mbox_c + (size_t)reqs[tid] * 256 + w, epoch);
}

template <typename W>
__device__ __forceinline__ void worker_main(const TreeArgs& a, unsigned char* lds) {
  const int w = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int kp = k_padded(a.ds);
  const int kc = a.kc, kcs = kc + STAGE_PAD;
  const int tile0 = w * a.tiles_per_worker;
  const int ntiles = max(0, min(a.tiles_per_worker, a.n_tiles - tile0));
  W* tiles_lds = reinterpret_cast<W*>(lds);
  W* stage = reinterpret_cast<W*>(lds + worker_stage_offset(a.tiles_per_worker, kp, (int)sizeof(W)));
  int* coln = reinterpret_cast<int*>(stage + (size_t)round_up(a.B * a.p, 16) * kcs);
  int* reqs = coln + TREE_MAX_COLS;  // requests with work this step
  int* misc = reqs + TREE_MAX_COLS;  // [0] columns (-1: failed), [1] requests

  if (!worker_wait_ready(a, misc)) return;
  // the block's Wc tiles stay in for the whole launch
  {
    const W* src = reinterpret_cast<const W*>(a.tiles) + (size_t)tile0 * 16 * kp;
    const size_t n16 = (size_t)ntiles * 16 * kp * sizeof(W) / 16;
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
    uint4* d4 = reinterpret_cast<uint4*>(tiles_lds);
    for (size_t i = tid; i < n16; i += NT) d4[i] = s4[i];
  }
  __syncthreads();

  for (int t = a.root ? 0 : 1;; ++t) {  // zero roots: step 0 needs no product (set up by the controllers)
    const uint32_t epoch = a.ebase + (uint32_t)t + 1u;
    worker_columns(a, w, t, 0, a.B, coln, reqs, misc);
    const int ncols = misc[0], nreq = misc[1];
    if (ncols <= 0) return;  // a wait ran out, or every request is finished
    const int ncb = (ncols + 15) / 16;
    if constexpr (sizeof(W) == 2) {
      const int pairs = ntiles * ncb;
      floatx4 acc[PPW][2];
#pragma unroll
      for (int i = 0; i < PPW; ++i) acc[i][0] = acc[i][1] = floatx4{0.f, 0.f, 0.f, 0.f};
      for (int k0 = 0; k0 < kp; k0 += kc) {
        if (k0 > 0) __syncthreads();  // the previous phase's operands are consumed
        worker_stage<W>(a, stage, coln, ncols, k0, kc, (int)slot_of(a, t, 0, 0));
        __syncthreads();
        worker_mfma_phase(reinterpret_cast<const uint16_t*>(tiles_lds), reinterpret_cast<const uint16_t*>(stage),
                          kp, k0 / 32, kc / 32, kcs, ncb, pairs, acc);
      }
      worker_epilogue_bf16(a, coln, ncols, tile0, ncb, pairs, acc);
    } else {
      worker_stage<W>(a, stage, coln, ncols, 0, kc, (int)slot_of(a, t, 0, 0));  // kc == kp for fp32
      __syncthreads();
      worker_compute_f32(a, reinterpret_cast<const float*>(tiles_lds), reinterpret_cast<const float*>(stage),
                         ncols, coln, tile0, ntiles, kp, kcs);
    }
    worker_ack(a, w, reqs, nreq, epoch);
  }
}


// ---- register-resident worker (bf16, d_s padded to RKB * 32 = 1024)
// Each wave owns TW tiles of [W_hh ; W1_S^T], held in registers as MFMA A
// operands for the whole launch.  A block owns CPB 16-column blocks of each
// step (block w: column blocks CPB (w % nb) + c, nb = ceil(ncbmax / CPB)) and
// its four waves four tile groups (wave v: tile group 4 (w / nb) + v, tiles
// TW g .. TW g + TW - 1).  Per step the block stages its columns' operands in
// LDS once (one batch of 8 CPB 16-byte loads per thread, whole 128-byte lines)
// and every wave runs RKB MFMAs per tile and column block on them, so an
// operand byte crosses the load path once per block rather than once per wave.
constexpr int RKB = 32;
constexpr int REGW_STAGE_OFFSET = round_up((2 * TREE_MAX_COLS + 64) * 4, 256);  // after coln, reqs, misc
constexpr int RSTRIDE = RKB * 32 + 8;  // staged column stride (elements): 16-byte skew per column

// Eight 16-byte loads from base + off[q] (byte offsets), issued back to back
// and completed together (one asm block, like load16_batch).
__device__ __forceinline__ void load8_batch(const void* base, const unsigned (&off)[8], u32x4 (&v)[8]) {
  asm volatile(
      "s_nop 4\n\t"  // as in load16_batch
      "global_load_dwordx4 %0, %8, %16\n\t"
      "global_load_dwordx4 %1, %9, %16\n\t"
      "global_load_dwordx4 %2, %10, %16\n\t"
      "global_load_dwordx4 %3, %11, %16\n\t"
      "global_load_dwordx4 %4, %12, %16\n\t"
      "global_load_dwordx4 %5, %13, %16\n\t"
      "global_load_dwordx4 %6, %14, %16\n\t"
      "global_load_dwordx4 %7, %15, %16\n\t"
      "s_waitcnt vmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "v"(off[4]), "v"(off[5]), "v"(off[6]), "v"(off[7]),
        "s"(uniform_ptr(base))
      : "memory");
}

// Eight 16-byte LDS reads at p + off[q] (immediate byte offsets below), issued
// back to back and completed together: the MFMA B operands of a group of k
// blocks.  CPB = 4: k blocks 0, 1 of column blocks 0..3 (a column block is 16
// staged columns = 33024 bytes; offsets stop at 65535, so blocks 2, 3 use a
// second base); CPB = 2: k blocks 0..3 of column blocks 0, 1; CPB = 1: k
// blocks 0..7.
template <int CPB>
__device__ __forceinline__ void lds_read8_b(const uint16_t* p, bf16x8 (&v)[8]) {
  const uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
  static_assert(16 * RSTRIDE * 2 == 33024, "column block stride");
  if constexpr (CPB == 4)
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:64\n\t"
        "ds_read_b128 %2, %8 offset:33024\n\t"
        "ds_read_b128 %3, %8 offset:33088\n\t"
        "ds_read_b128 %4, %9\n\t"
        "ds_read_b128 %5, %9 offset:64\n\t"
        "ds_read_b128 %6, %9 offset:33024\n\t"
        "ds_read_b128 %7, %9 offset:33088\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
        : "v"(a), "v"(a + 2u * 33024u)
        : "memory");
  else if constexpr (CPB == 2)
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:64\n\t"
        "ds_read_b128 %2, %8 offset:128\n\t"
        "ds_read_b128 %3, %8 offset:192\n\t"
        "ds_read_b128 %4, %8 offset:33024\n\t"
        "ds_read_b128 %5, %8 offset:33088\n\t"
        "ds_read_b128 %6, %8 offset:33152\n\t"
        "ds_read_b128 %7, %8 offset:33216\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
        : "v"(a)
        : "memory");
  else
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:64\n\t"
        "ds_read_b128 %2, %8 offset:128\n\t"
        "ds_read_b128 %3, %8 offset:192\n\t"
        "ds_read_b128 %4, %8 offset:256\n\t"
        "ds_read_b128 %5, %8 offset:320\n\t"
        "ds_read_b128 %6, %8 offset:384\n\t"
        "ds_read_b128 %7, %8 offset:448\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
        : "v"(a)
        : "memory");
}

// Advance the GRU states of nc columns (d_s = 1024, bf16 operand copies):
// S_y = GRU(S_x, E[tok]) with W_ih E[tok] + b_ih = G[tok] and gh_x published
// by the workers at the parent's step; column cc has slot cslot[cc], token
// ctok[cc] and parent slot csrc[cc] (from the controller's node entries).  The
// group's nq blocks share the float4 items: block q takes items q NT + i +
// k nq NT.
constexpr int WG = 3;  // advance items per thread in flight
__device__ __forceinline__ void worker_advance(const TreeArgs& a, const int* cslot, const int* ctok, const int* csrc,
                                               int nc, int q, int nq, floatx4 (&dv)[WG],
                                               float* (&dp)[WG]) {
  const int ds = a.ds, n4 = ds >> 2;
  const int items = nc * n4;
#pragma unroll
  for (int g = 0; g < WG; ++g) dp[g] = nullptr;
  for (int base = q * NT; base < items; base += nq * NT * WG) {
    // the states of the last batch are stored after the group's exchange
    // (later steps read them; the group needs only the operand copies now)
    const bool last = base + nq * NT * WG >= items;
    int tok[WG], src[WG], sl[WG], qv[WG];
#pragma unroll
    for (int g = 0; g < WG; ++g) {  // clamped: every lane reads a present column
      const int item = min(base + g * nq * NT + (int)threadIdx.x, items - 1);
      const int cc = item / n4;
      qv[g] = (item - cc * n4) * 4;
      sl[g] = cslot[cc];
      tok[g] = ctok[cc];
      src[g] = csrc[cc];
    }
    float4 ir[WG], iz[WG], in_[WG], hr[WG], hz[WG], hn[WG], sp[WG];
#pragma unroll
    for (int g = 0; g < WG; ++g) {
      const float* gi = a.G + (size_t)tok[g] * 3 * ds + qv[g];
      const float* gh = a.gh + (size_t)src[g] * gh_stride(ds) + qv[g];
      ir[g] = *reinterpret_cast<const float4*>(gi);
      iz[g] = *reinterpret_cast<const float4*>(gi + ds);
      in_[g] = *reinterpret_cast<const float4*>(gi + 2 * ds);
      hr[g] = *reinterpret_cast<const float4*>(gh);
      hz[g] = *reinterpret_cast<const float4*>(gh + ds);
      hn[g] = *reinterpret_cast<const float4*>(gh + 2 * ds);
      sp[g] = *reinterpret_cast<const float4*>(a.state + (size_t)src[g] * st_stride(ds) + qv[g]);
    }
    keep_batch();
#pragma unroll
    for (int g = 0; g < WG; ++g) {
      if (base + g * nq * NT + (int)threadIdx.x < items) {
        const float a0[4] = {ir[g].x, ir[g].y, ir[g].z, ir[g].w}, b0[4] = {hr[g].x, hr[g].y, hr[g].z, hr[g].w};
        const float a1[4] = {iz[g].x, iz[g].y, iz[g].z, iz[g].w}, b1[4] = {hz[g].x, hz[g].y, hz[g].z, hz[g].w};
        const float a2[4] = {in_[g].x, in_[g].y, in_[g].z, in_[g].w}, b2[4] = {hn[g].x, hn[g].y, hn[g].z, hn[g].w};
        const float s0[4] = {sp[g].x, sp[g].y, sp[g].z, sp[g].w};
        floatx4 o;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const float rg = sigm(a0[qq] + b0[qq]);
          const float zg = sigm(a1[qq] + b1[qq]);
          const float ng = tanh_(a2[qq] + rg * b2[qq]);
          o[qq] = (1.0f - zg) * ng + zg * s0[qq];
        }
        float* stp = a.state + (size_t)sl[g] * st_stride(ds) + qv[g];
        if (last) {  // deferred: dv, dp
          dv[g] = o;
          dp[g] = stp;
        } else {
          st_dev_f32x4(stp, o);
        }
        uint16_t* ap = reinterpret_cast<uint16_t*>(a.act) + (size_t)sl[g] * act_stride(ds) + qv[g];
        const uint32_t lo = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
        st_dev_u32x2(ap, lo, hi);  // device-wide even within one XCD: measured faster than into the L2
      }
    }
  }
}

template <int TW, int CPB>
__device__ __forceinline__ void worker_regs(const TreeArgs& a, unsigned char* lds) {
  const int w = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  int* coln = reinterpret_cast<int*>(lds);
  int* reqs = coln + TREE_MAX_COLS;
  int* misc = reqs + TREE_MAX_COLS;
  uint16_t* stage = reinterpret_cast<uint16_t*>(lds + REGW_STAGE_OFFSET);  // [16 CPB][RSTRIDE]
  const int kp = RKB * 32;
  const int as = act_stride(a.ds);
  const int nb = a.ncg;  // column groups
  const int col0 = (w % nb) * CPB * 16;  // first column of the block (a.cpg = 16 CPB)
  const int tile0 = ((w / nb) * 4 + wv) * TW;
  const int grp = w % nb, gq = w / nb, ngq = a.n_workers / nb;  // the blocks sharing these columns
  // the group's exchange: -1 undecided (device-wide until the first one has
  // shown whether every block of the group runs on this XCD), 0 device-wide,
  // 1 through the XCD's L2
  int xmode = a.xlocal ? -1 : 0;
  const uint32_t xcc = __builtin_amdgcn_s_getreg(0xF814);  // HW_REG_XCC_ID
  if (a.xlocal && tid == 0) st_dev_u32(a.xccw + w, xcc);  // drained before this block's first flag

  if (!worker_wait_ready(a, misc)) return;
  // this wave's A operands: tile rows (lane & 15), k 8 (lane >> 4) + 32 kb
  bf16x8 wa[TW][RKB];
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    const bool ok = tile0 + i < a.n_tiles;
    const bf16x8* src = reinterpret_cast<const bf16x8*>(reinterpret_cast<const uint16_t*>(a.tiles) +
                                                        (size_t)(ok ? tile0 + i : 0) * 16 * kp) + lane;
#pragma unroll
    for (int kb = 0; kb < RKB; ++kb) wa[i][kb] = src[kb * 64];
  }

  // With two halves the block serves the requests [0, bh) and then [bh, B) of
  // each step; a half whose requests are all finished is passed over.
  bool done[2] = {false, a.halves < 2};
  unsigned long long fin0 = 0ull, fin1 = 0ull;  // wave 0: columns whose request has finished, per half
  int t = a.root ? 0 : 1;  // zero roots: step 0 needs no product (set up by the controllers)
  for (int h = 0;; h = (h + 1) % a.halves, t += h == 0) {
    if (done[0] && done[1]) return;
    if (done[h]) continue;
    const uint32_t epoch = a.ebase + (uint32_t)t + 1u;
    // group flags: 2 epoch + h, increasing over (step, half) and across launches
    // whatever their number of halves
    const uint32_t gepoch = 2u * epoch + (uint32_t)h;
    unsigned long long fin = h ? fin1 : fin0;
    worker_columns_fixed(a, t, h ? a.bh : 0, h ? a.B - a.bh : a.bh, col0, 16 * CPB, fin, coln, reqs, misc);
    if (h)
      fin1 = fin;
    else
      fin0 = fin;
    const int nval = misc[0], nreq = misc[1];
    const unsigned long long vmask = (unsigned long long)(uint32_t)misc[6] | ((unsigned long long)(uint32_t)misc[7] << 32);
    if (nval < 0) return;  // a wait ran out
    if (misc[4]) {         // every request of these columns is finished
      done[h] = true;
      __syncthreads();     // misc is read by every thread before wave 0 writes it again
      continue;
    }
    if (nval > 0) {  // the same for every block of the group (it reads the same words)
      floatx4 sv[WG];  // this block's last advanced states, stored once the operands are staged
      float* sp[WG];
#pragma unroll
      for (int g = 0; g < WG; ++g) sp[g] = nullptr;
      if (a.wadv && t > 0) {
        // the group advances the states of its columns, then waits for all of it
        const bool loc = xmode == 1;
        worker_advance(a, coln + 64, coln + 128, coln + 192, nval, gq, ngq, sv, sp);
        stores_done();
        __syncthreads();
        if (tid == 0) {
          if (loc)
            st_l2_u32(a.gflag + grp * 64 + gq, gepoch);
          else
            st_dev_u32(a.gflag + grp * 64 + gq, gepoch);
        }
        if (tid < 64) {
          const bool ok = wait_mbox(a.gflag + grp * 64, ngq, gepoch, a.err, a.spin_limit);
          if (lane == 0) misc[2] = ok;
          if (xmode < 0) {
            // the first exchange: every block of the group wrote its XCC word
            // before its flag; one XCD for all of them means one L2
            const uint32_t x = lane < ngq ? ld_dev_u32(a.xccw + lane * nb + grp) : xcc;
            const bool same = __all(x == xcc);
            if (lane == 0) misc[3] = same;
          }
        }
        __syncthreads();
        if (xmode < 0) xmode = misc[3] ? 1 : 0;  // the same for every block of the group
        if (!misc[2]) return;
      }
      // stage the operands in two halves of k (16-byte pieces [0, 64) and
      // [64, 128) of each column's 128): the second half's loads are in flight
      // while the first half's products run.  Thread: piece tid & 63 of
      // columns (tid >> 6) + 4 q.
      const int slot0 = (int)slot_of(a, t, 0, 0);
      const int ph = tid & 63;
      const char* base = reinterpret_cast<const char*>(reinterpret_cast<const uint16_t*>(a.act) + (size_t)slot0 * as);
      constexpr int NL = 4 * CPB;  // loads per thread and half
      unsigned off[NL];
#pragma unroll
      for (int q = 0; q < NL; ++q)  // coln holds a present column's slot for every column
        off[q] = (unsigned)(((coln[(tid >> 6) + 4 * q] - slot0) * as + ph * 8) * 2);
      u32x4 v[NL];
#pragma unroll
      for (int q = 0; q < NL; ++q) v[q] = *reinterpret_cast<const u32x4*>(base + off[q]);
      keep_batch();
#pragma unroll
      for (int q = 0; q < NL; ++q) *reinterpret_cast<u32x4*>(stage + ((tid >> 6) + 4 * q) * RSTRIDE + ph * 8) = v[q];
#pragma unroll
      for (int q = 0; q < NL; ++q) v[q] = *reinterpret_cast<const u32x4*>(base + off[q] + 64 * 16);
      keep_batch();
      // the states (read by later steps' advances) drain during the products
      // and before the acknowledgement
#pragma unroll
      for (int g = 0; g < WG; ++g)
        if (sp[g]) st_dev_f32x4(sp[g], sv[g]);
      lds_barrier();  // the first half is staged (the second half's loads stay in flight)
      // B operands: column (lane & 15) of each column block, k 8 (lane >> 4) + 32 kb
      const uint16_t* sb = stage + (lane & 15) * RSTRIDE + 8 * (lane >> 4);
      // independent accumulation chains: two per (column block, tile) unless
      // the column blocks give enough
      constexpr int NACC = CPB >= 4 ? 1 : 2;
      floatx4 acc[CPB][TW][NACC];
#pragma unroll
      for (int c = 0; c < CPB; ++c)
#pragma unroll
        for (int i = 0; i < TW; ++i)
#pragma unroll
          for (int n = 0; n < NACC; ++n) acc[c][i][n] = floatx4{0.f, 0.f, 0.f, 0.f};
      // the products of k blocks [16 hk, 16 hk + 16): B operands four 16-byte
      // reads at a time (KG k blocks of the CPB column blocks), in two register
      // sets, the next group's reads issued before this group's products
      constexpr int KG = 4 / CPB, NG = RKB / KG / 2;
      auto products = [&](auto hkc) {
        constexpr int hk = decltype(hkc)::value;
        bf16x8 bv[2][4];  // [set][c KG + q]: column block c, k block 16 hk + g KG + q
        const uint16_t* sbh = sb + hk * 16 * 32;
#pragma unroll
        for (int q = 0; q < KG; ++q)
#pragma unroll
          for (int c = 0; c < CPB; ++c)
            bv[0][c * KG + q] = *reinterpret_cast<const bf16x8*>(sbh + c * 16 * RSTRIDE + q * 32);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          if (g + 1 < NG) {
#pragma unroll
            for (int q = 0; q < KG; ++q)
#pragma unroll
              for (int c = 0; c < CPB; ++c)
                bv[(g + 1) & 1][c * KG + q] =
                    *reinterpret_cast<const bf16x8*>(sbh + c * 16 * RSTRIDE + ((g + 1) * KG + q) * 32);
          }
#pragma unroll
          for (int q = 0; q < KG; ++q) {
            const int kb = g * KG + q;  // within the half
#pragma unroll
            for (int c = 0; c < CPB; ++c)
#pragma unroll
              for (int i = 0; i < TW; ++i)
                acc[c][i][kb % NACC] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    wa[i][16 * hk + kb], bv[g & 1][c * KG + q], acc[c][i][kb % NACC], 0, 0, 0);
          }
          // the schedule: this group's reads of the next set, then its products
          if (g == 0) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
          if (g + 1 < NG) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 4 * TW, 0);
        }
      };
      if (tile0 < a.n_tiles) products(std::integral_constant<int, 0>{});
#pragma unroll
      for (int q = 0; q < NL; ++q)
        *reinterpret_cast<u32x4*>(stage + ((tid >> 6) + 4 * q) * RSTRIDE + (64 + ph) * 8) = v[q];
      lds_barrier();  // the second half is staged
      if (tile0 < a.n_tiles) {
        products(std::integral_constant<int, 1>{});
        // lane holds column col, rows 4 (lane >> 4) + q of each tile
        const int ds3 = 3 * a.ds;
#pragma unroll
        for (int c = 0; c < CPB; ++c) {
          const int col = c * 16 + (lane & 15);
          if (!((vmask >> col) & 1ull)) continue;  // no node in this column
          const size_t slot = (size_t)coln[col];
#pragma unroll
          for (int i = 0; i < TW; ++i) {
            if (tile0 + i >= a.n_tiles) continue;
            floatx4 sum = acc[c][i][0];
            if constexpr (NACC == 2) sum = acc[c][i][0] + acc[c][i][1];
            const int row0 = (tile0 + i) * 16 + 4 * (lane >> 4);
            if (row0 + 3 < ds3 && (ds3 & 3) == 0) {
              floatx4 o = sum;
              if (a.b_hh) {
                o[0] += a.b_hh[row0];
                o[1] += a.b_hh[row0 + 1];
                o[2] += a.b_hh[row0 + 2];
                o[3] += a.b_hh[row0 + 3];
              }
              st_dev_f32x4(a.gh + slot * gh_stride(a.ds) + row0, o);
            } else if (row0 >= ds3 && row0 + 3 < ds3 + a.r && (ds3 & 3) == 0 && (a.r & 3) == 0) {
              // W1_S rows: u, the rows the controller waits for first
              st_dev_f32x4(a.u + slot * u_stride(a.r) + (row0 - ds3), sum);
            } else {
              for (int q = 0; q < 4; ++q) worker_store_out(a, slot, row0 + q, sum[q]);
            }
          }
        }
      }
    }
    worker_ack(a, w, reqs, nreq, epoch);  // its barrier also ends this step's stage reads
  }
}

// ---------------------------------------------------------------------------
// controller: one request's candidates, records, frontier and GRU states


enum {
  C_NF,      // frontier entries [fh, nf) of buffer fb
  C_FH,
  C_FB,
  C_NX,      // records
  C_E,       // nodes to expand in the next step
  C_OK,
  C_TAUSET,  // frontier entries with key_u < tau are known to be out
  C_STOP,
  C_NL,      // depth slots to load
  C_G,       // where the best entry of an over-long tie group came from
  C_NV,      // live new entries of a merge
  C_TIE,     // the merge's cut after N + 1 entries falls inside a group of equal key_u
  C_MISC
};

// A node record and a candidate of a depth, as kept in LDS.
struct Rec {
  uint64_t key;  // record key; record 0 is the root
  int par;       // parent record (-1 for the root)
  int slot;      // exchange slot holding the record's state (-1: not expanded)
};
struct Cand {
  int id;     // token id
  int rank;   // rank of the token id within its depth
  float val;  // base logit
  int pad;
};

// Fixed-size per-step state at the start of a controller's (compile-time
// offsets, so that accesses need no address registers).
struct CtlFixed {
  int misc[32];
  uint64_t tau;        // frontier entries with key_u < tau are out (when C_TAUSET)
  int cnt[QCAP];       // records ahead of each tested frontier entry
  int perm[QCAP];      // tested entries in the total order
  int acc[QCAP];       // tested entries taken
  int ex_rec[PMAX];    // records expanded in the step
  int ex_ws[PMAX];     // their depth slots
  int ex_dep[PMAX];    // their depths
  int ex_tok[PMAX];    // their tokens
  int ex_src[PMAX];    // exchange slots of their parents
  int wdep[PMAX];      // depth held by each W2 slot (-1: none)
  int wclaim[PMAX];    // slot used by a node of the next step
  int lslots[PMAX];    // slots to load before the next step
  float z[PMAX * 64];  // corrected, tempered candidate logits
};

// LDS arrays of a controller
struct CtlLds {
  CtlFixed* f;
  Cand* cand;           // [D*M]
  float* tailv;         // [D]
  Rec* rec;             // [xcap]
  int* rrank;           // [xcap] position in the total order (compaction and output)
  Rec* trec;            // [xcap] compaction staging
  uint64_t* front;      // [2][fcap] frontier keys, sorted descending, in buffer misc[C_FB]
  uint64_t* nc;         // [p*k] children keys of this step (0 = none)
  uint64_t* ncs;        // [p*k] live children sorted descending
  int* pn;              // [p*k] their insertion points in the frontier
  unsigned char* w2s;   // [nslots][M][r + pad] W2 rows of the candidates of each slot's depth
  float* ps;            // [nslots][r] P rows
  float* av;            // [p][r] SiLU(u + P); bf16 weights with r % 32 == 0: three bf16 pieces
                        // [3][p][av_stride(r)] (hi, mid, lo) whose sum is SiLU(u + P)
};

enum { L_FIXED, L_CAND, L_TAIL, L_REC, L_RRANK, L_TREC, L_FRONT, L_NC, L_NCS, L_PN, L_W2S, L_PS, L_AV, L_COUNT };

// elements per row of W2 candidate weights: r plus 16 bytes, so that the
// rows of consecutive candidates start in different banks
__host__ __device__ inline int w2s_stride(int r, int esz) { return r + 16 / esz; }
// bf16 elements per node row of the activation pieces (bf16 weights): r plus
// 16 bytes, so that the rows of the step's nodes start in different banks
__host__ __device__ inline int av_stride(int r) { return r + 8; }
// whether the expansions take dL on the matrix cores (bf16 weights)
__host__ __device__ inline bool dl_on_mfma(const TreeArgs& a, int esz) {
  return esz == 2 && (a.r & 31) == 0 && !a.marginal && !a.dlfma;
}

// byte offsets of the controller's arrays; returns the total
__host__ __device__ inline size_t ctl_offsets(const TreeArgs& a, int esz, size_t* off) {
  const size_t DM = (size_t)a.D * a.M, pk = (size_t)a.p * a.k, X = (size_t)a.xcap, P = (size_t)a.p;
  size_t sz[L_COUNT];
  sz[L_FIXED] = sizeof(CtlFixed);
  sz[L_CAND] = DM * sizeof(Cand);
  sz[L_TAIL] = (size_t)a.D * 4;
  sz[L_REC] = X * sizeof(Rec);
  sz[L_RRANK] = X * 4;
  sz[L_TREC] = X * sizeof(Rec);
  sz[L_FRONT] = (size_t)2 * a.fcap * 8;
  sz[L_NC] = (pk + 31) / 32 * 32 * 8;  // read in blocks of 32 keys
  sz[L_NCS] = pk * 8;
  sz[L_PN] = 0;
  sz[L_W2S] = (size_t)a.nslots * a.M * w2s_stride(a.r, esz) * esz;
  sz[L_PS] = (size_t)a.nslots * a.r * 4;
  sz[L_AV] = dl_on_mfma(a, esz) ? (size_t)3 * P * av_stride(a.r) * 2 : P * a.r * 4;
  size_t o = 0;
  for (int i = 0; i < L_COUNT; ++i) {
    off[i] = o;
    o += (sz[i] + 15) / 16 * 16;
  }
  return o;
}

__device__ __forceinline__ CtlLds ctl_carve(unsigned char* lds, const TreeArgs& a, int esz) {
  size_t off[L_COUNT];
  ctl_offsets(a, esz, off);
  CtlLds c;
  c.f = reinterpret_cast<CtlFixed*>(lds);
  c.cand = reinterpret_cast<Cand*>(lds + off[L_CAND]);
  c.tailv = reinterpret_cast<float*>(lds + off[L_TAIL]);
  c.rec = reinterpret_cast<Rec*>(lds + off[L_REC]);
  c.rrank = reinterpret_cast<int*>(lds + off[L_RRANK]);
  c.trec = reinterpret_cast<Rec*>(lds + off[L_TREC]);
  c.front = reinterpret_cast<uint64_t*>(lds + off[L_FRONT]);
  c.nc = reinterpret_cast<uint64_t*>(lds + off[L_NC]);
  c.ncs = reinterpret_cast<uint64_t*>(lds + off[L_NCS]);
  c.pn = reinterpret_cast<int*>(lds + off[L_PN]);
  c.w2s = lds + off[L_W2S];
  c.ps = reinterpret_cast<float*>(lds + off[L_PS]);
  c.av = reinterpret_cast<float*>(lds + off[L_AV]);
  return c;
}

// the frontier buffer currently in use
__device__ __forceinline__ uint64_t* cur_front(const TreeArgs& a, const CtlLds& c) {
  return c.front + (size_t)c.f->misc[C_FB] * a.fcap;
}

// Total order between two records of equal depth whose keys tie on
// (score, depth, token): the parents' order decides, recursively.
__device__ __forceinline__ bool rec_better(const CtlLds& c, int x, int y) {
  for (int it = 0; it < 32; ++it) {
    if (x == y || x < 0 || y < 0) return false;
    const uint64_t ux = key_u(c.rec[x].key), uy = key_u(c.rec[y].key);
    if (ux != uy) return ux > uy;
    x = c.rec[x].par;
    y = c.rec[y].par;
  }
  return false;
}

// frontier entry f precedes frontier entry g in the total order
__device__ __forceinline__ bool entry_better(const CtlLds& c, uint64_t f, uint64_t g) {
  const uint64_t uf = key_u(f), ug = key_u(g);
  if (uf != ug) return uf > ug;
  return rec_better(c, key_parent(f), key_parent(g));
}

// rrank[x] = number of records that precede record x
__device__ __forceinline__ void ctl_rank(const CtlLds& c, int nx) {
  for (int x = threadIdx.x; x < nx; x += NT) {
    const uint64_t xu = key_u(c.rec[x].key);
    const int xp = c.rec[x].par;
    int r = 0, ties = 0;
    for (int y = 0; y < nx; ++y) {
      const uint64_t yu = key_u(c.rec[y].key);
      r += yu > xu;
      ties += yu == xu;
    }
    if (ties > 1)  // equal keys: the parents' order decides
      for (int y = 0; y < nx; ++y)
        if (y != x && key_u(c.rec[y].key) == xu && rec_better(c, c.rec[y].par, xp)) ++r;
    c.rrank[x] = r;
  }
}

// Load the W2 candidate rows and the P row of each depth slot listed in
// lslots.  Issued while the workers run the step, so that scoring reads LDS.
template <typename W>
__device__ __forceinline__ void ctl_prefetch(const TreeArgs& a, const CtlLds& c, int b) {
  const int tid = threadIdx.x, M = a.M, r = a.r;
  const int nl = c.f->misc[C_NL];
  if (nl == 0 || a.marginal) return;  // marginal scores use neither W2 nor P
  const W* w2t = reinterpret_cast<const W*>(a.w2t);
  const int rs = w2s_stride(r, (int)sizeof(W));
  const int rows = nl * M;
  const int per = r * (int)sizeof(W) / 16;   // 16-byte pieces per row
  const int rsp = rs * (int)sizeof(W) / 16;  // pieces per row
  if ((r * (int)sizeof(W)) % 16 == 0 && per <= 256 && 256 % per == 0) {
    const int rpt = 256 / per;  // rows per pass
    const int pc = tid % per, r0 = tid / per;
    constexpr int U = 4;
    uint4* dst4 = (uint4*)c.w2s;
    for (int rb = 0; rb < rows; rb += U * rpt) {
      uint4 v[U];
      int dst[U];
#pragma unroll
      for (int q = 0; q < U; ++q) {  // clamped: every lane loads a valid piece
        const int row = min(rb + r0 + q * rpt, rows - 1);
        const int li = row / M, m = row - li * M;
        const int s = c.f->lslots[li];
        dst[q] = (s * M + m) * rsp + pc;
        v[q] = reinterpret_cast<const uint4*>(w2t + (size_t)c.cand[c.f->wdep[s] * M + m].id * r)[pc];
      }
#pragma unroll
      for (int q = 0; q < U; ++q) dst4[dst[q]] = v[q];  // unconditional
    }
  } else {
    W* w2s = (W*)c.w2s;
    for (int i = tid; i < rows * r; i += NT) {
      const int row = i / r, j = i % r;
      const int s = c.f->lslots[row / M], m = row % M;
      w2s[((size_t)s * M + m) * rs + j] = w2t[(size_t)c.cand[c.f->wdep[s] * M + m].id * r + j];
    }
  }
  for (int i = tid; i < nl * r; i += NT) {
    const int s = c.f->lslots[i / r], j = i % r;
    const size_t idx = ((size_t)b * a.D + c.f->wdep[s]) * r + j;
    float v = a.P[idx];
    for (int q = 1; q < a.p_parts; ++q) v += a.P[q * a.p_stride + idx];  // partials in order
    c.ps[(size_t)s * r + j] = v;
  }
}

// Score the children of the e nodes expanded at step t and write the keys of
// each node's k best into nc[j k .. j k + k) (0 where a child has no finite
// log-prob).
// One lane's operands of two k steps of the correction products: 16 bytes at
// w[c] and w[c] + 64 for four W2 rows, and 16 bytes at a + 0, 16, 128, 144 of
// the node's activations, read from LDS in one batch completed together.
__device__ __forceinline__ void lds_read_dl(const uint16_t* const (&w)[4], const float* av, u32x4 (&wv)[8],
                                            float4 (&xv)[4]) {
  uint32_t wa[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) wa[i] = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)w[i];
  const uint32_t aa = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)av;
  asm volatile(
      "ds_read_b128 %0, %12\n\t"
      "ds_read_b128 %1, %13\n\t"
      "ds_read_b128 %2, %14\n\t"
      "ds_read_b128 %3, %15\n\t"
      "ds_read_b128 %4, %12 offset:64\n\t"
      "ds_read_b128 %5, %13 offset:64\n\t"
      "ds_read_b128 %6, %14 offset:64\n\t"
      "ds_read_b128 %7, %15 offset:64\n\t"
      "ds_read_b128 %8, %16\n\t"
      "ds_read_b128 %9, %16 offset:16\n\t"
      "ds_read_b128 %10, %16 offset:128\n\t"
      "ds_read_b128 %11, %16 offset:144\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(wv[0]), "=&v"(wv[1]), "=&v"(wv[2]), "=&v"(wv[3]), "=&v"(wv[4]), "=&v"(wv[5]), "=&v"(wv[6]),
        "=&v"(wv[7]), "=&v"(xv[0]), "=&v"(xv[1]), "=&v"(xv[2]), "=&v"(xv[3])
      : "v"(wa[0]), "v"(wa[1]), "v"(wa[2]), "v"(wa[3]), "v"(aa)
      : "memory");
}

// The 32 keys (256 bytes) at p, read from LDS in one batch of sixteen 16-byte
// reads completed together.
__device__ __forceinline__ void lds_read_keys32(const uint64_t* p, u32x4 (&v)[16]) {
  const uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
  asm volatile(
      "ds_read_b128 %0, %16\n\t"
      "ds_read_b128 %1, %16 offset:16\n\t"
      "ds_read_b128 %2, %16 offset:32\n\t"
      "ds_read_b128 %3, %16 offset:48\n\t"
      "ds_read_b128 %4, %16 offset:64\n\t"
      "ds_read_b128 %5, %16 offset:80\n\t"
      "ds_read_b128 %6, %16 offset:96\n\t"
      "ds_read_b128 %7, %16 offset:112\n\t"
      "ds_read_b128 %8, %16 offset:128\n\t"
      "ds_read_b128 %9, %16 offset:144\n\t"
      "ds_read_b128 %10, %16 offset:160\n\t"
      "ds_read_b128 %11, %16 offset:176\n\t"
      "ds_read_b128 %12, %16 offset:192\n\t"
      "ds_read_b128 %13, %16 offset:208\n\t"
      "ds_read_b128 %14, %16 offset:224\n\t"
      "ds_read_b128 %15, %16 offset:240\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7]),
        "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]), "=&v"(v[12]), "=&v"(v[13]), "=&v"(v[14]),
        "=&v"(v[15])
      : "v"(a)
      : "memory");
}

// a = SiLU(u + P_d) of the step's e nodes as three bf16 pieces per element
// (hi, mid, lo: each the nearest bf16 of what the previous ones leave, so their
// sum is a to fp32 precision and each product with bf16 W2 is exact in fp32),
// pairs of elements: item i is node i / (r / 2), elements 2 (i % (r / 2)) + 0,
// 1; a thread takes items tid, tid + NT, ..., eight of them a batch, and
// writes each piece of a pair as one word.
__device__ __forceinline__ void ctl_silu_pieces(const TreeArgs& a, const CtlLds& c, int b, int t, int e) {
  const int tid = threadIdx.x, r = a.r;
  const int us = u_stride(r);
  const float* ub = a.u + slot_of(a, t, b, 0) * us;  // the e slots are consecutive
  uint32_t* avw = reinterpret_cast<uint32_t*>(c.av);
  const int r2 = r >> 1, tot = e * r2, dj = NT / r2, dq = NT - dj * r2;
  const size_t piece = (size_t)a.p * av_stride(r) / 2;  // words
  int j = tid / r2, q = tid - j * r2;
  for (int b0 = 0; b0 < tot; b0 += 8 * NT) {
    // the batch's u loads, its depth-slot reads and its P reads each go out
    // together: no load is conditional (an item past the end re-reads the
    // last node's pair, which is in bounds, and is not stored), so none
    // waits behind a branch
    float2 uv[8], pv[8];
    int jj[8], qq[8], ws[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      jj[x] = min(j, e - 1);
      qq[x] = q;
      uv[x] = *reinterpret_cast<const float2*>(ub + (size_t)jj[x] * us + 2 * q);
      q += dq;
      j += dj;
      if (q >= r2) {
        q -= r2;
        ++j;
      }
    }
#pragma unroll
    for (int x = 0; x < 8; ++x) ws[x] = c.f->ex_ws[jj[x]];
#pragma unroll
    for (int x = 0; x < 8; ++x) pv[x] = *reinterpret_cast<const float2*>(c.ps + ws[x] * r + 2 * qq[x]);
    keep_batch();
#pragma unroll
    for (int x = 0; x < 8; ++x)
      if (b0 + x * NT + tid < tot) {
        const float x0 = uv[x].x + pv[x].x, x1 = uv[x].y + pv[x].y;
        const float v0 = x0 * sigm(x0), v1 = x1 * sigm(x1);
        const uint16_t h0 = f32_to_bf16(v0), h1 = f32_to_bf16(v1);
        const float s0 = v0 - bf16_to_f32(h0), s1 = v1 - bf16_to_f32(h1);
        const uint16_t m0 = f32_to_bf16(s0), m1 = f32_to_bf16(s1);
        const uint16_t l0 = f32_to_bf16(s0 - bf16_to_f32(m0)), l1 = f32_to_bf16(s1 - bf16_to_f32(m1));
        uint32_t* o = avw + (size_t)jj[x] * (av_stride(r) / 2) + qq[x];
        o[0] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        o[piece] = (uint32_t)m0 | ((uint32_t)m1 << 16);
        o[2 * piece] = (uint32_t)l0 | ((uint32_t)l1 << 16);
      }
  }
}

// a = SiLU(u + P_d) in fp32 (the vector-FMA correction), element i of every
// node by thread i mod NT.
__device__ __forceinline__ void ctl_silu_f32(const TreeArgs& a, const CtlLds& c, int b, int t, int e) {
  const int tid = threadIdx.x, r = a.r;
  const int us = u_stride(r);
  const float* ub = a.u + slot_of(a, t, b, 0) * us;
  for (int i = tid; i < r; i += NT) {
    float uv[PMAX];
#pragma unroll
    for (int j = 0; j < PMAX; ++j) uv[j] = ub[(size_t)min(j, e - 1) * us + i];  // in bounds, no branch
    keep_batch();
#pragma unroll
    for (int j = 0; j < PMAX; ++j)
      if (j < e) {
        const float x = uv[j] + c.ps[c.f->ex_ws[j] * r + i];
        c.av[j * r + i] = x * sigm(x);
      }
  }
}

// Within each half-wave (32 lanes): how many other lanes hold a greater value
// than this lane.  The lanes of the same row of 16 come from DPP rotations
// (row_ror), those of the other row from one swizzle (lane ^ 16) and its
// rotations: no LDS traffic.
template <int R>
__device__ __forceinline__ uint32_t row_ror_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x120 + R, 0xF, 0xF, false);
}
__device__ __forceinline__ int half_rank32(uint32_t v) {
  int gt = 0;
  auto acc = [&](uint32_t o) { gt += o > v; };
#define DT_ROW_RORS(x)                                                                                          \
  acc(row_ror_u32<1>(x)), acc(row_ror_u32<2>(x)), acc(row_ror_u32<3>(x)), acc(row_ror_u32<4>(x)),              \
      acc(row_ror_u32<5>(x)), acc(row_ror_u32<6>(x)), acc(row_ror_u32<7>(x)), acc(row_ror_u32<8>(x)),          \
      acc(row_ror_u32<9>(x)), acc(row_ror_u32<10>(x)), acc(row_ror_u32<11>(x)), acc(row_ror_u32<12>(x)),       \
      acc(row_ror_u32<13>(x)), acc(row_ror_u32<14>(x)), acc(row_ror_u32<15>(x))
  DT_ROW_RORS(v);
  const uint32_t x = (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);  // lane ^ 16 within 32 lanes
  acc(x);
  DT_ROW_RORS(x);
#undef DT_ROW_RORS
  return gt;
}
// The same over the whole wave (64 lanes): the other row of this half by a
// swizzle, the other half by one permute and its swizzle, each rotated.
__device__ __forceinline__ int wave_rank32(uint32_t v) {
  int gt = 0;
  auto acc = [&](uint32_t o) { gt += o > v; };
#define DT_ROW_RORS(x)                                                                                          \
  acc(row_ror_u32<1>(x)), acc(row_ror_u32<2>(x)), acc(row_ror_u32<3>(x)), acc(row_ror_u32<4>(x)),              \
      acc(row_ror_u32<5>(x)), acc(row_ror_u32<6>(x)), acc(row_ror_u32<7>(x)), acc(row_ror_u32<8>(x)),          \
      acc(row_ror_u32<9>(x)), acc(row_ror_u32<10>(x)), acc(row_ror_u32<11>(x)), acc(row_ror_u32<12>(x)),       \
      acc(row_ror_u32<13>(x)), acc(row_ror_u32<14>(x)), acc(row_ror_u32<15>(x))
  DT_ROW_RORS(v);
  const uint32_t x1 = (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);  // lane ^ 16
  acc(x1);
  DT_ROW_RORS(x1);
  const int lane = threadIdx.x & 63;
  const uint32_t x2 = (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, (int)v);  // lane ^ 32
  acc(x2);
  DT_ROW_RORS(x2);
  const uint32_t x3 = (uint32_t)__builtin_amdgcn_ds_swizzle((int)x2, 0x401F);  // lane ^ 48
  acc(x3);
  DT_ROW_RORS(x3);
#undef DT_ROW_RORS
  return gt;
}

// OR over each half-wave.
__device__ __forceinline__ uint32_t half_or32(uint32_t v) {
  v |= row_ror_u32<1>(v);
  v |= row_ror_u32<2>(v);
  v |= row_ror_u32<4>(v);
  v |= row_ror_u32<8>(v);
  return v | (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
}

template <typename W>
__device__ __forceinline__ void ctl_expand(const TreeArgs& a, const CtlLds& c, int b, int t, int e) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int M = a.M, r = a.r, k = a.k;
  // dL on the matrix cores (bf16 weights; not needed for marginal scores)
  const bool mf = dl_on_mfma(a, (int)sizeof(W));
  // a_j = SiLU(u_j + P_{d_j}); the u loads of all nodes are issued first
  if (!a.marginal) {
    if (mf)
      ctl_silu_pieces(a, c, b, t, e);
    else
      ctl_silu_f32(a, c, b, t, e);
  }
  __syncthreads();
  // dL_{j,m} = W2[:, cand_m] . a_j.
  if (a.marginal) {
    // the factorised scores: base logits alone
    for (int i = tid; i < e * M; i += NT) {
      const int j = i / M, m = i - j * M;
      c.f->z[j * 64 + m] = c.cand[c.f->ex_dep[j] * M + m].val / a.T + 0.0f;
    }
  } else if (mf) {
    // On the matrix cores: for each depth slot s in use, the slot's W2
    // candidate rows [M x r] (A, 16 candidates a block) times the step's
    // activations [r x 16] (B, column n node n, the columns of nodes of other
    // slots zero), v_mfma_f32_16x16x32_bf16 over r in 32-k steps, one
    // accumulator per piece.  Wave w takes the candidate block w % nrb and
    // every (4 / nrb)-th slot in use from w / nrb on; a node's column thus
    // sums the products of its own slot only and is written by one wave.
    const int nrb = (M + 15) >> 4;  // 1..4
    const int nkp = (NT / WAVE) / nrb;
    const int rb = wv % nrb, part = wv / nrb;
    const int n = lane & 15, kq = 8 * (lane >> 4);
    const int wsn = n < e ? c.f->ex_ws[n] : -1;
    uint32_t smask = 0;
    for (int s = 0; s < a.nslots; ++s)
      if (__ballot(wsn == s)) smask |= 1u << s;
    const bool mine = wsn >= 0 && __popc(smask & ((1u << wsn) - 1u)) % nkp == part;
    if (part < nkp) {  // nrb = 3 leaves wave 3 idle
      // Operand rows past M (A) or of nodes past e (B) are read as they
      // stand: they only reach output rows and columns that are not kept.
      const uint16_t* avh = reinterpret_cast<const uint16_t*>(c.av);
      const int piece = a.p * av_stride(r);
      const int rs = w2s_stride(r, 2);
      const uint16_t* arow = avh + (size_t)n * av_stride(r) + kq;
      const uint16_t* w2b = reinterpret_cast<const uint16_t*>(c.w2s) + (size_t)min(rb * 16 + n, M - 1) * rs + kq;
      float res[4] = {0.f, 0.f, 0.f, 0.f};
      int si = 0;
      for (uint32_t mm = smask; mm; mm &= mm - 1u, ++si) {
        if (si % nkp != part) continue;
        const int s = __ffs(mm) - 1;
        const uint16_t* wrow = w2b + (size_t)s * M * rs;
        floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0, acc2 = acc0;
        // two operand sets, X for the even and Y for the odd 32-k steps: a
        // set is read again while the other set's products run
        bf16x8 xw, x0, x1, x2, yw, y0, y1, y2;
        auto ld = [&](int k0, bf16x8& w, bf16x8& o0, bf16x8& o1, bf16x8& o2) {
          w = *reinterpret_cast<const bf16x8*>(wrow + k0);
          o0 = *reinterpret_cast<const bf16x8*>(arow + k0);
          o1 = *reinterpret_cast<const bf16x8*>(arow + piece + k0);
          o2 = *reinterpret_cast<const bf16x8*>(arow + 2 * piece + k0);
        };
        ld(0, xw, x0, x1, x2);
        if (r > 32) ld(32, yw, y0, y1, y2);
        for (int k0 = 0; k0 < r; k0 += 64) {
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xw, x0, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xw, x1, acc1, 0, 0, 0);
          acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xw, x2, acc2, 0, 0, 0);
          if (k0 + 64 < r) ld(k0 + 64, xw, x0, x1, x2);
          if (k0 + 32 < r) {
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(yw, y0, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(yw, y1, acc1, 0, 0, 0);
            acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(yw, y2, acc2, 0, 0, 0);
            if (k0 + 96 < r) ld(k0 + 96, yw, y0, y1, y2);
          }
        }
        if (wsn == s) {
#pragma unroll
          for (int q = 0; q < 4; ++q) res[q] = acc0[q] + (acc1[q] + acc2[q]);
        }
      }
      // lane: node n, candidates rb 16 + 4 (lane >> 4) + q
      if (mine) {
        const int dep = c.f->ex_dep[n];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int mc = rb * 16 + 4 * (lane >> 4) + q;
          if (mc < M) c.f->z[n * 64 + mc] = (c.cand[dep * M + mc].val + res[q]) / a.T + 0.0f;
        }
      }
    }
  } else if (sizeof(W) == 2 && (M & 3) == 0 && (r & 63) == 0) {
    // bf16 rows: a quad of threads per (node,
    // 4 candidates), thread h of the quad taking elements 32 i + 8 h .. + 7 of
    // all four rows (each a_j read serves four rows; a quad reads 64 consecutive
    // bytes of a row), combined in a fixed order.
    const int G4 = M >> 2;
    const int rs = w2s_stride(r, 2);
    for (int base = 0; base < e * G4 * 4; base += NT) {
      const int idx = base + tid, h = idx & 3, rest = idx >> 2;
      const int j = rest / G4, g = rest - j * G4;
      const bool valid = j < e;
      const int jr = valid ? j : 0;
      const float* avj = c.av + jr * r + 8 * h;
      const uint16_t* w0 = reinterpret_cast<const uint16_t*>(c.w2s) + (size_t)(c.f->ex_ws[jr] * M + 4 * g) * rs + 8 * h;
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      for (int q0 = 0; q0 < r; q0 += 64) {  // two k steps of 32 per LDS batch
        const uint16_t* const wr[4] = {w0 + q0, w0 + rs + q0, w0 + 2 * rs + q0, w0 + 3 * rs + q0};
        u32x4 wv[8];
        float4 xv[4];
        lds_read_dl(wr, avj + q0, wv, xv);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const float xa[8] = {xv[2 * st].x, xv[2 * st].y, xv[2 * st].z, xv[2 * st].w,
                               xv[2 * st + 1].x, xv[2 * st + 1].y, xv[2 * st + 1].z, xv[2 * st + 1].w};
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            const uint32_t wd[4] = {wv[4 * st + cc].x, wv[4 * st + cc].y, wv[4 * st + cc].z, wv[4 * st + cc].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              acc[cc] = fmaf(__uint_as_float(wd[q] << 16), xa[2 * q], acc[cc]);
              acc[cc] = fmaf(__uint_as_float(wd[q] & 0xFFFF0000u), xa[2 * q + 1], acc[cc]);
            }
          }
        }
      }
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        acc[cc] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc[cc]), 0xB1, 0xF, 0xF, false));
        acc[cc] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc[cc]), 0x4E, 0xF, 0xF, false));
      }
      const float dl = h == 0 ? acc[0] : h == 1 ? acc[1] : h == 2 ? acc[2] : acc[3];
      const int m = 4 * g + h;
      if (valid) c.f->z[j * 64 + m] = (c.cand[c.f->ex_dep[j] * M + m].val + dl) / a.T + 0.0f;
    }
  } else {
    // candidates padded to a power of two so that the index splits are shifts
    int lm = 0;
    while ((1 << lm) < M) ++lm;
    const int nd = e << lm;
    int lt = 0;  // log2 of the threads per (node, candidate)
    while ((2 << lt) * nd <= NT && lt < 6) ++lt;
    const int tpc = 1 << lt;
    const int len = (r + tpc - 1) >> lt;
    const int rs = w2s_stride(r, (int)sizeof(W));
    constexpr int VE = 16 / sizeof(W);  // elements per 16-byte piece
    const bool vec = (len % VE) == 0 && (r * (int)sizeof(W)) % 16 == 0 && (len << lt) == r;
    for (int base = 0; base < nd * tpc; base += NT) {
      const int idx = base + tid;
      const int pr = idx >> lt, part = idx & (tpc - 1);
      const int j = pr >> lm, m = pr & ((1 << lm) - 1);
      const bool valid = pr < nd && m < M;
      float dl = 0.f;
      if (valid) {
        const W* wrow = (const W*)c.w2s + (c.f->ex_ws[j] * M + m) * rs;
        const float* avj = c.av + j * r;
        const int j0 = part * len, j1 = min(r, j0 + len);
        if (vec) {
          for (int q0 = j0; q0 < j1; q0 += VE) {
            const uint4 wv4 = *(const uint4*)(wrow + q0);
            const W* we = reinterpret_cast<const W*>(&wv4);
#pragma unroll
            for (int q = 0; q < VE; q += 4) {
              const float4 a4 = *(const float4*)(avj + q0 + q);
              dl = fmaf(w_to_f32<W>(we[q]), a4.x, dl);
              dl = fmaf(w_to_f32<W>(we[q + 1]), a4.y, dl);
              dl = fmaf(w_to_f32<W>(we[q + 2]), a4.z, dl);
              dl = fmaf(w_to_f32<W>(we[q + 3]), a4.w, dl);
            }
          }
        } else {
          for (int q = j0; q < j1; ++q) dl = fmaf(w_to_f32<W>(wrow[q]), avj[q], dl);
        }
      }
      for (int s = 1; s < tpc; s <<= 1) dl += __shfl_xor(dl, s);
      if (valid && part == 0) c.f->z[j * 64 + m] = (c.cand[c.f->ex_dep[j] * M + m].val + dl) / a.T + 0.0f;
    }
  }
  __syncthreads();
  // one half-wave (M <= 32) or wave per node, one candidate per lane:
  // log-softmax over the candidates (plus the base tail under fullv), rank by
  // (z desc, token asc), keep the k best with a finite log-prob.  -inf
  // log-probs rank after every finite one.
  if (M <= 32) {
    // half-wave h of wave w takes nodes 2 w + h and 2 w + h + 8 (e <= 16),
    // both at once so that their latency chains overlap
    const int half = lane >> 5, l32 = lane & 31;
    const int hw = 2 * wv + half;
    if (2 * wv < e) {
      constexpr float L2E = 1.4426950408889634f, LN2 = 0.6931471805599453f;
      int jr[2], y[2], dy[2];
      bool node[2], has[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = hw + 8 * u;
        node[u] = j < e;
        jr[u] = node[u] ? j : 2 * wv;  // a valid node of this wave for the reads
        has[u] = node[u] && l32 < M;
        y[u] = c.f->ex_rec[jr[u]];
        dy[u] = c.f->ex_dep[jr[u]];
      }
      float yscore[2], zv[2], tl[2];
      int idv[2], crk[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        yscore[u] = key_score(c.rec[y[u]].key);
        zv[u] = has[u] ? c.f->z[jr[u] * 64 + l32] : -INFINITY;
        const Cand cd = c.cand[dy[u] * M + (has[u] ? l32 : 0)];
        idv[u] = has[u] ? cd.id : 0x7FFFFFFF;
        crk[u] = cd.rank;
        tl[u] = a.fullv ? c.tailv[dy[u]] : -INFINITY;
      }
      float lz[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float mx = fmaxf(half_max_dpp(zv[u]), tl[u]);
        const bool live = mx > -INFINITY;
        float se = half_sum_dpp(has[u] && live ? __builtin_amdgcn_exp2f((zv[u] - mx) * L2E) : 0.f);
        if (tl[u] > -INFINITY) se += __builtin_amdgcn_exp2f((tl[u] - mx) * L2E);
        lz[u] = live ? mx + __builtin_amdgcn_logf(se) * LN2 : -INFINITY;
      }
      // ranks among each node's candidates by (value desc, token asc): by the
      // value keys alone (lanes past M hold 0, below every value) unless a
      // half-wave holds equal values, then by the full composites, rotated
      // one lane at a time through the permute network
      int rank[2];
      bool tie = false;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        rank[u] = half_rank32(has[u] ? f32_key(zv[u]) : 0u);
        // distinct values take the ranks 0 .. M - 1 once each; equal values
        // share a rank and leave others unused
        const uint32_t seen = half_or32(has[u] ? 1u << rank[u] : 0u);
        tie |= node[u] && __popc(seen) != M;
      }
      if (__ballot(tie)) {
        uint64_t me[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          me[u] = has[u] ? cand_pack(f32_key(zv[u]), (uint32_t)idv[u]) : 0ull;
          rank[u] = 0;
        }
#pragma unroll
        for (int q = 1; q < 32; ++q) {
          const int src = (((l32 + q) & 31) | (half << 5)) << 2;  // byte address of the source lane
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const uint32_t oh = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(me[u] >> 32));
            const uint32_t ol = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)me[u]);
            rank[u] += (((uint64_t)oh << 32) | ol) > me[u];  // lanes past M hold 0, which precedes nothing
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float lp = zv[u] - lz[u];
        const bool ok = has[u] && isfinite(lp);
        if (has[u] && rank[u] < k)
          c.nc[(hw + 8 * u) * k + rank[u]] = ok ? make_key(yscore[u] + lp, dy[u] + 1, crk[u], y[u], l32) : 0ull;
      }
    }
  } else {
    // one wave per node (M <= 64): nodes wv + 8 i and wv + 8 i + 4 at once, so
    // that their latency chains overlap
    for (int j0 = wv; j0 < e; j0 += 8) {
      int jr[2], y[2], dy[2];
      bool node[2], has[2];
      float yscore[2], zv[2], tl[2];
      int idv[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = j0 + 4 * u;
        node[u] = j < e;
        jr[u] = node[u] ? j : j0;  // a valid node of this wave for the reads
        has[u] = node[u] && lane < M;
        y[u] = c.f->ex_rec[jr[u]];
        dy[u] = c.f->ex_dep[jr[u]];
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        yscore[u] = key_score(c.rec[y[u]].key);
        zv[u] = has[u] ? c.f->z[jr[u] * 64 + lane] : -INFINITY;
        idv[u] = has[u] ? c.cand[dy[u] * M + lane].id : 0x7FFFFFFF;
        tl[u] = a.fullv ? c.tailv[dy[u]] : -INFINITY;
      }
      float lz[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float mx = fmaxf(wave_max_dpp(zv[u]), tl[u]);
        lz[u] = -INFINITY;
        if (mx > -INFINITY) {
          float se = wave_sum_dpp(has[u] ? expf(zv[u] - mx) : 0.f);
          if (tl[u] > -INFINITY) se += expf(tl[u] - mx);
          lz[u] = mx + logf(se);
        }
      }
      // rank by (value desc, token asc): on the value keys alone (absent
      // lanes 0, below every value) unless the ranks show equal values
      // (distinct ones take the ranks 0 .. M - 1 once each, summing to
      // M (M - 1) / 2; equal ones share a rank), then by the composite
      // (value key, complemented id)
      int rank[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) rank[u] = wave_rank32(has[u] ? f32_key(zv[u]) : 0u);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (node[u] && wave_sum_dpp(has[u] ? (float)rank[u] : 0.f) != (float)(M * (M - 1) / 2)) {
          const uint64_t me = has[u] ? cand_pack(f32_key(zv[u]), (uint32_t)idv[u]) : 0ull;
          const uint32_t mlo = (uint32_t)me, mhi = (uint32_t)(me >> 32);
          int rk = 0;
          for (int q = 0; q < M; ++q) {
            const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)mhi, q) << 32) |
                               (uint32_t)__builtin_amdgcn_readlane((int)mlo, q);
            rk += o > me;
          }
          rank[u] = rk;
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float lp = zv[u] - lz[u];
        const bool ok = has[u] && isfinite(lp);
        if (has[u] && rank[u] < k)
          c.nc[jr[u] * k + rank[u]] =
              ok ? make_key(yscore[u] + lp, dy[u] + 1, c.cand[dy[u] * M + lane].rank, y[u], lane) : 0ull;
      }
    }
  }
  // zero the new keys past e k up to a multiple of 32 (the merge reads blocks of 32)
  for (int i = e * k + tid; i < (e * k + 31) / 32 * 32; i += NT) c.nc[i] = 0ull;
  if (tid == 0) c.f->misc[C_NV] = 0;
  __syncthreads();
}

// Merge this step's children into the sorted frontier (written to the other
// buffer), dropping new entries that are known to be out (key_u < tau); the
// old entries are all live, since whatever raises tau also cuts the frontier
// there.  Keys are unique.  First the live new entries are ranked among
// themselves (S threads per entry), then each thread writes its share of the
// merged order, found by a binary search on its first output's diagonal
// (merge path).  Only the first N + 1 merged entries are kept, unless the
// next one has the same key_u as entry N: an entry with N + 1 entries of
// greater key_u ahead of it could only be taken after all of them, with N + 1
// records ahead, so it never is.  Also resets the pop state of the step.
__device__ __forceinline__ void ctl_merge(const TreeArgs& a, const CtlLds& c, int nnew) {
  const int tid = threadIdx.x;
  const int fh = c.f->misc[C_FH], nf = c.f->misc[C_NF], fb = c.f->misc[C_FB];
  const bool tauset = c.f->misc[C_TAUSET] != 0;
  const uint64_t tau = c.f->tau;
  const uint64_t* F = c.front + (size_t)fb * a.fcap + fh;
  uint64_t* O = c.front + (size_t)(1 - fb) * a.fcap;
  const int na = nf - fh;
  {
    int np = 1;
    while (np < nnew) np <<= 1;
    const int ls = NT / np >= 4 ? 2 : NT / np >= 2 ? 1 : 0;  // log2 of the threads per entry
    const int S = 1 << ls;
    for (int base = 0; base < (nnew << ls); base += NT) {
      const int idx = base + tid, i = idx >> ls, s = idx & (S - 1);
      const uint64_t key = i < nnew ? c.nc[i] : 0ull;
      // new entries ahead (any key above a live one is live): thread s of the
      // group counts a contiguous share, 32 keys per LDS batch
      const int CH = ((nnew + S - 1) / S + 31) & ~31;
      const int qe = min(nnew, (s + 1) * CH);
      int rn = 0;
      for (int q0 = s * CH; q0 < qe; q0 += 32) {
        u32x4 kv[16];
        lds_read_keys32(c.nc + q0, kv);
#pragma unroll
        for (int i2 = 0; i2 < 16; ++i2) {
          const uint64_t k0 = ((uint64_t)kv[i2].y << 32) | kv[i2].x, k1 = ((uint64_t)kv[i2].w << 32) | kv[i2].z;
          rn += k0 > key;  // keys past nnew are 0, which precedes nothing
          rn += k1 > key;
        }
      }
      if (ls >= 1) rn += __builtin_amdgcn_update_dpp(0, rn, 0xB1, 0xF, 0xF, false);  // lane ^ 1
      if (ls >= 2) rn += __builtin_amdgcn_update_dpp(0, rn, 0x4E, 0xF, 0xF, false);  // lane ^ 2
      const bool live = i < nnew && s == 0 && key != 0 && (!tauset || key_u(key) >= tau);
      if (live) c.ncs[rn] = key;
      const unsigned long long bl = __ballot(live);
      if ((tid & 63) == 0 && bl) atomicAdd(&c.f->misc[C_NV], __popcll(bl));
    }
  }
  if (tid == 0) c.f->misc[C_TIE] = 0;
  __syncthreads();
  const int nv = c.f->misc[C_NV];
  const uint64_t* Nw = c.ncs;
  // (k - 1) xcap + 1 bounds the frontier; the guard only keeps intact
  const int full = min(na + nv, a.fcap);
  const int cut = min(full, a.N + 1);
  int total = cut;
  for (int pass = 0; pass < 2; ++pass) {
    // outputs [o0, o1): the first N + 1, then (rarely) the rest
    const int o0 = pass ? cut : 0, o1 = pass ? full : cut;
    const int L = (o1 - o0 + NT - 1) / NT;
    const int d0 = min(o0 + tid * L, o1), d1 = min(d0 + L, o1);
    if (d0 < d1) {
      // i old and d0 - i new entries precede output d0
      int lo = max(0, d0 - nv), hi = min(d0, na);
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (F[mid] > Nw[d0 - mid - 1]) lo = mid + 1;
        else hi = mid;
      }
      int i = lo, j = d0 - lo;
      uint64_t fi = i < na ? F[i] : 0ull, nj = j < nv ? Nw[j] : 0ull;
      uint64_t last = 0ull;
      for (int d = d0; d < d1; ++d) {
        const bool old = j >= nv || (i < na && fi > nj);
        last = old ? fi : nj;
        O[d] = last;
        if (old) {
          ++i;
          fi = i < na ? F[i] : 0ull;
        } else {
          ++j;
          nj = j < nv ? Nw[j] : 0ull;
        }
      }
      if (!pass && d1 == cut && cut < full) {
        // the entry after the cut: does it share entry N's key_u?
        const uint64_t nxt = (j >= nv || (i < na && fi > nj)) ? fi : nj;
        if (key_u(nxt) == key_u(last)) c.f->misc[C_TIE] = 1;
      }
    }
    if (pass) break;
    __syncthreads();
    if (!c.f->misc[C_TIE]) break;
    total = full;
  }
  if (tid == 0) {
    if (na + nv > a.fcap) atomicOr(a.err, 4);
    c.f->misc[C_FB] = 1 - fb;
    c.f->misc[C_FH] = 0;
    c.f->misc[C_NF] = total;
    c.f->misc[C_E] = 0;
    c.f->misc[C_STOP] = 0;
    c.f->misc[C_NL] = 0;
    for (int s = 0; s < a.nslots; ++s) c.f->wclaim[s] = 0;
  }
  __syncthreads();
}

// Keep the N + 1 first records (renumbered by rank, so X becomes sorted), remap
// parents, and cut the frontier after the entries that can still get in:
// every entry ranked below record N in key_u is out, and no other entry has a
// dropped parent.
__device__ __forceinline__ void ctl_compact(const TreeArgs& a, const CtlLds& c) {
  const int tid = threadIdx.x, N = a.N;
  const int nx = c.f->misc[C_NX];
  ctl_rank(c, nx);
  __syncthreads();
  for (int x = tid; x < nx; x += NT) {
    const int rk = c.rrank[x];
    if (rk <= N) {
      c.trec[rk].key = c.rec[x].key;
      c.trec[rk].par = c.rec[x].par >= 0 ? c.rrank[c.rec[x].par] : -1;
      c.trec[rk].slot = c.rec[x].slot;
    }
    if (rk == N) {
      const uint64_t u = key_u(c.rec[x].key);
      if (!c.f->misc[C_TAUSET] || u > c.f->tau) c.f->tau = u;
    }
  }
  __syncthreads();
  const int fh = c.f->misc[C_FH], nf = c.f->misc[C_NF], fb = c.f->misc[C_FB];
  const uint64_t* F = c.front + (size_t)fb * a.fcap + fh;
  uint64_t* O = c.front + (size_t)(1 - fb) * a.fcap;
  const uint64_t tauN = c.f->tau;
  int na = nf - fh;
  {
    int lo = 0, hi = na;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (key_u(F[mid]) >= tauN) lo = mid + 1;
      else hi = mid;
    }
    na = lo;
  }
  for (int i = tid; i < na; i += NT) O[i] = key_with_parent(F[i], c.rrank[key_parent(F[i])]);
  const int nk = min(nx, N + 1);
  for (int x = tid; x < nk; x += NT) {
    c.rec[x].key = c.trec[x].key;
    c.rec[x].par = c.trec[x].par;
    c.rec[x].slot = c.trec[x].slot;
  }
  __syncthreads();
  if (tid == 0) {
    c.f->misc[C_NX] = nk;
    c.f->misc[C_FB] = 1 - fb;
    c.f->misc[C_FH] = 0;
    c.f->misc[C_NF] = na;
    c.f->misc[C_TAUSET] = 1;
  }
  __syncthreads();
}

// An over-long group of equal key_u at the head: rotate its best entry (in the
// total order) to the head; it is then tested alone.  Thread 0 only.
__device__ __forceinline__ void ctl_batch_group(const CtlLds& c, uint64_t* F, int fh, int nf, uint64_t u) {
  int g = fh;
  for (int i = fh + 1; i < nf && key_u(F[i]) == u; ++i)
    if (entry_better(c, F[i], F[g])) g = i;
  const uint64_t best = F[g];
  for (int i = g; i > fh; --i) F[i] = F[i - 1];
  F[fh] = best;
  c.f->misc[C_G] = g;  // where to put it back if it is neither taken nor out
}

// Take frontier entries for the next step (t + 1): up to p nodes to expand,
// plus the depth-D leaves met on the way.  Returns the number to expand.
__device__ __forceinline__ int ctl_pop(const TreeArgs& a, const CtlLds& c, int b, int t) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int N = a.N, D = a.D, M = a.M;
  for (int round = 0; round < 4 * XMAX; ++round) {
    if (c.f->misc[C_NX] + a.qmax > a.xcap) {
      if (c.f->misc[C_E] > 0) break;  // expand what was taken; compact next step
      ctl_compact(a, c);
    }
    // the batch: the first Q entries, not ending inside a group of equal key_u
    // (every thread computes the same Q from the same words)
    const int fh = c.f->misc[C_FH], nf = c.f->misc[C_NF], nx = c.f->misc[C_NX];
    uint64_t* F = cur_front(a, c) + fh;
    int Q = min(min(nf - fh, a.qmax), a.xcap - nx);
    bool group = false;
    if (Q > 0 && Q < nf - fh && key_u(F[Q - 1]) == key_u(F[Q])) {
      const uint64_t u = key_u(F[Q - 1]);
      while (Q > 0 && key_u(F[Q - 1]) == u) --Q;
      if (Q == 0) {
        group = true;
        Q = 1;
        if (tid == 0) ctl_batch_group(c, F - fh, fh, nf, u);
        __syncthreads();
      }
    }
    if (Q <= 0) break;
    // cnt[j] = records that precede entry j of the batch.  Entry j is out when
    // cnt[j] + j >= N + 1; cnt[j] <= nx, so while nx + Q - 1 < N + 1 no entry
    // of the batch can be out and the counts are not needed.
    const bool counts = nx + Q - 1 >= N + 1;
    if (counts) {
      int Qp = 1;
      while (Qp < Q) Qp <<= 1;
      const int S = min(64, 256 / Qp);
      const int j = tid / S, s = tid % S;
      int cv = 0, tie = 0;
      uint64_t fu = 0;
      if (j < Q) {
        fu = key_u(F[j]);
        // eight records per batch, their LDS reads issued together (clamped
        // indices: every read is of a valid record; past nx nothing counts)
        for (int y0 = s; y0 < nx; y0 += 8 * S) {
          uint64_t yk[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) yk[u] = c.rec[min(y0 + u * S, nx - 1)].key;
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const uint64_t yu = key_u(yk[u]);
            const bool in = y0 + u * S < nx;
            cv += in && yu > fu;
            tie |= in && yu == fu;
          }
        }
        if (tie) {  // equal keys: the parents' order decides
          const int fp = key_parent(F[j]);
          for (int y = s; y < nx; y += S)
            if (key_u(c.rec[y].key) == fu && rec_better(c, c.rec[y].par, fp)) ++cv;
        }
      }
      for (int m = S >> 1; m >= 1; m >>= 1) cv += __shfl_xor(cv, m);
      if (j < Q && s == 0) c.f->cnt[j] = cv;
      __syncthreads();
    }
    // wave 0, lane jj = the jj-th batch entry in the total order: the taken
    // entries are the longest prefix that is not out and fits the step
    if (tid < 64) {
      const bool has = lane < Q;
      const uint64_t fl = has ? F[lane] : 0ull;
      const uint64_t fprev = ((uint64_t)dpp_wave_shr1((uint32_t)(fl >> 32)) << 32) | dpp_wave_shr1((uint32_t)fl);
      const bool anytie = __ballot(has && lane > 0 && key_u(fl) == key_u(fprev)) != 0;
      if (!anytie) {
        // key order is the total order: everything on registers and ballots
        const int e0 = c.f->misc[C_E];
        const int nl0 = c.f->misc[C_NL];
        const int cl = has && counts ? c.f->cnt[lane] : 0;
        int wdl = lane < a.nslots ? c.f->wdep[lane] : -1;  // lane s: slot s
        int wcl = lane < a.nslots ? c.f->wclaim[lane] : 0;
        const uint64_t key = fl;
        const int d = key_depth(key);
        const bool expd = has && d < D;
        const bool out = has && cl + lane >= N + 1;
        // depths held by a slot, and by a claimed slot
        uint32_t hm = 0, cm = 0;
        int nclaimed = 0;
        for (int s = 0; s < a.nslots; ++s) {
          const int ws = __builtin_amdgcn_readlane(wdl, s), wc = __builtin_amdgcn_readlane(wcl, s);
          if (ws >= 0) {
            hm |= 1u << ws;
            if (wc) cm |= 1u << ws;
          }
          nclaimed += wc;
        }
        const bool held = (hm >> d) & 1u, held_claimed = (cm >> d) & 1u;
        const unsigned long long bexp = __ballot(expd);
        // depths expanded by this lane and the earlier ones (inclusive), and by
        // the earlier ones only
        const uint32_t dmi = wave_or_scan_incl(expd ? 1u << d : 0u);
        const uint32_t dmx = dpp_wave_shr1(dmi);
        const bool first = !((dmx >> d) & 1u);
        const unsigned long long le = lane == 63 ? ~0ull : ((2ull << lane) - 1ull);  // lanes <= lane
        const unsigned long long bnew = __ballot(expd && first && !held);
        const unsigned long long bhu = __ballot(expd && first && held && !held_claimed);
        const int need = nclaimed + __popcll(bhu & le) + __popcll(bnew & le);
        const bool fits = has && !out && (!expd || (e0 + __popcll(bexp & le) <= a.p && need <= a.nslots));
        const unsigned long long bfail = __ballot(has && !fits);
        const int A = bfail ? __ffsll((long long)bfail) - 1 : Q;
        const bool isout = A < Q && ((__ballot(out) >> A) & 1ull);
        const unsigned long long lowA = A >= 64 ? ~0ull : ((1ull << A) - 1ull);
        // claim the slots of the taken depths, then give new depths free slots
        const uint32_t dm = A > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)dmi, A - 1) : 0u;
        if (lane < a.nslots && wdl >= 0 && ((dm >> wdl) & 1u)) wcl = 1;
        unsigned long long fm = __ballot(lane < a.nslots && !wcl);
        int nl = nl0;
        for (unsigned long long bn = bnew & lowA; bn; bn &= bn - 1) {
          const int dq = __builtin_amdgcn_readlane(d, __ffsll((long long)bn) - 1);
          const int sl = __ffsll((long long)fm) - 1;  // need <= nslots: a free slot exists
          fm &= fm - 1;
          if (lane == sl) {
            wdl = dq;
            wcl = 1;
          }
          if (lane == 0) c.f->lslots[nl] = sl;
          ++nl;
        }
        if (lane < a.nslots) {
          c.f->wdep[lane] = wdl;
          c.f->wclaim[lane] = wcl;
        }
        // the taken lanes write their records and the tables of the next step
        int ws = 0;  // the slot holding this lane's depth
        for (int s = 0; s < a.nslots; ++s)
          if (__builtin_amdgcn_readlane(wdl, s) == d) ws = s;
        if (has && lane < A) {
          const int x = nx + lane;
          const int par = key_parent(key);
          c.rec[x].key = key;
          c.rec[x].par = par;
          if (expd) {
            const int ei = e0 + __popcll(bexp & le) - 1;
            c.f->ex_rec[ei] = x;
            c.f->ex_ws[ei] = ws;
            c.f->ex_dep[ei] = d;
            c.f->ex_tok[ei] = c.cand[(d - 1) * M + key_m(key)].id;
            c.f->ex_src[ei] = c.rec[par].slot;
            c.rec[x].slot = (int)slot_of(a, t + 1, b, ei);
          } else {
            c.rec[x].slot = -1;
          }
        }
        if (lane == 0) {
          if (group && A == 0 && !isout) {  // put the group's best entry back in key order
            const int g = c.f->misc[C_G] - fh;
            const uint64_t best = F[0];
            for (int i = 0; i < g; ++i) F[i] = F[i + 1];
            F[g] = best;
          }
          if (isout) {
            const uint64_t u = key_u(F[A]);
            if (!c.f->misc[C_TAUSET] || u > c.f->tau) c.f->tau = u;
            c.f->misc[C_TAUSET] = 1;
            c.f->misc[C_NF] = c.f->misc[C_FH] = 0;  // the rest of the frontier is out
          } else {
            c.f->misc[C_FH] = fh + A;
          }
          const int e1 = e0 + __popcll(bexp & lowA);
          c.f->misc[C_E] = e1;
          c.f->misc[C_NX] = nx + A;
          c.f->misc[C_NL] = nl;
          c.f->misc[C_STOP] = isout || A < Q || e1 == a.p;
        }
      } else {
      if (has) {
        c.f->perm[lane] = lane;
        c.f->acc[lane] = 0;
      }
      if (anytie && lane == 0)
        for (int i = 1; i < Q; ++i) {  // insertion sort in the total order
          const int v = c.f->perm[i];
          int jj = i;
          while (jj > 0 && entry_better(c, F[v], F[c.f->perm[jj - 1]])) {
            c.f->perm[jj] = c.f->perm[jj - 1];
            --jj;
          }
          c.f->perm[jj] = v;
        }
      const int j = has ? c.f->perm[lane] : 0;
      const uint64_t key = has ? F[j] : 0ull;
      const int d = key_depth(key);
      const bool expd = has && d < D;
      const bool out = has && counts && c.f->cnt[j] + lane >= N + 1;
      const int e0 = c.f->misc[C_E];
      // depth slots: a depth is new if no slot holds it and no earlier lane has it
      int held = 0, held_claimed = 0, nclaimed = 0;
      for (int s = 0; s < a.nslots; ++s) {
        const int ws = c.f->wdep[s], wc = c.f->wclaim[s];
        held |= ws == d;
        held_claimed |= ws == d && wc;
        nclaimed += wc;
      }
      const unsigned long long bexp = __ballot(expd);
      bool first = true;  // no earlier lane expands a node of the same depth
      for (int q = 0; q < Q; ++q) {
        const int dq = __builtin_amdgcn_readlane(d, q);
        first &= !(q < lane && ((bexp >> q) & 1ull) && dq == d);
      }
      const unsigned long long le = lane == 63 ? ~0ull : ((2ull << lane) - 1ull);  // lanes <= lane
      const unsigned long long bnew = __ballot(expd && first && !held);
      const unsigned long long bhu = __ballot(expd && first && held && !held_claimed);
      const int need = nclaimed + __popcll(bhu & le) + __popcll(bnew & le);
      const bool fits = has && !out && (!expd || (e0 + __popcll(bexp & le) <= a.p && need <= a.nslots));
      const unsigned long long bfail = __ballot(has && !fits);
      const int A = bfail ? __ffsll((long long)bfail) - 1 : Q;
      const bool isout = A < Q && ((__ballot(out) >> A) & 1ull);
      const unsigned long long lowA = A >= 64 ? ~0ull : ((1ull << A) - 1ull);
      // lane 0 claims the slots of the taken depths, then gives new depths free slots
      if (lane == 0) {
        uint32_t dm = 0;  // depths of the taken nodes to expand
        for (unsigned long long mm = bexp & lowA; mm; mm &= mm - 1)
          dm |= 1u << __builtin_amdgcn_readlane(d, __ffsll((long long)mm) - 1);
        for (int s = 0; s < a.nslots; ++s)
          if (c.f->wdep[s] >= 0 && ((dm >> c.f->wdep[s]) & 1u)) c.f->wclaim[s] = 1;
        for (unsigned long long mm = bnew & lowA; mm; mm &= mm - 1) {
          const int dq = __builtin_amdgcn_readlane(d, __ffsll((long long)mm) - 1);
          for (int s = 0; s < a.nslots; ++s)
            if (!c.f->wclaim[s]) {
              c.f->wclaim[s] = 1;
              c.f->wdep[s] = dq;
              c.f->lslots[c.f->misc[C_NL]++] = s;
              break;
            }
        }
      }
      // the taken lanes write their records and the tables of the next step
      if (has && lane < A) {
        const int x = nx + lane;
        const int par = key_parent(key);
        c.rec[x].key = key;
        c.rec[x].par = par;
        c.f->acc[j] = 1;
        if (expd) {
          const int ei = e0 + __popcll(bexp & le) - 1;
          int ws = 0;
          for (int s = 0; s < a.nslots; ++s)
            if (c.f->wdep[s] == d) ws = s;
          c.f->ex_rec[ei] = x;
          c.f->ex_ws[ei] = ws;
          c.f->ex_dep[ei] = d;
          c.f->ex_tok[ei] = c.cand[(d - 1) * M + key_m(key)].id;
          c.f->ex_src[ei] = c.rec[par].slot;
          c.rec[x].slot = (int)slot_of(a, t + 1, b, ei);
        } else {
          c.rec[x].slot = -1;
        }
      }
      if (lane == 0) {
        if (group && A == 0 && !isout) {  // put the group's best entry back in key order
          const int g = c.f->misc[C_G] - fh;
          const uint64_t best = F[0];
          for (int i = 0; i < g; ++i) F[i] = F[i + 1];
          F[g] = best;
        }
        if (isout) {
          const uint64_t u = key_u(F[c.f->perm[A]]);
          if (!c.f->misc[C_TAUSET] || u > c.f->tau) c.f->tau = u;
          c.f->misc[C_TAUSET] = 1;
          c.f->misc[C_NF] = c.f->misc[C_FH] = 0;  // the rest of the frontier is out
        } else {
          if (anytie) {  // the taken entries may not be a key-order prefix
            int wpos = Q;
            for (int jj = Q - 1; jj >= 0; --jj)
              if (!c.f->acc[jj]) F[--wpos] = F[jj];
          }
          c.f->misc[C_FH] = fh + A;
        }
        const int e1 = e0 + __popcll(bexp & lowA);
        c.f->misc[C_E] = e1;
        c.f->misc[C_NX] = nx + A;
        c.f->misc[C_STOP] = isout || A < Q || e1 == a.p;
      }
      }
    }
    __syncthreads();
    if (c.f->misc[C_STOP]) break;
  }
  return c.f->misc[C_E];
}

// Advance the GRU state of each node taken for step t1 from its parent's:
// S_y = GRU(S_x, E[tok]) with W_ih E[tok] + b_ih = G[tok] and
// gh_x = W_hh S~_x + b_hh published by the workers at the parent's step.
// The e nodes' float4 items are spread over the block; the loads of GA items
// are issued before their stores.
template <typename W>
__device__ __forceinline__ void ctl_advance(const TreeArgs& a, const CtlLds& c, int b, int t1, int e) {
  const int ds = a.ds;
  const size_t sl0 = slot_of(a, t1, b, 0);  // the e slots are consecutive
  if ((ds & 3) == 0) {
    const int n4 = ds >> 2;
    const int total = e * n4;
    for (int base = 0; base < total; base += GA * (int)NT) {
      float4 ir[GA], iz[GA], in[GA], hr[GA], hz[GA], hn[GA], sp[GA];
      int jv[GA], qv[GA];
#pragma unroll
      for (int g = 0; g < GA; ++g) {  // clamped: every lane loads valid addresses
        const int item = min(base + g * (int)NT + (int)threadIdx.x, total - 1);
        const int j = item / n4;
        const int q = (item - j * n4) * 4;
        jv[g] = j;
        qv[g] = q;
        int xs = c.f->ex_src[j];
        if (xs < 0) {  // every parent was expanded; the guard keeps addresses valid
          atomicOr(a.err, 8);
          xs = 0;
        }
        const float* gi = a.G + (size_t)c.f->ex_tok[j] * 3 * ds + q;
        const float* gh = a.gh + (size_t)xs * gh_stride(ds) + q;
        ir[g] = *reinterpret_cast<const float4*>(gi);
        iz[g] = *reinterpret_cast<const float4*>(gi + ds);
        in[g] = *reinterpret_cast<const float4*>(gi + 2 * ds);
        hr[g] = *reinterpret_cast<const float4*>(gh);
        hz[g] = *reinterpret_cast<const float4*>(gh + ds);
        hn[g] = *reinterpret_cast<const float4*>(gh + 2 * ds);
        sp[g] = *reinterpret_cast<const float4*>(a.state + (size_t)xs * st_stride(ds) + q);
      }
      keep_batch();
#pragma unroll
      for (int g = 0; g < GA; ++g) {
        if (base + g * (int)NT + (int)threadIdx.x < total) {
          const float a0[4] = {ir[g].x, ir[g].y, ir[g].z, ir[g].w}, b0[4] = {hr[g].x, hr[g].y, hr[g].z, hr[g].w};
          const float a1[4] = {iz[g].x, iz[g].y, iz[g].z, iz[g].w}, b1[4] = {hz[g].x, hz[g].y, hz[g].z, hz[g].w};
          const float a2[4] = {in[g].x, in[g].y, in[g].z, in[g].w}, b2[4] = {hn[g].x, hn[g].y, hn[g].z, hn[g].w};
          const float s0[4] = {sp[g].x, sp[g].y, sp[g].z, sp[g].w};
          floatx4 o;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const float rg = sigm(a0[qq] + b0[qq]);
            const float zg = sigm(a1[qq] + b1[qq]);
            const float ng = tanh_(a2[qq] + rg * b2[qq]);
            o[qq] = (1.0f - zg) * ng + zg * s0[qq];
          }
          const size_t sl = sl0 + jv[g];
          st_dev_f32x4(a.state + sl * st_stride(ds) + qv[g], o);
          st_dev_act4<W>(reinterpret_cast<W*>(a.act) + sl * act_stride(ds) + qv[g], o, a.act_bf16);
        }
      }
    }
  } else {
    for (int j = 0; j < e; ++j) {
      const int xs = max(c.f->ex_src[j], 0);
      const float* gi = a.G + (size_t)c.f->ex_tok[j] * 3 * ds;
      const float* gh = a.gh + (size_t)xs * gh_stride(ds);
      const float* sx = a.state + (size_t)xs * st_stride(ds);
      float* sy = a.state + (sl0 + j) * st_stride(ds);
      W* ay = reinterpret_cast<W*>(a.act) + (sl0 + j) * act_stride(ds);
      for (int q = threadIdx.x; q < ds; q += NT) {
        const float rg = sigm(gi[q] + gh[q]);
        const float zg = sigm(gi[ds + q] + gh[ds + q]);
        const float ng = tanh_(gi[2 * ds + q] + rg * gh[2 * ds + q]);
        const float s = (1.0f - zg) * ng + zg * sx[q];
        st_dev_f32(sy + q, s);
        st_dev_act<W>(ay + q, s, a.act_bf16);
      }
    }
  }
  const int kpad = k_padded(ds) - ds;  // zero k padding of the operand copies
  for (int i = threadIdx.x; i < e * kpad; i += NT)
    st_dev_act<W>(reinterpret_cast<W*>(a.act) + (sl0 + i / kpad) * act_stride(ds) + ds + i % kpad, 0.f, 0);
}

// outputs in the total order (node i = the record ranked i), padded past n
__device__ __forceinline__ void ctl_output(const TreeArgs& a, const CtlLds& c, int b, bool failed) {
  const int tid = threadIdx.x, N = a.N, M = a.M;
  const int nx = c.f->misc[C_NX];
  ctl_rank(c, nx);
  __syncthreads();
  const int n = min(N, nx - 1);
  const size_t o = (size_t)b * (N + 1);
  for (int x = tid; x < nx; x += NT) {
    const int rk = c.rrank[x];
    if (rk > N) continue;
    const uint64_t key = c.rec[x].key;
    const bool root = x == 0;
    const int d = key_depth(key);
    a.tokens[o + rk] = root ? -1 : c.cand[(d - 1) * M + key_m(key)].id;
    a.parents[o + rk] = root ? -1 : c.rrank[c.rec[x].par];
    a.depths[o + rk] = d;
    a.scores[o + rk] = key_score(key);
  }
  for (int i = n + 1 + tid; i <= N; i += NT) {
    a.tokens[o + i] = -1;
    a.parents[o + i] = -1;
    a.depths[o + i] = -1;
    a.scores[o + i] = -INFINITY;
  }
  if (tid == 0) a.n_nodes[b] = failed ? -1 : n;
}

// Register workers: the acknowledgement words request b waits for, those of
// the blocks of tile groups [q0, q1] in the column groups its p columns fall
// in (block (q0 + i / ng) ncg + g0 + i % ng for word i); two per lane
// (at most 128 words), lanes past the set re-reading its last word.
__device__ __forceinline__ void ack_ptrs(const TreeArgs& a, const uint32_t* box, int b, int q0, int q1,
                                         const uint32_t* (&p)[2]) {
  const int lane = threadIdx.x & 63;
  const int hb0 = (a.halves == 2 && b >= a.bh) ? a.bh : 0;
  const int c0 = (b - hb0) * a.p;
  const int g0 = c0 / a.cpg, ng = (c0 + a.p - 1) / a.cpg - g0 + 1;
  const int n = (q1 - q0 + 1) * ng;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = min(lane + 64 * q, n - 1);
    p[q] = box + (size_t)(q0 + i / ng) * a.ncg + g0 + i % ng;
  }
}

// Register workers: wave 0 writes the node entries of request b's p columns at
// step ts: the e nodes' (token, parent slot), NINFO_NONE for the columns past
// them, or NINFO_DONE for every column once the request has finished.
__device__ __forceinline__ void ctl_entries(const TreeArgs& a, const CtlLds& c, int b, int ts, int e, bool done) {
  const int tid = threadIdx.x;
  if (tid < a.p) {
    uint32_t tok = done ? NINFO_DONE : NINFO_NONE, src = 0;
    if (!done && tid < e) {
      int xs = c.f->ex_src[tid];
      if (xs < 0) {  // every parent was expanded; the guard keeps addresses valid
        atomicOr(a.err, 8);
        xs = 0;
      }
      tok = (uint32_t)c.f->ex_tok[tid];
      src = (uint32_t)xs;
    }
    st_dev_u64(a.ninfo + (size_t)ts * TREE_MAX_COLS + (size_t)b * a.p + tid,
               ninfo_entry(a.ebase + (uint32_t)ts + 1u, tok, src));
  }
}

template <typename W>
__device__ __forceinline__ void controller_main(const TreeArgs& a, unsigned char* lds) {
  const int b = blockIdx.x - a.n_workers;
  const int tid = threadIdx.x;
  const int D = a.D, M = a.M;
  const CtlLds c = ctl_carve(lds, a, (int)sizeof(W));

  for (int i = tid; i < D * M; i += NT) {
    c.cand[i].id = a.cand_ids[(size_t)b * D * M + i];
    c.cand[i].val = a.cand_vals[(size_t)b * D * M + i];
    c.cand[i].rank = a.tokrank[(size_t)b * D * M + i];
  }
  for (int i = tid; i < D; i += NT) c.tailv[i] = a.tail[(size_t)b * D + i];
  if (tid == 0) {
    // the root: score 0, depth 0; it precedes every other node
    c.rec[0].key = make_key(0.f, 0, 0, 0, 0);
    c.rec[0].par = -1;
    c.rec[0].slot = (int)slot_of(a, 0, b, 0);
    c.f->misc[C_NX] = 1;
    c.f->misc[C_NF] = c.f->misc[C_FH] = c.f->misc[C_FB] = 0;
    c.f->misc[C_TAUSET] = 0;
    c.f->tau = 0;
    for (int s = 0; s < a.nslots; ++s) c.f->wdep[s] = -1;
    c.f->wdep[0] = 0;  // the root's children are at depth 1: row 0 of the tables
    c.f->lslots[0] = 0;
    c.f->misc[C_NL] = 1;
    c.f->ex_rec[0] = 0;
    c.f->ex_ws[0] = 0;
    c.f->ex_dep[0] = 0;
    c.f->misc[C_E] = 1;
  }
  // root state and its GEMM operand copy (marginal scores need no states)
  if (!a.marginal) {
    const int ds = a.ds;
    const size_t sl = slot_of(a, 0, b, 0);
    float* s0 = a.state + sl * st_stride(ds);
    W* a0 = reinterpret_cast<W*>(a.act) + sl * act_stride(ds);
    for (int j = tid; j < ds; j += NT) {
      const float v = a.root ? a.root[(size_t)b * ds + j] : 0.f;
      st_dev_f32(s0 + j, v);
      st_dev_act<W>(a0 + j, v, a.act_bf16);
    }
    for (int j = ds + tid; j < k_padded(ds); j += NT) st_dev_act<W>(a0 + j, 0.f, 0);
    if (!a.root) {
      // a zero root state: W_hh S + b_hh = b_hh and W1_S^T S = 0, without the workers
      float* g0 = a.gh + sl * gh_stride(ds);
      for (int j = tid; j < 3 * ds; j += NT) st_dev_f32(g0 + j, a.b_hh ? a.b_hh[j] : 0.f);
      float* u0 = a.u + sl * u_stride(a.r);
      for (int j = tid; j < a.r; j += NT) st_dev_f32(u0 + j, 0.f);
    }
  }
  stores_done();
  __syncthreads();
  const bool regws = a.regw != 0 && a.n_workers > 0;  // register workers: node entries, not mailbox words
  if (a.root) {  // step 0: the workers take the root's products (its state is set above)
    if (regws) {
      if (tid < a.p) st_dev_u64(a.ninfo + (size_t)b * a.p + tid, ninfo_entry(a.ebase + 1, tid ? NINFO_NONE : 0u, 0u));
    } else if (tid < MBOX_REPL) {
      st_dev_u32(a.mbox_w + (size_t)tid * 32 + b, mbox_word(a.ebase + 1, 1));
    }
  }
  stores_done();
  ctl_prefetch<W>(a, c, b);
  __syncthreads();
  if (tid == 0) st_dev_u32(a.ready + b, a.ebase + 1);  // start-up loads done: workers may load weights

  bool failed = false;
  int steps = 0, expanded = 0;
  for (int t = 0;; ++t) {
    const int e = c.f->misc[C_E];
    steps = t + 1;
    expanded += e;
    const uint32_t epoch = a.ebase + (uint32_t)t + 1u;
    // the workers' acknowledgements of step t.  Register workers: only the
    // blocks of this request's column groups; scoring needs u alone, so here
    // only the blocks holding the W1_S^T tiles are waited for, and the others'
    // (gh rows, which the next step's advance reads) are checked before the
    // next publication, their words read while the step is scored.  Other
    // workers: all of them, here.
    const bool ack_wait = !(t == 0 && !a.root);  // zero roots: step 0's products are set up above
    const bool fixed = a.regw != 0 && a.n_workers > 0;
    const uint32_t* box = a.mbox_c + (size_t)b * 256;
    if (tid < 64) {
      bool ok = true;
      if (ack_wait && fixed) {
        const uint32_t* p[2];
        ack_ptrs(a, box, b, a.ugq0, a.ugq1, p);
        ok = wait_ptrs<2>(p, epoch, a.err, a.spin_limit, nullptr);
      } else if (ack_wait) {
        ok = wait_mbox(box, a.n_workers, epoch, a.err, a.spin_limit);
      }
      if (tid == 0) c.f->misc[C_OK] = ok;
    }
    __syncthreads();
    if (!c.f->misc[C_OK]) {
      failed = true;
      break;
    }
    ctl_expand<W>(a, c, b, t, e);
    const bool ack_rest = ack_wait && fixed;
    const uint32_t* pr[2];
    uint32_t acks[2];  // wave 0: the rest of the words, read while merge and pop run
    if (ack_rest && tid < 64) {
      ack_ptrs(a, box, b, 0, a.n_workers / a.ncg - 1, pr);
#pragma unroll
      for (int q = 0; q < 2; ++q) acks[q] = __hip_atomic_load(pr[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    ctl_merge(a, c, e * a.k);
    const int e2 = ctl_pop(a, c, b, t);
    if (ack_rest && e2 > 0) {
      if (tid < 64) {
        const bool ok = __all(acks[0] >= epoch && acks[1] >= epoch) ||
                        wait_ptrs<2>(pr, epoch, a.err, a.spin_limit, nullptr);
        if (tid == 0 && !ok) c.f->misc[C_OK] = 0;
      }
      __syncthreads();
      if (!c.f->misc[C_OK]) {
        failed = true;
        break;
      }
    }
    if (e2 == 0) break;
    if (t + 1 > a.N) {  // cannot happen: every step takes one of the N best nodes
      if (tid == 0) atomicOr(a.err, 2);
      failed = true;
      break;
    }
    if (a.marginal) {
      // marginal scores: no states to advance (and no workers)
    } else if (a.wadv) {
      // the workers advance the states: the node entries (token and parent
      // slot, carrying the step's epoch) are all they need
      if (tid < 64) ctl_entries(a, c, b, t + 1, e2, false);
    } else {
      ctl_advance<W>(a, c, b, t + 1, e2);
      stores_done();
      __syncthreads();
      if (regws) {
        if (tid < 64) ctl_entries(a, c, b, t + 1, e2, false);
      } else if (tid < MBOX_REPL) {
        st_dev_u32(a.mbox_w + (size_t)tid * 32 + b, mbox_word(a.ebase + t + 2, e2));
      }
    }
    ctl_prefetch<W>(a, c, b);  // overlaps the workers' step
    __syncthreads();
  }
  // release the workers from this request: register workers read it in the
  // entries of the step after the last (a failed build's workers leave on
  // the error word)
  if (regws) {
    if (!failed && tid < 64) ctl_entries(a, c, b, steps, 0, true);
  } else if (tid < MBOX_REPL) {
    st_dev_u32(a.mbox_w + (size_t)tid * 32 + b, mbox_word(a.ebase + tree_epoch_span(a.N) - 1, MBOX_DONE_E));
  }
  stores_done();
  ctl_output(a, c, b, failed);
  if (a.stats && tid == 0) {
    a.stats[2 * b] = steps;
    a.stats[2 * b + 1] = expanded;
  }
  // a launch that ends with the error word set tells the host through the
  // mirror, which the next build call reads without a synchronisation
  if (tid == 0) {
    const uint32_t e = ld_dev_u32(a.err);
    if (e != 0) {
      __hip_atomic_store(a.err_host, (int)e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      __threadfence_system();
    }
  }
}

template <typename W>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void tree_kernel(TreeArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  // no cache line of an exchange slot may survive from an earlier launch: an
  // acquire (cache invalidate) suffices; the writes of earlier kernels were
  // released at their end
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if ((int)blockIdx.x < a.n_workers) {
    if constexpr (sizeof(W) == 2) {
      if (a.regw == 1) return worker_regs<1, 1>(a, lds);
      if (a.regw == 2) return worker_regs<2, 1>(a, lds);
      if (a.regw == 3) return worker_regs<2, 2>(a, lds);
      if (a.regw == 4) return worker_regs<2, 4>(a, lds);
    }
    worker_main<W>(a, lds);
  } else {
    controller_main<W>(a, lds);
  }
}

// ---------------------------------------------------------------------------
// host side: schedule and launch

size_t plan_tree(TreeArgs& a, int wdtype_bf16, int pops, int max_workers, int lds_workers, int halves,
                 int ctl_advance, int device_exchange) {
  const int esz = wdtype_bf16 ? 2 : 4;
  const size_t lds_max = 160 * 1024;
  const int kp = k_padded(a.ds);
  if (a.N + 1 > XMAX || a.M > 64 || a.k > a.M || a.D > 31) return 0;
  // nodes per request per step: fill about TREE_MAX_COLS columns
  int p = pops > 0 ? pops : TREE_MAX_COLS / a.B;
  p = std::max(1, std::min(std::min(p, PMAX), TREE_MAX_COLS / a.B));
  const int lds_n_workers = a.n_workers;
  for (; p >= 1; --p) {
    const int cols = a.B * p;
    // register workers: one tile per wave if that many blocks fit, else two.
    // Two halves of the batch need the first half's columns to fill whole
    // 16-column blocks: the halves' node tables then share no cache line, so
    // a worker's reads of the first half's entries cannot cache the second's
    // before its controllers have written them.
    const bool regok = wdtype_bf16 && a.ds == RKB * 32 && !lds_workers;
    const int bh2 = (a.B + 1) / 2;
    const bool split = regok && a.B >= 2 && (bh2 * p) % 16 == 0 && (halves == 2 || halves == 0);
    int regw = 0, n_workers = lds_n_workers, hv = 1, ncb = (cols + 15) / 16;
    for (int hc = split ? 2 : 1; regok && hc >= 1 && !regw; --hc) {
      const int ncb_h = ((hc == 2 ? bh2 : a.B) * p + 15) / 16;
      // (tiles per wave, column blocks per block): 1 = (1, 1), 2 = (2, 1), 3 = (2, 2), 4 = (2, 4)
      for (int m = 1; m <= 4 && !regw; ++m) {
        const int tw = m == 1 ? 1 : 2, cpb = m == 4 ? 4 : m == 3 ? 2 : 1;
        const int ngq = ((a.n_tiles + tw - 1) / tw + 3) / 4;  // blocks per column group (64 flags each)
        const int nw = ngq * ((ncb_h + cpb - 1) / cpb);
        if (nw <= max_workers && ngq <= 64) regw = m, n_workers = nw, hv = hc, ncb = ncb_h;
      }
    }
    int kc = kp;
    size_t wl = REGW_STAGE_OFFSET + (size_t)(regw == 4 ? 64 : regw == 3 ? 32 : 16) * RSTRIDE * 2;
    if (!regw) {
      if (a.tiles_per_worker * ncb > 4 * PPW) continue;
      // worker staging phases: kc | kp, 32 | kc, stage within its share of LDS
      const size_t stage_cap = wdtype_bf16 ? 68 * 1024 : lds_max - worker_stage_offset(a.tiles_per_worker, kp, esz) -
                                                             (size_t)(2 * TREE_MAX_COLS + 64) * 4;
      while ((size_t)round_up(cols, 16) * (kc + STAGE_PAD) * esz > stage_cap && kc % 64 == 0 && wdtype_bf16) kc /= 2;
      wl = worker_lds_bytes(a.tiles_per_worker, kp, kc, cols, esz);
      if (wl > lds_max) continue;
    }
    // controller: records for the budget, the root and speculation room; the
    // frontier bound (k - 1) xcap + 1 must fit the merge's registers
    int qmax = p == 1 ? 8 : QCAP;
    int xcap = 0, fcap = 0;
    for (; qmax >= 1; qmax /= 2) {
      xcap = std::min(XMAX, a.N + 1 + 2 * qmax);
      fcap = (a.k - 1) * xcap + 1;
      if (fcap <= FCAPMAX) break;
    }
    if (qmax < 1) continue;
    a.p = p;
    a.kc = kc;
    a.regw = regw;
    a.ncbmax = ncb;
    a.halves = hv;
    a.bh = hv == 2 ? bh2 : a.B;
    a.wadv = regw && !ctl_advance ? 1 : 0;
    a.xlocal = a.wadv && !device_exchange ? 1 : 0;
    // register workers: column groups, and the tile groups holding the W1_S^T
    // tiles (block w has tile group w / ncg)
    a.ncg = 1;
    a.cpg = 16;
    a.ugq0 = a.ugq1 = 0;
    if (regw) {
      const int tw = regw == 1 ? 1 : 2, cpb = regw == 4 ? 4 : regw == 3 ? 2 : 1;
      const int tpb = 4 * tw;  // tiles per block
      const int u0 = 3 * a.ds / 16, u1 = (3 * a.ds + a.r + 15) / 16;  // tiles [u0, u1) hold u rows
      a.ncg = (ncb + cpb - 1) / cpb;
      a.cpg = 16 * cpb;
      a.ugq0 = u0 / tpb;
      a.ugq1 = (u1 - 1) / tpb;
    }
    a.n_workers = n_workers;
    a.qmax = qmax;
    a.xcap = xcap;
    a.fcap = fcap;
    // depth slots: as many as fit, at most p
    size_t off[L_COUNT];
    for (int ns = std::min(p, a.D); ns >= 1; --ns) {
      a.nslots = ns;
      const size_t cl = ctl_offsets(a, esz, off);
      if (cl <= lds_max) return std::max(cl, wl);
    }
  }
  return 0;
}

hipError_t launch_tree(const TreeArgs& a, int wdtype_bf16, size_t lds_bytes, hipStream_t stream, bool plain) {
  void* args[] = {const_cast<TreeArgs*>(&a)};
  const dim3 grid(a.n_workers + a.B), block(NT);
  const void* fn = wdtype_bf16 ? (const void*)tree_kernel<uint16_t> : (const void*)tree_kernel<float>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
  if (e != hipSuccess) return e;
  if (plain) return hipLaunchKernel(fn, grid, block, args, lds_bytes, stream);
  return hipLaunchCooperativeKernel(fn, grid, block, args, (unsigned)lds_bytes, stream);
}

}  // namespace dt
