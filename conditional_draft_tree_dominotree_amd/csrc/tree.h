// Arguments, schedule and launch of the persistent tree builder (tree.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dt {

// ---- the tree builder (tree.hip)
struct TreeArgs {
  // shapes and parameters
  int B, D, ds, r, M, k, N;
  float T;
  int fullv;
  int act_bf16;
  int marginal;         // 1: no correction (dL = 0), the factorised scores of the base logits
  int dlfma;            // 1: dL with vector FMAs even where the matrix cores could take it
  int n_workers;        // worker blocks; block ids [0, n_workers) are workers
  int tiles_per_worker;
  int n_tiles;          // (3 ds + r) / 16
  // schedule (set by plan_tree)
  int p;                // nodes a request may expand per step (exchange columns per request)
  int kc;               // state elements a worker stages per phase (kp / kc phases)
  int regw;             // 0: workers stage operands in LDS; register workers: 1 (1 tile per wave, 1
                        // column block per block), 2 (2 tiles, 1 block), 3 (2 tiles, 2 blocks),
                        // 4 (2 tiles, 4 blocks)
  int ncbmax;           // register workers: 16-column blocks per step (per half of the batch)
  int halves;           // register workers: 2 serve the requests [0, bh) and [bh, B) of a step in
                        // turn, so that one half's products overlap the other half's scoring; else 1
  int bh;               // requests in the first half (B when halves = 1)
  int wadv;             // 1: the workers advance the GRU states of a step's nodes (register workers)
  int ncg, cpg;         // register workers: column groups and columns per group (16 per column block).
                        // Column c of a half's p B_h columns is node c % p of the half's request c / p;
                        // block w serves the columns [cpg g, cpg (g + 1)) of group g = w % ncg, with the
                        // tile group w / ncg
  int ugq0, ugq1;       // register workers: the tile groups [ugq0, ugq1] hold the W1_S^T tiles; once
                        // they acknowledge a step, its u rows are stored
  int xlocal;           // register workers: 1 lets a column group whose blocks all run on one XCD
                        // (checked at the launch's first exchange) raise its group flags in that
                        // XCD's L2 instead of device-wide
  int xcap;             // node records per request (budget + root + speculation room)
  int fcap;             // frontier entries per request
  int qmax;             // frontier entries tested per pop round
  int nslots;           // depth slots of W2 candidate rows in a controller's LDS
  // read-only inputs
  const void* tiles;       // packed [W_hh ; W1_S^T] tiles
  const float* b_hh;       // [3 ds] or NULL
  const float* G;          // [V, 3 ds]: W_ih E[v] + b_ih
  const void* w2t;         // [V, r] (wdtype)
  const float* P;          // [p_parts][B, D, r]: H_d W1_H, the sum of p_parts partials
  int p_parts;             // 1, or P_KSPLIT when P comes from the candidate merge's launch
  size_t p_stride;         // floats between partials
  const int32_t* cand_ids; // [B, D, M]
  const float* cand_vals;  // [B, D, M]
  const float* tail;       // [B, D]
  const int32_t* tokrank;  // [B, D, M]
  const float* root;       // [B, ds] or NULL
  // write-once exchange slots, step-major: slot (t, b, j) = (t B + b) p + j
  float* state;            // [slots, ds] fp32 GRU state of the node expanded in the slot
  void* act;               // [slots, ds] its GEMM operand copy (wdtype)
  float* gh;               // [slots, 3 ds]
  float* u;                // [slots, r]
  uint64_t* ninfo;         // [N + 2][TREE_MAX_COLS]: node entries (ninfo_entry) of each step's columns
  uint32_t* gflag;         // [16][64] worker group flags: 2 epoch + half once a group's states of
                           // that step and half of the batch are advanced
  uint32_t* ready;         // [64] controller b: its start-up loads are done (the workers then load weights)
  uint32_t* xccw;          // [256] worker w: the XCC (XCD) its block runs on, this launch
  uint32_t* mbox_w;        // [MBOX_REPL][32] controller -> worker mailbox words, one copy of a request's
                           // word per line; worker w polls copy w % MBOX_REPL
  uint32_t* mbox_c;        // [B][256] worker -> controller mailboxes
  int* err;                // device error word
  int* err_host;           // pinned host mirror: a controller that ends with err set copies it there
  // outputs
  int32_t *tokens, *parents, *depths, *n_nodes;
  float* scores;
  int32_t* stats;          // [B, 2] or NULL: steps of the request's loop, nodes it expanded
  unsigned spin_limit;
  uint32_t ebase;          // epochs of this launch: ebase + 1 .. ebase + tree_epoch_span(N) - 1
};
// Copies of the controller -> worker mailbox line: each controller writes its
// word into every copy, and the workers' polls spread over the copies.
constexpr int MBOX_REPL = 8;
// Exchange columns a build may use per step (slots per step = B p <= this).
constexpr int TREE_MAX_COLS = 512;
constexpr int GFLAG_WORDS = 16 * 64 + 64 + 256;  // worker group flags, controller ready flags and the
                                                  // workers' XCC words, before the worker mailboxes
// Epochs a launch may use (at most N + 1 steps, the first post and the last).
__host__ __device__ inline uint32_t tree_epoch_span(int N) { return (uint32_t)N + 8u; }
// mailbox words hold the epoch in 27 bits, node entries in 24: epochs stay
// below 2^24, and the mailboxes and node entries are cleared when they wrap
constexpr uint32_t TREE_EPOCH_LIMIT = 1u << 24;
// A node entry of the node table: the epoch of the step it is published for
// (24 bits), the token (20 bits) and the parent's exchange slot (20 bits).  It
// validates itself: a reader compares its epoch with the step's.
__host__ __device__ inline uint64_t ninfo_entry(uint32_t epoch, uint32_t tok, uint32_t src) {
  return ((uint64_t)(epoch & 0xFFFFFFu) << 40) | ((uint64_t)(tok & 0xFFFFFu) << 20) | (uint64_t)(src & 0xFFFFFu);
}
// Token fields of entries that are not nodes.  With register workers a
// controller writes an entry for each of its p columns of every step: the
// node's, NINFO_NONE where it expands fewer than p nodes, and NINFO_DONE in
// the step after its last (the request has finished).
constexpr uint32_t NINFO_NONE = 0xFFFFFu, NINFO_DONE = 0xFFFFEu;
constexpr int NINFO_MAX_VOCAB = 0xFFFFE;  // tokens stay below the markers
// Fills the schedule fields of `a` (p from `pops`, 0 = automatic) and returns
// the dynamic LDS bytes the launch needs, or 0 if the shape cannot be served.
// With register workers (allowed unless `lds_workers`) it also sets
// n_workers, at most `max_workers`; otherwise n_workers and tiles_per_worker
// are the caller's.
// `halves`: 1 or 2 forces the split of the batch, 0 = automatic (2 for register
// workers with at least 2 requests whose first half fills whole 16-column blocks).
// `device_exchange`: 1 keeps the register workers' group exchange device-wide
// even where a group runs on one XCD.
size_t plan_tree(TreeArgs& a, int wdtype_bf16, int pops, int max_workers, int lds_workers, int halves,
                 int ctl_advance, int device_exchange);
hipError_t launch_tree(const TreeArgs& a, int wdtype_bf16, size_t lds_bytes, hipStream_t stream, bool plain);

}  // namespace dt
