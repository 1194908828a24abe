/*
 * dominotree.h -- C ABI of the MI355X (gfx950) conditional draft-tree builder.
 *
 * The library builds, for each request of a batch, the best-first draft tree
 * of DominoTree: per-depth top-M candidates of the drafter's base logits, then
 * a best-first loop that pops the frontier node with the highest cumulative
 * path log-probability, advances Domino's GRU causal state along that node's
 * path, applies the low-rank logit correction on the M candidate columns of the
 * next depth only, log-softmaxes the corrected logits and pushes the k best
 * children, until a fixed number of nodes has been popped.
 *
 * Sources (page title, then section):
 *   [Domino, Method]  "Domino: decoupling causal modeling from autoregressive
 *                     drafting in speculative decoding" (Chinese summary),
 *                     section 核心方法 -- S = GRU(embeddings of the earlier
 *                     draft tokens); dL = W2 SiLU(W1 [H_i; S]) with rank r;
 *                     final logits = base + dL.
 *   [Domino, Steps]   same page, 方法步骤详情 -- base logits are the frozen LM
 *                     head applied to the parallel backbone's hidden states.
 *   [DominoTree, 1]   "Riassunto Tecnico: DominoTree", Componenti Core 1 --
 *                     best-first max-heap on cumulative path log-probability;
 *                     children are scored by re-running the GRU correction on
 *                     the node's own path; H_d is shared by every path.
 *   [DominoTree, 2]   same page, Componenti Core 2 -- the correction is
 *                     restricted to each depth's top-M marginal candidates
 *                     (the r x M slice of W2) before the top-k children are
 *                     chosen.
 *   [DominoTree, 4]   same page, Componenti Core 4 -- fixed node budget.
 *
 * Conventions the pages leave open, fixed here (and in the CPU oracle):
 *   - GRU gate rows are (reset, update, new) as in torch.nn.GRUCell; the reset
 *     gate multiplies (W_hn S + b_hn); S' = (1 - z) n + z S.
 *   - A child at depth d uses H_d and its parent's state; the root's children
 *     use root_state and no GRU step is taken at the root.
 *   - Scores: z_m = (base_m + dL_m) / T; log-prob = z_m - LSE(z_1..z_M)
 *     (DT_NORM_TOPM) or z_m - LSE(z_1..z_M, tail) where tail is the LSE of
 *     base/T over the tokens outside the candidates (DT_NORM_FULLV).
 *   - Orders: candidates by (base logit desc, token id asc), +0 == -0, NaN
 *     last; children by (z desc, token id asc), -inf log-probs never pushed;
 *     pops by (score desc, depth asc, token id asc, parent index asc).
 *   - The budget N counts non-root nodes; a node joins the tree when popped;
 *     the N-th popped node and nodes at depth D are not expanded; a build ends
 *     after N pops or when the frontier is empty.
 *   - bf16 weights: every product accumulates in fp32; the GRU state is kept
 *     in fp32 and rounded to bf16 (nearest-even) only as a matrix operand when
 *     DT_ACT_BF16 is set; gates, SiLU, softmax and scores are fp32.
 *
 * Memory: every pointer in dt_weights, dt_inputs and dt_outputs is a DEVICE
 * pointer on the handle's device; every struct is passed by HOST pointer.
 * Tensors are dense row-major.  Streams are hipStream_t passed as void*
 * (NULL = the null stream).
 *
 * Errors: every entry point returns a dt_status; dt_last_error() gives the
 * calling thread's message for the last non-OK status.  Arguments are checked
 * on the host before anything is enqueued.  A device-side failure (a bounded
 * wait of the builder that ran out, or a broken invariant) sets the handle's
 * device error word; the launch that sees it set at its end also sets a
 * host-visible copy.  From then on dt_build_trees refuses with DT_EDEVICE
 * (without a synchronisation, so once the failing build has finished), and
 * dt_sync_status() reports DT_EDEVICE and resets the handle, after which
 * builds work again.  The trees of a failed build are undefined (its
 * n_nodes may hold -1).
 */
#ifndef DOMINOTREE_H
#define DOMINOTREE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DT_OK = 0,
  DT_EINVAL = -1,       /* a bad argument: NULL pointer, size out of range */
  DT_EUNSUPPORTED = -2, /* valid but beyond this build's limits */
  DT_ENOMEM = -3,       /* device allocation failed in dt_create */
  DT_EHIP = -4,         /* a HIP runtime call failed (message has the text) */
  DT_EDEVICE = -5       /* a builder's bounded wait ran out or an invariant broke on the device */
} dt_status;

typedef enum { DT_F32 = 0, DT_BF16 = 1 } dt_dtype;
typedef enum { DT_NORM_TOPM = 0, DT_NORM_FULLV = 1 } dt_norm;

/* dt_params.flags */
#define DT_ACT_BF16 1u  /* round the GRU state to bf16 where it is a GEMM operand */
#define DT_VALIDATE 2u  /* scan the base logits for NaN first (DT_EINVAL if any) */
#define DT_TIMING 4u    /* record HIP events between the phases of the build (dt_phase_times) */
#define DT_MARGINAL 8u  /* score with the base logits alone (dL = 0): the factorised, DDTree-style
                           tree that the conditional correction is compared against
                           ("Riassunto Tecnico: DominoTree", Definizione del Problema: scores
                           that depend on the position only); such a build computes no
                           per-node products (no GRU states, no W1/W2 work): only the
                           per-request blocks run */

/* Limits of this build (DT_EUNSUPPORTED beyond them). */
#define DT_MAX_BATCH 32
#define DT_MAX_DEPTHS 31
#define DT_MAX_TOPM 64
#define DT_MAX_BUDGET 1024
#define DT_MAX_FRONTIER 4096 /* budget * (top_k - 1) + 1 */
#define DT_MAX_VOCAB 1048574 /* 2^20 - 2: the builder's node entries hold a token in 20 bits */

typedef struct {
  int32_t vocab;     /* V, 1..DT_MAX_VOCAB */
  int32_t depths;    /* D = draft block size - 1 */
  int32_t hidden;    /* h: rows of H_d, rows of the H half of W1 */
  int32_t emb_dim;   /* e: embedding size (GRU input) */
  int32_t state_dim; /* d_s: GRU state size */
  int32_t rank;      /* r: correction rank */
  int32_t max_batch; /* largest batch a build will be given */
  dt_dtype wdtype;   /* dtype of emb, w_ih, w_hh, w1, w2, w_lm and hidden */
} dt_dims;

/* Weights, all device pointers of dtype dims.wdtype unless noted.
 * emb is referenced, not copied: it must stay valid while the handle lives.
 * The others are copied (re-laid out) by dt_create and may be freed after. */
typedef struct {
  const void* emb;   /* [V, e] token embeddings (GRU input E[token]) */
  const void* w_ih;  /* [3 d_s, e] GRU input weights, row blocks (r, z, n) */
  const void* w_hh;  /* [3 d_s, d_s] GRU state weights, row blocks (r, z, n) */
  const float* b_ih; /* [3 d_s] fp32 or NULL (zeros) */
  const float* b_hh; /* [3 d_s] fp32 or NULL (zeros) */
  const void* w1;    /* [h + d_s, r]: u = [H_d; S] @ w1 (rows 0..h-1 act on H_d) */
  const void* w2;    /* [r, V]: dL = a @ w2 */
  const void* w_lm;  /* [h, V] LM head, or NULL (then base logits must be given) */
} dt_weights;

typedef struct {
  int32_t top_m;     /* M, 1..min(V, DT_MAX_TOPM) */
  int32_t top_k;     /* k, 1..M */
  int32_t budget;    /* N, 1..DT_MAX_BUDGET, with N (k - 1) + 1 <= DT_MAX_FRONTIER */
  float temperature; /* T > 0 */
  dt_norm norm;
  uint32_t flags;    /* DT_ACT_BF16 | DT_VALIDATE | DT_TIMING */
} dt_params;

typedef struct {
  int32_t batch;            /* b, 1..dims.max_batch (<= DT_MAX_BATCH) */
  const float* base_logits; /* [b, D, V] fp32, or NULL: computed as H @ w_lm */
  const void* hidden;       /* [b, D, h] backbone hidden states H_1..H_D (wdtype) */
  const float* root_state;  /* [b, d_s] fp32, or NULL (zeros) */
} dt_inputs;

/* Outputs (device pointers, caller-owned, sized for the batch and budget).
 * Node 0 is the root: token -1, parent -1, depth 0, score 0.  Nodes 1..n are
 * in pop order; slots past n_nodes hold token -1, parent -1, depth -1,
 * score -inf.  The cand_* / lse / stats / logits pointers are optional (NULL to skip):
 * the per-depth candidates (sorted), their base logits and the LSE of base/T
 * over the whole vocabulary. */
typedef struct {
  int32_t* tokens;   /* [b, N + 1] */
  int32_t* parents;  /* [b, N + 1] */
  int32_t* depths;   /* [b, N + 1] */
  float* scores;     /* [b, N + 1] cumulative log-prob (natural log) */
  int32_t* n_nodes;  /* [b] non-root nodes produced (N unless the frontier emptied) */
  int32_t* cand_ids; /* [b, D, M] or NULL */
  float* cand_logits;/* [b, D, M] or NULL */
  float* lse;        /* [b, D] or NULL */
  int32_t* stats;    /* [b, 2] or NULL: per request, the steps of the builder's loop and the
                        nodes it expanded (several nodes per step, speculative ones included) */
  float* logits;     /* [b, D, V] or NULL: a copy of the base logits the LM head computed
                        (written only when inputs.base_logits is NULL) */
} dt_outputs;

typedef struct dt_handle dt_handle;

/* Create a handle on the current HIP device: copy and re-lay-out the weights
 * into handle-owned device memory (w2 -> [V, r]; w_lm -> the LM-head GEMM's
 * tile order; GRU and W1 in the builder's tile order) and allocate the
 * workspace for dims.max_batch and for every params no larger than
 * *max_params (top_m, top_k, budget).
 * Enqueued on `stream` and synchronised before returning.
 * Errors: DT_EINVAL (NULL h/dims/weights/max_params, non-positive sizes,
 * missing required weight), DT_EUNSUPPORTED (limits, dims not multiples of
 * the tile sizes: for bf16, e, d_s and h multiples of 32 and r of 16; d_s a
 * multiple of 4), DT_ENOMEM, DT_EHIP.  On error *h is NULL. */
dt_status dt_create(dt_handle** h, const dt_dims* dims, const dt_weights* w,
                    const dt_params* max_params, void* stream);

/* Build the trees of one batch [DominoTree, 1, 2, 4].  Enqueues the kernels on
 * `stream` and returns: no host synchronisation and no allocation (except
 * under DT_VALIDATE, which synchronises to read its NaN scan).  Results
 * are valid once the stream reaches this point.  P = H W1_H runs first on
 * `stream` when base logits are given; with the LM head it runs on a stream
 * the handle owns (default priority), forked from and joined back into
 * `stream` with events, beside the LM-head GEMM.  A handle must not be
 * used by two builds at once (one workspace).  When in->base_logits is NULL the
 * base logits are computed from in->hidden with w_lm [Domino, Steps] into a
 * handle-owned fp32 workspace, from which the candidates and LSE are taken.
 * Errors: DT_EINVAL (NULL pointers, batch out of range, params out of range
 * or above the handle's max_params, NaN logits under DT_VALIDATE, w_lm
 * missing with NULL base logits), DT_EUNSUPPORTED, DT_EHIP, DT_EDEVICE (a
 * finished earlier build on the handle set the device error word; nothing is
 * enqueued until dt_sync_status resets the handle). */
dt_status dt_build_trees(dt_handle* h, const dt_inputs* in, const dt_params* p,
                         dt_outputs* out, void* stream);

/* Synchronise `stream` and report a device-side failure of the handle's
 * builds so far: DT_OK, or DT_EDEVICE after clearing the error word, its host
 * copy and the builder's mailboxes (synchronising again), so that the next
 * build runs as on a fresh handle.  Errors: DT_EINVAL (NULL h), DT_EHIP. */
dt_status dt_sync_status(dt_handle* h, void* stream);

/* Schedule of the tree builder.  These change how the work is spread over the
 * GPU, not what is computed: the trees are the same up to the rounding of the
 * per-node products, whose summation order can depend on the worker layout.
 * Zero in a field keeps the default. */
typedef struct {
  int32_t pops;             /* nodes a request may expand per step, 0..16 (default: fill the 512
                               exchange columns of a step, at most 16) */
  int32_t halves;           /* 0 (default: two from 2 requests on where the first half fills whole
                               16-column blocks), 1 (the workers serve the batch whole per step) or 2
                               (in two halves, one half's products beside the other's scoring) */
  int32_t lds_workers;      /* 1: workers that stage operands in LDS even where register-resident
                               workers fit; 0: default */
  int32_t tiles_per_worker; /* LDS-staging workers: weight tiles per worker block, 0..64 (default:
                               one per worker when the workers fit beside the controllers) */
  int32_t advance;          /* who advances the GRU states of a step's nodes beside register-resident
                               workers: 0 (default) or 1 the workers, 2 the controllers (the
                               LDS-staging workers always leave it to the controllers) */
  int32_t launch;           /* the builder's blocks wait on each other, so all of them must be resident
                               at once (one per compute unit, at most as many as the GPU has).
                               0 (default) or 1: a plain launch, which has them all resident when the
                               build does not share the GPU with other streams' kernels; if other work
                               keeps some blocks waiting for a compute unit long enough, the bounded
                               waits end the build with DT_EDEVICE.  2: a cooperative launch, which
                               guarantees it, for callers that share the GPU (it costs about 20 us) */
  int32_t dl;               /* the correction dL = W2[:, candidates]^T a of each expansion: 0 (default)
                               on the matrix cores where the weights are bf16 and r is a multiple of
                               32, else with vector FMAs; 1: always with vector FMAs */
  int32_t exchange;         /* register-resident workers tell the other blocks of their column group
                               that a step's advanced states are stored: 0 (default) with flags kept
                               in the L2 of their XCD when the launch's first exchange finds the whole
                               group on one XCD, else device-wide; 1: always device-wide */
} dt_schedule;

/* Set the schedule the handle's next builds use (NULL restores the defaults).
 * Host only; takes effect at the next dt_build_trees.  A schedule that does
 * not fit a build's shape makes that build return DT_EUNSUPPORTED.
 * Errors: DT_EINVAL (NULL h, a field out of range). */
dt_status dt_set_schedule(dt_handle* h, const dt_schedule* s);

/* For tests of the failure path: enqueue on `stream` a write of `code` (> 0)
 * into the handle's device error word, as a builder wait that ran out would.
 * Every wait of the next build then gives up at its next periodic check of
 * the word instead of waiting for its bound, so the build ends promptly, and
 * the error is reported as any device failure (see Errors above).
 * Errors: DT_EINVAL (NULL h, code <= 0), DT_EHIP. */
dt_status dt_set_device_error(dt_handle* h, int32_t code, void* stream);

/* Mean durations, in milliseconds, of the phases of the builds made with
 * DT_TIMING since the previous call (at most the last 256 of them), measured
 * with HIP events recorded on each build's stream: ms[0] the LM head, or
 * P = H W1_H when base logits are given, ms[1] per-depth candidates (top-M +
 * LSE), ms[2] the wait for P after them (LM head only), ms[3]
 * the builder's set-up (a mailbox clear only when the epoch space wraps),
 * ms[4] the tree builder kernel.  Waits for
 * those events, writes min(n, 5) values and the number of builds averaged to
 * *count, then starts a new averaging window.
 * Errors: DT_EINVAL (NULL h, ms or count), DT_EHIP. */
dt_status dt_phase_times(dt_handle* h, float* ms, int n, int32_t* count);

/* ---- Greedy chain head ----------------------------------------------------
 * The Domino head as a chain over the whole vocabulary [Domino, Method;
 * Domino, Steps]: for each draft position d = 1..D in turn,
 *   dL_d = W2^T SiLU(W1^T [H_d; S]) for every token, x_d = argmax(base_d + dL_d)
 *   (ties to the lowest token id), then S <- GRU(S, E[x_d]),
 * starting from S = root_state (zeros when NULL).  Uses the handle's weights
 * and workspace (not at the same time as a dt_build_trees on the handle);
 * in->base_logits NULL computes the base logits with w_lm as dt_build_trees
 * does.  flags: DT_ACT_BF16 (required with bf16 weights, refused with fp32).
 * Outputs (device, caller-owned): tokens [b, D]; logits [b, D] or NULL, the
 * corrected logit base + dL of each pick.  Enqueued on `stream`, no
 * synchronisation, no allocation.
 * Errors: DT_EINVAL (NULL h/in/tokens/hidden, batch outside 1..max_batch,
 * unknown flags, no base logits and no w_lm), DT_EUNSUPPORTED (rank above 256
 * or not a multiple of 8, the DT_ACT_BF16 rule), DT_EHIP. */
dt_status dt_draft_chain(dt_handle* h, const dt_inputs* in, uint32_t flags, int32_t* tokens, float* logits,
                         void* stream);

/* ---- Sampled chain head --------------------------------------------------
 * The chain with each draft token sampled from the refined logits at
 * temperature T [Domino, Steps: at inference each draft token is sampled from
 * the final logits l_i + c_i], i.e. from softmax((base_d + dL_d) / T), by the
 * Gumbel-max rule:
 *   x_d = argmax_v ((base_d + dL_d)_v / T + g_{b,d,v})   (ties to the lowest id),
 *   g = -ln(-ln u),  u = (floor(w / 2^9) + 1/2) / 2^23,
 *   w = word (v mod 4) of Philox4x32-10 (Salmon et al., SC 2011) at counter
 *       (floor(v / 4), d, b, 0) under key (seed mod 2^32, floor(seed / 2^32)),
 * with b the request's row in the call and d the 0-based position; then
 * S <- GRU(S, E[x_d]) as in the greedy chain.  The seed fixes every draw:
 * the same seed and inputs give the same tokens; use a new seed for each
 * call that should draw afresh.  Arguments, workspace and outputs as for
 * dt_draft_chain (logits: the corrected logit base + dL of each pick, not its
 * perturbed score).
 * Errors: as dt_draft_chain, and DT_EINVAL for a temperature that is not
 * positive and finite (T = 0 is the greedy chain). */
dt_status dt_draft_chain_sample(dt_handle* h, const dt_inputs* in, uint32_t flags, float temperature,
                                uint64_t seed, int32_t* tokens, float* logits, void* stream);

/* ---- Allocation-free chain head ------------------------------------------
 * For callers that cannot allocate device memory during a call: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Computes exactly what dt_draft_chain computes, with the same arguments,
 * results and errors, but its per-call workspace (P = H W1_H for every
 * position, the per-position products [W_hh S | W1_S^T S], the state and its
 * operand copy, the block-wise best candidates) lives in a fixed device array
 * of DT_NOALLOC_SCRATCH_BYTES that the library holds on each GPU until the
 * process ends (its address is taken when the first handle is created on
 * that GPU), instead of in the handle's workspace.  It calls no allocating
 * routine.  Differences: in->base_logits is required (NULL gives DT_EINVAL:
 * the LM head's logits do not fit the array), and a batch whose workspace
 * exceeds the array gives DT_EUNSUPPORTED (the Qwen3-8B shape, d_s 1024,
 * r 256, 15 positions, uses about 1.4 MB at batch 32).  Nothing in the array
 * needs clearing: every value is written before it is read.  Every call on a
 * GPU shares that GPU's array, whatever the handle, stream or thread: calls
 * that overlap on one GPU race, so the caller serialises them. */
#define DT_NOALLOC_SCRATCH_BYTES (4u << 20)
dt_status dt_draft_chain_noalloc(dt_handle* h, const dt_inputs* in, uint32_t flags, int32_t* tokens,
                                 float* logits, void* stream);

/* ---- Folding committed tokens into the causal state ------------------------
 * The causal state before a draft block is the GRU over the tokens committed
 * so far [Domino, Method: S_{i-1} = GRU(embeddings of the tokens before i)].
 * For each request, S <- GRU(S, E[t]) over tokens[b, 0..n_tokens-1] in order,
 * starting from prev_state (zeros when NULL), and the result goes to
 * state_out: pass it as root_state to dt_build_trees / dt_draft_chain, or as
 * prev_state to the next fold (the state carried across rounds).
 * tokens [b, n_tokens] int32 (ids clamped to 0..V-1), prev_state and
 * state_out [b, d_s] fp32, all device pointers (state_out may equal
 * prev_state).  flags: DT_ACT_BF16 as for dt_draft_chain.  Uses the handle's
 * workspace (not at the same time as another call on the handle).
 * Errors: DT_EINVAL (NULL h/tokens/state_out, batch outside 1..max_batch,
 * n_tokens < 1, unknown flags), DT_EUNSUPPORTED (the DT_ACT_BF16 rule),
 * DT_EHIP. */
dt_status dt_fold_state(dt_handle* h, int32_t batch, int32_t n_tokens, const int32_t* tokens,
                        const float* prev_state, float* state_out, uint32_t flags, void* stream);

/* ---- Verification inputs ------------------------------------------------
 * The drafted tree is verified with the standard tree attention of
 * DDTree/SpecInfer: a causal mask built from each node's ancestors
 * ("Riassunto Tecnico: DominoTree", Componenti Core 5).  The view below reads
 * trees in dt_outputs' layout (row stride cols = N + 1); every pointer is a
 * DEVICE pointer. */
typedef struct {
  int32_t batch;              /* b >= 1 */
  int32_t cols;               /* row stride of the arrays: N + 1, 1..DT_MAX_BUDGET + 1 */
  const int32_t* parents;     /* [b, cols] (dt_outputs.parents) */
  const int32_t* depths;      /* [b, cols] */
  const int32_t* tokens;      /* [b, cols], or NULL (then no flattened tokens) */
  const int32_t* n_nodes;     /* [b] */
  const int32_t* prefix_len;  /* [b] committed prefix length, or NULL (0) */
  const int32_t* anchor;      /* [b] last committed token (the root), or NULL (-1) */
} dt_tree_view;

typedef struct {
  uint32_t* mask;      /* [b, cols, ceil(cols / 32)]: bit j % 32 of word j / 32 of
                          row i is set when node j is node i or an ancestor of it
                          (root included); rows and columns past n_nodes are 0 */
  int32_t* positions;  /* [b, cols]: prefix_len + depth, -1 past n_nodes */
  int32_t* tokens;     /* [b, cols] or NULL: the anchor at 0, node tokens at
                          1..n_nodes, -1 past n_nodes */
  int32_t* bad;        /* [b] or NULL: 1 when a tree breaks the builder's
                          invariants (n_nodes outside 0..cols-1, a parent not
                          smaller than its child, a path not ending at the
                          root, a depth other than the path length), else 0 */
} dt_verify_outputs;

/* Build the tree-attention inputs of b trees on `stream` (one kernel, no
 * synchronisation, no allocation).  A bad tree's mask rows hold the nodes
 * that its walk reached before the break; its positions use the given depths.
 * Errors: DT_EINVAL (NULL trees/out, NULL required pointers, batch or cols
 * below 1, out->tokens without trees->tokens), DT_EUNSUPPORTED (cols above
 * DT_MAX_BUDGET + 1), DT_EHIP. */
dt_status dt_tree_attention_inputs(const dt_tree_view* trees, const dt_verify_outputs* out, void* stream);

/* Free everything the handle owns (synchronises the device first). NULL is a no-op. */
dt_status dt_destroy(dt_handle* h);

/* Message of the calling thread's last non-OK status ("" if none). */
const char* dt_last_error(void);

/* Library version string. */
const char* dt_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DOMINOTREE_H */
