// Host side of the C ABI declared in include/dominotree.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/dominotree.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

dt_status fail(dt_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

// what the bits of the device error word mean (several may be set)
std::string device_error_text(int e) {
  static const char* const why[] = {
      "a bounded wait ran out",                                // 1
      "a request needed more steps than its budget allows",    // 2
      "a frontier outgrew its capacity",                       // 4
      "a node's parent had no state slot",                     // 8
      "the LM head's candidate lists did not agree with the recomputed logits",  // 16
  };
  std::string s;
  for (int b = 0; b < 5; ++b)
    if (e & (1 << b)) s += (s.empty() ? "" : "; ") + std::string(why[b]);
  if (e >> 5) s += (s.empty() ? "" : "; ") + std::string("unknown bits");
  return s;
}

#define HIPCHK(expr)                                                                     \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess) return fail(DT_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

}  // namespace

// Workspace of dt_draft_chain_noalloc: a file-scope device array, one copy per
// GPU, held until the process ends.  Host code uses only the address that
// hipGetSymbolAddress returns for the current device (scratch_setup), never
// the array's name, which on the host is a stand-in and not a device address.
static __device__ __align__(256) unsigned char scratch[DT_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
unsigned char* g_scratch[MAX_DEVICES] = {};

// Take the array's address on `device`, which must be current; once per device.
dt_status scratch_setup(int device) {
  if (device < 0 || device >= MAX_DEVICES) return fail(DT_EUNSUPPORTED, "device %d >= %d", device, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[device]) return DT_OK;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) return fail(DT_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
  g_scratch[device] = static_cast<unsigned char*>(p);
  return DT_OK;
}

unsigned char* scratch_of(int device) {
  if (device < 0 || device >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch[device];
}

}  // namespace

struct dt_handle {
  dt_dims dims{};
  dt_params maxp{};
  int device = 0;
  int n_cu = 0;
  int bf16 = 0;
  size_t esz = 4;
  const void* emb = nullptr;
  // handle-owned weights
  float* G = nullptr;       // [V, 3 ds]
  void* tiles = nullptr;    // packed [W_hh ; W1_S^T]
  float* b_hh = nullptr;    // [3 ds] or null
  void* w1h_t = nullptr;    // [r, h]
  void* w2t = nullptr;      // [V, r]
  void* wlm_t = nullptr;    // W_lm^T: tiled for the LM-head GEMM (wlm_tiled) or [V, h]; or null
  bool wlm_tiled = false;
  uint16_t* a_tiles = nullptr;  // H in the LM-head GEMM's tile order (per call)
  float* logits = nullptr;  // [max_batch, D, V] base logits computed by the LM head (the chain head)
  uint64_t* lm_lists = nullptr;  // LM head fused with the candidate selection: per-row lists and statistics
  float2* lm_stats = nullptr;
  void* wc_rm = nullptr;    // [3 ds + r, ds] row-major [W_hh ; W1_S^T] (the chain head)
  void* w2f = nullptr;      // bf16 W2^T in the chain head's MFMA fragment order, or null
  int n_tiles = 0;
  // workspace
  uint64_t* chunk_cand = nullptr;
  float4* chunk_stat = nullptr;
  int32_t* cand_ids = nullptr;
  float* cand_vals = nullptr;
  int32_t* tokrank = nullptr;
  float* lse = nullptr;
  float* tail = nullptr;
  float* P = nullptr;
  float* state = nullptr;
  void* act = nullptr;
  float* gh = nullptr;
  float* u = nullptr;
  uint64_t* ninfo = nullptr;
  size_t ninfo_words = 0;      // 32-bit words of ninfo (for clearing)
  uint32_t* mbox_w = nullptr;  // group flags, then the worker mailboxes
  uint32_t* mbox_c = nullptr;
  int* err = nullptr;
  int* err_host = nullptr;  // pinned mirror of err, set by a builder launch that ends with err set
  int* nanflag = nullptr;
  dt_schedule sched{};      // schedule overrides (dt_set_schedule); zeros: defaults
  float* chain_gu = nullptr;     // chain head: [max_batch, 3 ds + r]
  float* chain_s = nullptr;      // [max_batch, ds]
  void* chain_sop = nullptr;     // [max_batch, ds] (wdtype)
  uint64_t* chain_part = nullptr;  // [max_batch, max(chain_blocks(V), chain_mfma_blocks(V))]
  size_t act_bytes = 0;
  uint32_t ebase = 0;  // epoch base of the next launch (mailboxes hold older epochs)
  hipStream_t side = nullptr;  // runs P = H W1_H beside the candidate selection
  hipEvent_t fork_ev = nullptr, join_ev = nullptr;
  int max_workers = 0;
  static constexpr int RING = 256;   // timed builds kept for dt_phase_times
  static constexpr int NPH = 5;       // timed phases
  hipEvent_t ev[RING][NPH + 1] = {};
  int timed = 0;                      // timed builds since the last dt_phase_times
};

namespace {

template <typename T>
dt_status dalloc(T** p, size_t bytes) {
  *p = nullptr;
  if (bytes == 0) bytes = 16;
  hipError_t e = hipMalloc(reinterpret_cast<void**>(p), bytes);
  if (e != hipSuccess) return fail(DT_ENOMEM, "hipMalloc(%zu): %s", bytes, hipGetErrorString(e));
  return DT_OK;
}

void free_all(dt_handle* h) {
  void* ptrs[] = {h->G,       h->tiles,    h->b_hh,     h->w1h_t, h->w2t,      h->wlm_t,  h->logits,
                  h->chunk_cand, h->chunk_stat, h->cand_ids, h->cand_vals, h->tokrank, h->lse,
                  h->tail,    h->P,        h->state,    h->act,   h->gh,       h->u,
                  h->ninfo,   h->mbox_w,   h->mbox_c,   h->err,   h->nanflag, h->wc_rm,
                  h->chain_gu, h->chain_s, h->chain_sop, h->chain_part, h->a_tiles, h->w2f, h->lm_lists,
                  h->lm_stats};
  for (void* p : ptrs)
    if (p) (void)hipFree(p);
  for (auto& set : h->ev)
    for (hipEvent_t& e : set)
      if (e) (void)hipEventDestroy(e);
  if (h->fork_ev) (void)hipEventDestroy(h->fork_ev);
  if (h->join_ev) (void)hipEventDestroy(h->join_ev);
  if (h->side) (void)hipStreamDestroy(h->side);
  if (h->err_host) (void)hipHostFree(h->err_host);
}

dt_status check_dims(const dt_dims* d) {
  if (d->vocab <= 0 || d->depths <= 0 || d->hidden <= 0 || d->emb_dim <= 0 || d->state_dim <= 0 ||
      d->rank <= 0 || d->max_batch <= 0)
    return fail(DT_EINVAL, "dims must be positive");
  if (d->wdtype != DT_F32 && d->wdtype != DT_BF16) return fail(DT_EINVAL, "unknown wdtype %d", (int)d->wdtype);
  if (d->max_batch > DT_MAX_BATCH) return fail(DT_EUNSUPPORTED, "max_batch %d > %d", d->max_batch, DT_MAX_BATCH);
  if (d->depths > DT_MAX_DEPTHS) return fail(DT_EUNSUPPORTED, "depths %d > %d", d->depths, DT_MAX_DEPTHS);
  if (d->vocab > DT_TOPM_MAX_CHUNKS * TOPM_CHUNK)
    return fail(DT_EUNSUPPORTED, "vocab %d > %d", d->vocab, DT_TOPM_MAX_CHUNKS * TOPM_CHUNK);
  static_assert(DT_MAX_VOCAB == dt::NINFO_MAX_VOCAB, "the header's vocabulary limit is the node entries'");
  if (d->vocab > DT_MAX_VOCAB)  // node entries hold tokens in 20 bits, beside two markers
    return fail(DT_EUNSUPPORTED, "vocab %d > %d", d->vocab, DT_MAX_VOCAB);
  if (d->wdtype == DT_BF16 && (d->emb_dim % 8 || d->hidden % 8))
    return fail(DT_EUNSUPPORTED, "bf16 weights need emb_dim and hidden multiples of 8");
  if (d->rank > 4096 || d->state_dim > 8192) return fail(DT_EUNSUPPORTED, "rank or state_dim too large");
  return DT_OK;
}

dt_status check_params(const dt_params* p, int V, const dt_params* maxp) {
  if (p->top_m < 1 || p->top_m > V) return fail(DT_EINVAL, "top_m %d outside 1..V", p->top_m);
  if (p->top_m > DT_MAX_TOPM) return fail(DT_EUNSUPPORTED, "top_m %d > %d", p->top_m, DT_MAX_TOPM);
  if (p->top_k < 1 || p->top_k > p->top_m) return fail(DT_EINVAL, "top_k %d outside 1..top_m", p->top_k);
  if (p->budget < 1) return fail(DT_EINVAL, "budget %d < 1", p->budget);
  if (p->budget > DT_MAX_BUDGET) return fail(DT_EUNSUPPORTED, "budget %d > %d", p->budget, DT_MAX_BUDGET);
  if ((long)p->budget * (p->top_k - 1) + 1 > DT_MAX_FRONTIER)
    return fail(DT_EUNSUPPORTED, "budget * (top_k - 1) + 1 > %d", DT_MAX_FRONTIER);
  if (!(p->temperature > 0.f) || !std::isfinite(p->temperature))
    return fail(DT_EINVAL, "temperature must be finite and > 0");
  if (p->norm != DT_NORM_TOPM && p->norm != DT_NORM_FULLV) return fail(DT_EINVAL, "unknown norm");
  if (p->flags & ~(DT_ACT_BF16 | DT_VALIDATE | DT_TIMING | DT_MARGINAL))
    return fail(DT_EINVAL, "unknown flags 0x%x", p->flags);
  if (maxp && (p->top_m > maxp->top_m || p->top_k > maxp->top_k || p->budget > maxp->budget))
    return fail(DT_EINVAL, "params exceed the handle's max_params");
  return DT_OK;
}

// tiles per worker: one per worker when the workers fit beside the controllers
int choose_tpw(const dt_handle* h, int B) {
  if (h->sched.tiles_per_worker > 0) return h->sched.tiles_per_worker;
  const int avail = h->n_cu - B;
  int tpw = 1;
  while ((h->n_tiles + tpw - 1) / tpw > avail) ++tpw;
  return tpw;
}

}  // namespace

extern "C" {

const char* dt_last_error(void) { return g_err.c_str(); }

const char* dt_version(void) { return "dominotree-mi355x 0.1 (gfx950)"; }

dt_status dt_create(dt_handle** out, const dt_dims* dims, const dt_weights* w, const dt_params* maxp,
                    void* stream_) {
  if (!out) return fail(DT_EINVAL, "h is NULL");
  *out = nullptr;
  if (!dims || !w || !maxp) return fail(DT_EINVAL, "dims, weights and max_params are required");
  dt_status s = check_dims(dims);
  if (s != DT_OK) return s;
  s = check_params(maxp, dims->vocab, nullptr);
  if (s != DT_OK) return s;
  if (!w->emb || !w->w_ih || !w->w_hh || !w->w1 || !w->w2) return fail(DT_EINVAL, "a required weight is NULL");
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);

  dt_handle* h = new dt_handle();
  h->dims = *dims;
  h->maxp = *maxp;
  h->bf16 = dims->wdtype == DT_BF16;
  h->esz = h->bf16 ? 2 : 4;
  h->emb = w->emb;
  auto bail = [&](dt_status st) {
    (void)hipStreamSynchronize(stream);
    free_all(h);
    delete h;
    return st;
  };
  if (hipGetDevice(&h->device) != hipSuccess) return bail(fail(DT_EHIP, "hipGetDevice failed"));
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, h->device) != hipSuccess) return bail(fail(DT_EHIP, "no device properties"));
  h->n_cu = prop.multiProcessorCount;
  if (!prop.cooperativeLaunch) return bail(fail(DT_EUNSUPPORTED, "device lacks cooperative launch"));
  {
    const dt_status st = scratch_setup(h->device);  // the allocation-free entry point's workspace
    if (st != DT_OK) return bail(st);
  }

  const int V = dims->vocab, D = dims->depths, hd = dims->hidden, e = dims->emb_dim, ds = dims->state_dim,
            r = dims->rank, Bm = dims->max_batch;
  const int M = maxp->top_m, N = maxp->budget;
  const size_t esz = h->esz;
  const int rows_p = round_up(3 * ds + r, 16), kp = round_up(ds, 32);
  h->n_tiles = rows_p / 16;
  if (h->n_tiles + 1 > h->n_cu * 64) return bail(fail(DT_EUNSUPPORTED, "state_dim too large"));

#define ALLOC(p, bytes)                 \
  do {                                  \
    dt_status st_ = dalloc(&(p), bytes); \
    if (st_ != DT_OK) return bail(st_); \
  } while (0)
#define HIPB(expr)                                                                               \
  do {                                                                                           \
    hipError_t e_ = (expr);                                                                      \
    if (e_ != hipSuccess) return bail(fail(DT_EHIP, "%s: %s", #expr, hipGetErrorString(e_))); \
  } while (0)

  // G = E W_ih^T + b_ih: the GRU input term of every token
  ALLOC(h->G, (size_t)V * 3 * ds * sizeof(float));
  if (h->bf16)
    HIPB(dt::launch_gemm_bf16((const uint16_t*)w->emb, nullptr, (const uint16_t*)w->w_ih, w->b_ih, h->G, V,
                              3 * ds, e, 3 * ds, stream));
  else
    HIPB(dt::launch_gemm_f32((const float*)w->emb, nullptr, (const float*)w->w_ih, w->b_ih, h->G, V, 3 * ds, e,
                             3 * ds, stream));
  ALLOC(h->tiles, (size_t)rows_p * kp * esz);
  HIPB(dt::launch_pack_node_tiles(w->w_hh, w->w1, hd, ds, r, (int)esz, h->tiles, stream));
  if (w->b_hh) {
    ALLOC(h->b_hh, (size_t)3 * ds * sizeof(float));
    HIPB(hipMemcpyAsync(h->b_hh, w->b_hh, (size_t)3 * ds * sizeof(float), hipMemcpyDeviceToDevice, stream));
  }
  ALLOC(h->w1h_t, (size_t)r * hd * esz);
  HIPB(dt::launch_transpose(w->w1, h->w1h_t, hd, r, (int)esz, stream));  // rows 0..h-1 of W1
  ALLOC(h->w2t, (size_t)V * r * esz);
  HIPB(dt::launch_transpose(w->w2, h->w2t, r, V, (int)esz, stream));
  if (w->w_lm) {
    if (!h->bf16) return bail(fail(DT_EUNSUPPORTED, "the LM head needs bf16 weights"));
    if (dt::gemm_b_tiles_ok(V, hd)) {
      // W_lm in the LM-head GEMM's tile order: each k stage of a 256-column
      // tile is one contiguous 16 KB piece
      h->wlm_tiled = true;
      ALLOC(h->wlm_t, dt::gemm_b_tiles_elems(V, hd) * esz);
      ALLOC(h->a_tiles, dt::gemm_a_tiles_elems(Bm * D, hd) * esz);
      HIPB(dt::launch_pack_b_tiles((const uint16_t*)w->w_lm, (uint16_t*)h->wlm_t, hd, V, stream));
    } else {
      ALLOC(h->wlm_t, (size_t)V * hd * esz);
      HIPB(dt::launch_transpose(w->w_lm, h->wlm_t, hd, V, (int)esz, stream));
    }
  }

  // the chain head's row-major [W_hh ; W1_S^T] and its workspace
  ALLOC(h->wc_rm, (size_t)(3 * ds + r) * ds * esz);
  HIPB(hipMemcpyAsync(h->wc_rm, w->w_hh, (size_t)3 * ds * ds * esz, hipMemcpyDeviceToDevice, stream));
  HIPB(dt::launch_transpose((const char*)w->w1 + (size_t)hd * r * esz, (char*)h->wc_rm + (size_t)3 * ds * ds * esz,
                            ds, r, (int)esz, stream));
  if (h->bf16 && r % 16 == 0 && r <= dt::CHAIN_MAX_RANK) {
    ALLOC(h->w2f, dt::chain_w2_frags_elems(V, r) * esz);
    HIPB(dt::launch_pack_w2_frags((const uint16_t*)h->w2t, (uint16_t*)h->w2f, V, r, stream));
  }
  ALLOC(h->chain_gu, (size_t)Bm * (3 * ds + r) * sizeof(float));
  ALLOC(h->chain_s, (size_t)Bm * ds * sizeof(float));
  ALLOC(h->chain_sop, (size_t)Bm * ds * esz);
  ALLOC(h->chain_part, (size_t)Bm * std::max(dt::chain_blocks(V), dt::chain_mfma_blocks(V)) * sizeof(uint64_t));

  // workspace for max_batch and max_params
  const int S = dt::topm_chunks(V);
  const size_t rows = (size_t)Bm * D;
  if (h->wlm_t) ALLOC(h->logits, rows * V * sizeof(float));
  if (h->wlm_tiled && dt::lm_topm_ok((int)rows, V, hd, M)) {
    const size_t nl = (size_t)dt::lm_lists_per_row(V);
    ALLOC(h->lm_lists, rows * nl * 8 * sizeof(uint64_t));
    ALLOC(h->lm_stats, rows * nl * sizeof(float2));
  }
  ALLOC(h->chunk_cand, rows * S * M * sizeof(uint64_t));
  ALLOC(h->chunk_stat, rows * S * sizeof(float4));
  ALLOC(h->cand_ids, rows * M * sizeof(int32_t));
  ALLOC(h->cand_vals, rows * M * sizeof(float));
  ALLOC(h->tokrank, rows * M * sizeof(int32_t));
  ALLOC(h->lse, rows * sizeof(float));
  ALLOC(h->tail, rows * sizeof(float));
  ALLOC(h->P, (size_t)dt::P_KSPLIT * rows * r * sizeof(float));  // partials of P (the candidate merge's)
  // exchange slots: at most N + 1 steps of at most TREE_MAX_COLS expanded nodes
  const size_t nodes = (size_t)(N + 1) * dt::TREE_MAX_COLS;
  ALLOC(h->state, nodes * round_up(ds, 32) * sizeof(float));
  h->act_bytes = nodes * round_up(ds, 64) * esz;
  ALLOC(h->act, h->act_bytes);
  HIPB(hipMemsetAsync(h->act, 0, h->act_bytes, stream));
  ALLOC(h->gh, nodes * round_up(3 * ds, 32) * sizeof(float));
  ALLOC(h->u, nodes * round_up(r, 32) * sizeof(float));
  // node entries: one more step than the slots (a finished request's last entries)
  const size_t ninfo_n = nodes + dt::TREE_MAX_COLS;
  ALLOC(h->ninfo, ninfo_n * sizeof(uint64_t));
  HIPB(hipMemsetAsync(h->ninfo, 0, ninfo_n * sizeof(uint64_t), stream));
  h->ninfo_words = ninfo_n * 2;
  h->max_workers = h->n_cu;
  ALLOC(h->mbox_w, (dt::GFLAG_WORDS + (size_t)h->max_workers * 32) * sizeof(uint32_t));
  ALLOC(h->mbox_c, (size_t)DT_MAX_BATCH * 256 * sizeof(uint32_t));
  ALLOC(h->err, 64);
  ALLOC(h->nanflag, 64);
  HIPB(hipMemsetAsync(h->err, 0, 64, stream));
  HIPB(hipHostMalloc(reinterpret_cast<void**>(&h->err_host), 64, hipHostMallocCoherent));
  *reinterpret_cast<volatile int*>(h->err_host) = 0;
  HIPB(hipMemsetAsync(h->mbox_w, 0, (dt::GFLAG_WORDS + (size_t)h->max_workers * 32) * sizeof(uint32_t), stream));
  HIPB(hipMemsetAsync(h->mbox_c, 0, (size_t)DT_MAX_BATCH * 256 * sizeof(uint32_t), stream));
  for (auto& set : h->ev)
    for (hipEvent_t& ev : set) HIPB(hipEventCreate(&ev));
  HIPB(hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking));  // default priority
  HIPB(hipEventCreateWithFlags(&h->fork_ev, hipEventDisableTiming));
  HIPB(hipEventCreateWithFlags(&h->join_ev, hipEventDisableTiming));
  HIPB(hipStreamSynchronize(stream));
#undef ALLOC
#undef HIPB
  *out = h;
  return DT_OK;
}

dt_status dt_build_trees(dt_handle* h, const dt_inputs* in, const dt_params* p, dt_outputs* out, void* stream_) {
  if (!h || !in || !p || !out) return fail(DT_EINVAL, "h, in, p and out are required");
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  const dt_dims& d = h->dims;
  dt_status s = check_params(p, d.vocab, &h->maxp);
  if (s != DT_OK) return s;
  if (in->batch < 1 || in->batch > d.max_batch)
    return fail(DT_EINVAL, "batch %d outside 1..%d", in->batch, d.max_batch);
  if (!in->hidden) return fail(DT_EINVAL, "inputs.hidden is required");
  if (!out->tokens || !out->parents || !out->depths || !out->scores || !out->n_nodes)
    return fail(DT_EINVAL, "tokens, parents, depths, scores and n_nodes outputs are required");
  if (!in->base_logits && !h->wlm_t) return fail(DT_EINVAL, "no base logits and no LM head weights");
  if (h->bf16 && !(p->flags & DT_ACT_BF16))
    return fail(DT_EUNSUPPORTED, "bf16 weights need DT_ACT_BF16 (bf16 GEMM operands)");
  // a finished launch that ended with the device error word set (the mirror
  // is read without a synchronisation; dt_sync_status reports and clears it)
  if (const int e = *reinterpret_cast<volatile int*>(h->err_host))
    return fail(DT_EDEVICE, "a previous build ended with a device error (word %d: %s); dt_sync_status resets the handle",
                e, device_error_text(e).c_str());

  const int B = in->batch, D = d.depths, V = d.vocab, M = p->top_m, N = p->budget;
  const int rows = B * D;
  const bool timing = (p->flags & DT_TIMING) != 0;
  hipEvent_t* evs = h->ev[h->timed % dt_handle::RING];
#define MARK(i) \
  if (timing) HIPCHK(hipEventRecord(evs[i], stream))

  if ((p->flags & DT_VALIDATE) && in->base_logits) {
    HIPCHK(hipMemsetAsync(h->nanflag, 0, sizeof(int), stream));
    HIPCHK(dt::launch_nan_scan(in->base_logits, (size_t)rows * V, h->nanflag, stream));
    int flag = 0;
    HIPCHK(hipMemcpyAsync(&flag, h->nanflag, sizeof(int), hipMemcpyDeviceToHost, stream));
    HIPCHK(hipStreamSynchronize(stream));
    if (flag) return fail(DT_EINVAL, "base logits contain NaN");
  }

  // a2: P = H W1_H (the path-independent half of W1 [H_d; S]) needs only the
  // hidden states.  Beside the LM-head GEMM (on the handle's side stream) it
  // costs nothing; with base logits given it runs first on the caller's
  // stream (measured: first is faster per round than on the side stream
  // beside the whole candidate selection or beside its merge alone)
  MARK(0);
  const bool p_inline = in->base_logits != nullptr;
  // bf16 with base logits given: P runs in extra blocks of the candidate
  // selection's launch, beside it
  const bool p_in_topm = p_inline && h->bf16;
  hipStream_t ps = p_inline ? stream : h->side;
  if (!p_inline) {
    HIPCHK(hipEventRecord(h->fork_ev, stream));
    HIPCHK(hipStreamWaitEvent(h->side, h->fork_ev, 0));
  }
  if (h->bf16 && !p_in_topm)
    HIPCHK(dt::launch_gemm_bf16((const uint16_t*)in->hidden, nullptr, (const uint16_t*)h->w1h_t, nullptr, h->P,
                                rows, d.rank, d.hidden, d.rank, ps));
  else if (!h->bf16)
    HIPCHK(dt::launch_gemm_f32((const float*)in->hidden, nullptr, (const float*)h->w1h_t, nullptr, h->P, rows,
                               d.rank, d.hidden, d.rank, ps));
  if (!p_inline) HIPCHK(hipEventRecord(h->join_ev, h->side));
  // a0 (LM head, when no base logits are given), then a1: candidates and LSE
  if (!in->base_logits && h->lm_lists) {
    // L_base = H W_lm (Domino summary, 方法步骤详情), fp32 accumulate, with
    // each depth's candidates taken in the GEMM's epilogue: the logits reach
    // memory only when the caller asks for a copy
    HIPCHK(dt::launch_lm_topm_gemm((const uint16_t*)in->hidden, (const uint16_t*)h->wlm_t, rows, V, d.hidden,
                                   h->a_tiles, p->temperature, h->lm_lists, h->lm_stats, out->logits, stream));
    MARK(1);
    HIPCHK(dt::launch_lm_select(h->lm_lists, h->lm_stats, rows, V, d.hidden, M, p->temperature,
                                (const uint16_t*)in->hidden, (const uint16_t*)h->wlm_t, h->cand_ids, h->cand_vals,
                                h->lse, h->tail, h->tokrank, out->cand_ids, out->cand_logits, out->lse, out->logits,
                                h->err, stream));
  } else {
    // the LM head's logits go to the caller's copy when one is asked for
    float* lm_logits = out->logits ? out->logits : h->logits;
    if (!in->base_logits) {
      if (h->wlm_tiled)
        HIPCHK(dt::launch_gemm_bf16_btiled((const uint16_t*)in->hidden, (const uint16_t*)h->wlm_t, lm_logits, rows,
                                           V, d.hidden, V, h->a_tiles, stream));
      else
        HIPCHK(dt::launch_gemm_bf16((const uint16_t*)in->hidden, nullptr, (const uint16_t*)h->wlm_t, nullptr,
                                    lm_logits, rows, V, d.hidden, V, stream));
    }
    MARK(1);
    const float* logits = in->base_logits ? in->base_logits : lm_logits;
    HIPCHK(dt::launch_topm(logits, rows, V, M, p->temperature, h->chunk_cand, h->chunk_stat, h->cand_ids,
                           h->cand_vals, h->lse, h->tail, h->tokrank, out->cand_ids, out->cand_logits, out->lse,
                           stream, p_in_topm ? (const uint16_t*)in->hidden : nullptr, (const uint16_t*)h->w1h_t,
                           h->P, d.rank, d.hidden));
  }
  // join: what P adds after the candidates are done
  MARK(2);
  if (!p_inline) HIPCHK(hipStreamWaitEvent(stream, h->join_ev, 0));

  // a3-a8: the persistent builder
  dt::TreeArgs a{};
  a.B = B;
  a.D = D;
  a.ds = d.state_dim;
  a.r = d.rank;
  a.M = M;
  a.k = p->top_k;
  a.N = N;
  a.T = p->temperature;
  a.fullv = p->norm == DT_NORM_FULLV;
  a.act_bf16 = (p->flags & DT_ACT_BF16) != 0;
  a.marginal = (p->flags & DT_MARGINAL) != 0;
  a.dlfma = h->sched.dl;
  a.n_tiles = h->n_tiles;
  a.tiles_per_worker = choose_tpw(h, B);
  a.n_workers = (h->n_tiles + a.tiles_per_worker - 1) / a.tiles_per_worker;
  if (a.n_workers + B > h->n_cu || a.n_workers > h->max_workers)
    return fail(DT_EUNSUPPORTED, "%d workers + %d requests exceed %d compute units", a.n_workers, B, h->n_cu);
  a.tiles = h->tiles;
  a.b_hh = h->b_hh;
  a.G = h->G;
  a.w2t = h->w2t;
  a.P = h->P;
  a.p_parts = p_in_topm ? dt::P_KSPLIT : 1;
  a.p_stride = (size_t)rows * d.rank;
  a.cand_ids = h->cand_ids;
  a.cand_vals = h->cand_vals;
  a.tail = h->tail;
  a.tokrank = h->tokrank;
  a.root = in->root_state;
  a.state = h->state;
  a.act = h->act;
  a.gh = h->gh;
  a.u = h->u;
  a.ninfo = h->ninfo;
  a.gflag = h->mbox_w;
  a.ready = h->mbox_w + 16 * 64;
  a.xccw = h->mbox_w + 16 * 64 + 64;
  a.mbox_w = h->mbox_w + dt::GFLAG_WORDS;
  a.mbox_c = h->mbox_c;
  a.err = h->err;
  a.err_host = h->err_host;
  a.tokens = out->tokens;
  a.parents = out->parents;
  a.depths = out->depths;
  a.scores = out->scores;
  a.n_nodes = out->n_nodes;
  a.stats = out->stats;
  a.spin_limit = 1u << 21;
  const size_t lds = dt::plan_tree(a, h->bf16, h->sched.pops, std::min(h->n_cu - B, h->max_workers),
                                   h->sched.lds_workers, h->sched.halves, h->sched.advance == 2,
                                   h->sched.exchange == 1);
  if (lds == 0 || lds > 160 * 1024) return fail(DT_EUNSUPPORTED, "no builder schedule fits this shape in LDS");
  if (a.marginal) a.n_workers = 0;  // marginal scores need no per-node products: controllers only
  if (a.n_workers + B > h->n_cu || a.n_workers > h->max_workers)
    return fail(DT_EUNSUPPORTED, "%d workers + %d requests exceed %d compute units", a.n_workers, B, h->n_cu);
  MARK(3);
  // mailboxes keep older epochs; clear them only when the epoch space wraps
  const uint32_t span = dt::tree_epoch_span(a.N);
  if (h->ebase + span >= dt::TREE_EPOCH_LIMIT) {
    HIPCHK(dt::launch_fill_u32(h->mbox_w, 0u, dt::GFLAG_WORDS + (size_t)h->max_workers * 32, stream));
    HIPCHK(dt::launch_fill_u32(h->mbox_c, 0u, (size_t)DT_MAX_BATCH * 256, stream));
    HIPCHK(dt::launch_fill_u32(reinterpret_cast<uint32_t*>(h->ninfo), 0u, h->ninfo_words, stream));
    h->ebase = 0;
  }
  a.ebase = h->ebase;
  h->ebase += span;
  MARK(4);
  HIPCHK(dt::launch_tree(a, h->bf16, lds, stream, h->sched.launch != 2));
  MARK(5);
  if (timing) ++h->timed;
#undef MARK
  return DT_OK;
}

dt_status dt_phase_times(dt_handle* h, float* ms, int n, int32_t* count) {
  if (!h || !ms || !count) return fail(DT_EINVAL, "h, ms and count are required");
  const int nb = h->timed < dt_handle::RING ? h->timed : dt_handle::RING;
  double sum[dt_handle::NPH] = {};
  for (int j = 0; j < nb; ++j) {
    hipEvent_t* evs = h->ev[(h->timed - 1 - j) % dt_handle::RING];
    HIPCHK(hipEventSynchronize(evs[dt_handle::NPH]));
    for (int i = 0; i < dt_handle::NPH; ++i) {
      float t = 0.f;
      HIPCHK(hipEventElapsedTime(&t, evs[i], evs[i + 1]));
      sum[i] += t;
    }
  }
  for (int i = 0; i < dt_handle::NPH && i < n; ++i) ms[i] = nb ? (float)(sum[i] / nb) : 0.f;
  *count = nb;
  h->timed = 0;
  return DT_OK;
}

dt_status dt_sync_status(dt_handle* h, void* stream_) {
  if (!h) return fail(DT_EINVAL, "h is NULL");
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  HIPCHK(hipStreamSynchronize(stream));
  int e = 0;
  HIPCHK(hipMemcpy(&e, h->err, sizeof(int), hipMemcpyDeviceToHost));
  if (!e) e = *reinterpret_cast<volatile int*>(h->err_host);
  if (!e) return DT_OK;
  // reset: clear the error word and its mirror, and re-base the epochs on
  // cleared mailboxes, so that the next build starts as on a new handle
  HIPCHK(dt::launch_fill_u32(reinterpret_cast<uint32_t*>(h->err), 0u, 16, stream));
  HIPCHK(dt::launch_fill_u32(h->mbox_w, 0u, dt::GFLAG_WORDS + (size_t)h->max_workers * 32, stream));
  HIPCHK(dt::launch_fill_u32(h->mbox_c, 0u, (size_t)DT_MAX_BATCH * 256, stream));
  HIPCHK(dt::launch_fill_u32(reinterpret_cast<uint32_t*>(h->ninfo), 0u, h->ninfo_words, stream));
  HIPCHK(hipStreamSynchronize(stream));
  h->ebase = 0;
  *reinterpret_cast<volatile int*>(h->err_host) = 0;
  return fail(DT_EDEVICE, "a build ended with a device error (word %d: %s); the handle is reset", e,
              device_error_text(e).c_str());
}

dt_status dt_set_schedule(dt_handle* h, const dt_schedule* s) {
  if (!h) return fail(DT_EINVAL, "h is NULL");
  if (!s) {
    h->sched = dt_schedule{};
    return DT_OK;
  }
  if (s->pops < 0 || s->pops > 16) return fail(DT_EINVAL, "pops %d outside 0..16", s->pops);
  if (s->halves < 0 || s->halves > 2) return fail(DT_EINVAL, "halves %d outside 0..2", s->halves);
  if (s->lds_workers != 0 && s->lds_workers != 1) return fail(DT_EINVAL, "lds_workers must be 0 or 1");
  if (s->tiles_per_worker < 0 || s->tiles_per_worker > 64)
    return fail(DT_EINVAL, "tiles_per_worker %d outside 0..64", s->tiles_per_worker);
  if (s->advance < 0 || s->advance > 2) return fail(DT_EINVAL, "advance %d outside 0..2", s->advance);
  if (s->dl != 0 && s->dl != 1) return fail(DT_EINVAL, "dl must be 0 or 1");
  if (s->launch < 0 || s->launch > 2) return fail(DT_EINVAL, "launch %d outside 0..2", s->launch);
  if (s->exchange < 0 || s->exchange > 1) return fail(DT_EINVAL, "exchange %d outside 0..1", s->exchange);
  h->sched = *s;
  return DT_OK;
}

dt_status dt_set_device_error(dt_handle* h, int32_t code, void* stream) {
  if (!h) return fail(DT_EINVAL, "h is NULL");
  if (code <= 0) return fail(DT_EINVAL, "code %d must be positive", code);
  HIPCHK(dt::launch_fill_u32(reinterpret_cast<uint32_t*>(h->err), (uint32_t)code, 1,
                             reinterpret_cast<hipStream_t>(stream)));
  return DT_OK;
}

dt_status dt_destroy(dt_handle* h) {
  if (!h) return DT_OK;
  (void)hipDeviceSynchronize();
  free_all(h);
  delete h;
  return DT_OK;
}

}  // extern "C"

namespace {

dt_status chain_check(const dt_handle* h, const dt_inputs* in, uint32_t flags, const int32_t* tokens) {
  if (!h || !in || !tokens) return fail(DT_EINVAL, "h, in and tokens are required");
  const dt_dims& d = h->dims;
  if (in->batch < 1 || in->batch > d.max_batch)
    return fail(DT_EINVAL, "batch %d outside 1..%d", in->batch, d.max_batch);
  if (!in->hidden) return fail(DT_EINVAL, "hidden is required");
  if (!in->base_logits && !h->wlm_t) return fail(DT_EINVAL, "no base logits and no LM head weights");
  if (flags & ~(uint32_t)DT_ACT_BF16) return fail(DT_EINVAL, "unknown flags 0x%x", flags);
  if (h->bf16 && !(flags & DT_ACT_BF16))
    return fail(DT_EUNSUPPORTED, "bf16 weights need DT_ACT_BF16 (bf16 GEMM operands)");
  if (!h->bf16 && (flags & DT_ACT_BF16)) return fail(DT_EUNSUPPORTED, "DT_ACT_BF16 needs bf16 weights");
  if (d.rank > dt::CHAIN_MAX_RANK || d.rank % 8)
    return fail(DT_EUNSUPPORTED, "the chain head needs rank <= %d and a multiple of 8", dt::CHAIN_MAX_RANK);
  return DT_OK;
}

// Sampling parameters of a chain (sample 0: the greedy pick)
struct ChainDraw {
  int sample = 0;
  float temperature = 1.f;
  uint64_t seed = 0;
};

// The chain head on a given workspace (P [B D, r], gu [B, 3 ds + r], s [B, ds],
// s_op [B, ds], part [B, chain blocks]): P = H W1_H, then the positions.
dt_status chain_run(const dt_handle* h, const dt_inputs* in, const float* base, int32_t* tokens, float* logits,
                    float* P, float* gu, float* s, void* s_op, uint64_t* part, hipStream_t stream,
                    const ChainDraw& draw = ChainDraw{}) {
  const dt_dims& d = h->dims;
  const int rows = in->batch * d.depths;
  // P = H W1_H for every position (the path-independent half of W1 [H_d; S])
  if (h->bf16)
    HIPCHK(dt::launch_gemm_bf16((const uint16_t*)in->hidden, nullptr, (const uint16_t*)h->w1h_t, nullptr, P, rows,
                                d.rank, d.hidden, d.rank, stream));
  else
    HIPCHK(dt::launch_gemm_f32((const float*)in->hidden, nullptr, (const float*)h->w1h_t, nullptr, P, rows, d.rank,
                               d.hidden, d.rank, stream));
  dt::ChainArgs c{};
  c.B = in->batch;
  c.D = d.depths;
  c.V = d.vocab;
  c.ds = d.state_dim;
  c.r = d.rank;
  c.bf16 = h->bf16;
  c.w2t = h->w2t;
  c.w2f = h->w2f;
  c.wc = h->wc_rm;
  c.G = h->G;
  c.b_hh = h->b_hh;
  c.base = base;
  c.P = P;
  c.root = in->root_state;
  c.gu = gu;
  c.s = s;
  c.s_op = s_op;
  c.part = part;
  c.tokens = tokens;
  c.logits = logits;
  c.sample = draw.sample;
  c.temperature = draw.temperature;
  c.key0 = (uint32_t)(draw.seed & 0xFFFFFFFFu);
  c.key1 = (uint32_t)(draw.seed >> 32);
  HIPCHK(dt::launch_chain(c, stream));
  return DT_OK;
}

// The base logits of a chain call: the caller's, or H W_lm into the handle's
// logits workspace
dt_status chain_base(dt_handle* h, const dt_inputs* in, hipStream_t stream, const float** base) {
  const dt_dims& d = h->dims;
  const int V = d.vocab, rows = in->batch * d.depths;
  if (!in->base_logits) {
    if (h->wlm_tiled)
      HIPCHK(dt::launch_gemm_bf16_btiled((const uint16_t*)in->hidden, (const uint16_t*)h->wlm_t, h->logits, rows, V,
                                         d.hidden, V, h->a_tiles, stream));
    else
      HIPCHK(dt::launch_gemm_bf16((const uint16_t*)in->hidden, nullptr, (const uint16_t*)h->wlm_t, nullptr,
                                  h->logits, rows, V, d.hidden, V, stream));
  }
  *base = in->base_logits ? in->base_logits : h->logits;
  return DT_OK;
}

}  // namespace

extern "C" {

dt_status dt_draft_chain(dt_handle* h, const dt_inputs* in, uint32_t flags, int32_t* tokens, float* logits,
                         void* stream_) {
  dt_status st = chain_check(h, in, flags, tokens);
  if (st != DT_OK) return st;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  const float* base = nullptr;
  if ((st = chain_base(h, in, stream, &base)) != DT_OK) return st;
  return chain_run(h, in, base, tokens, logits, h->P, h->chain_gu, h->chain_s, h->chain_sop, h->chain_part, stream);
}

dt_status dt_draft_chain_sample(dt_handle* h, const dt_inputs* in, uint32_t flags, float temperature, uint64_t seed,
                                int32_t* tokens, float* logits, void* stream_) {
  dt_status st = chain_check(h, in, flags, tokens);
  if (st != DT_OK) return st;
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(DT_EINVAL, "temperature %g is not positive and finite", (double)temperature);
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  const float* base = nullptr;
  if ((st = chain_base(h, in, stream, &base)) != DT_OK) return st;
  ChainDraw draw;
  draw.sample = 1;
  draw.temperature = temperature;
  draw.seed = seed;
  return chain_run(h, in, base, tokens, logits, h->P, h->chain_gu, h->chain_s, h->chain_sop, h->chain_part, stream,
                   draw);
}

dt_status dt_draft_chain_noalloc(dt_handle* h, const dt_inputs* in, uint32_t flags, int32_t* tokens, float* logits,
                                 void* stream_) {
  dt_status st = chain_check(h, in, flags, tokens);
  if (st != DT_OK) return st;
  if (!in->base_logits)
    return fail(DT_EINVAL, "dt_draft_chain_noalloc needs base logits (the LM head's logits do not fit its scratch)");
  const dt_dims& d = h->dims;
  const int B = in->batch;
  // the workspace, carved from the device's scratch array in 256-byte pieces
  const size_t a = 256;
  auto piece = [a](size_t bytes) { return (bytes + a - 1) / a * a; };
  const size_t p_bytes = piece((size_t)B * d.depths * d.rank * sizeof(float));
  const size_t gu_bytes = piece((size_t)B * (3 * d.state_dim + d.rank) * sizeof(float));
  const size_t s_bytes = piece((size_t)B * d.state_dim * sizeof(float));
  const size_t sop_bytes = piece((size_t)B * d.state_dim * h->esz);
  const size_t part_bytes =
      piece((size_t)B * std::max(dt::chain_blocks(d.vocab), dt::chain_mfma_blocks(d.vocab)) * sizeof(uint64_t));
  const size_t total = p_bytes + gu_bytes + s_bytes + sop_bytes + part_bytes;
  if (total > DT_NOALLOC_SCRATCH_BYTES)
    return fail(DT_EUNSUPPORTED, "batch %d needs %zu bytes of scratch, more than the %u the library holds", B, total,
                (unsigned)DT_NOALLOC_SCRATCH_BYTES);
  unsigned char* base = scratch_of(h->device);
  if (!base) return fail(DT_EHIP, "no scratch address for device %d", h->device);
  float* P = reinterpret_cast<float*>(base);
  float* gu = reinterpret_cast<float*>(base + p_bytes);
  float* s = reinterpret_cast<float*>(base + p_bytes + gu_bytes);
  void* s_op = base + p_bytes + gu_bytes + s_bytes;
  uint64_t* part = reinterpret_cast<uint64_t*>(base + p_bytes + gu_bytes + s_bytes + sop_bytes);
  return chain_run(h, in, in->base_logits, tokens, logits, P, gu, s, s_op, part, reinterpret_cast<hipStream_t>(stream_));
}

dt_status dt_fold_state(dt_handle* h, int32_t batch, int32_t n_tokens, const int32_t* tokens,
                        const float* prev_state, float* state_out, uint32_t flags, void* stream) {
  if (!h || !tokens || !state_out) return fail(DT_EINVAL, "h, tokens and state_out are required");
  if (batch < 1 || batch > h->dims.max_batch)
    return fail(DT_EINVAL, "batch %d outside 1..%d", batch, h->dims.max_batch);
  if (n_tokens < 1) return fail(DT_EINVAL, "n_tokens %d < 1", n_tokens);
  if (flags & ~(uint32_t)DT_ACT_BF16) return fail(DT_EINVAL, "unknown flags 0x%x", flags);
  if (h->bf16 && !(flags & DT_ACT_BF16))
    return fail(DT_EUNSUPPORTED, "bf16 weights need DT_ACT_BF16 (bf16 GEMM operands)");
  if (!h->bf16 && (flags & DT_ACT_BF16)) return fail(DT_EUNSUPPORTED, "DT_ACT_BF16 needs bf16 weights");
  dt::ChainArgs c{};
  c.B = batch;
  c.V = h->dims.vocab;
  c.ds = h->dims.state_dim;
  c.r = h->dims.rank;
  c.bf16 = h->bf16;
  c.wc = h->wc_rm;
  c.G = h->G;
  c.b_hh = h->b_hh;
  c.root = prev_state;
  c.gu = h->chain_gu;
  c.s = h->chain_s;
  c.s_op = h->chain_sop;
  HIPCHK(dt::launch_fold(c, tokens, n_tokens, state_out, reinterpret_cast<hipStream_t>(stream)));
  return DT_OK;
}

dt_status dt_tree_attention_inputs(const dt_tree_view* trees, const dt_verify_outputs* out, void* stream) {
  if (!trees || !out) return fail(DT_EINVAL, "NULL trees or out");
  if (trees->batch < 1) return fail(DT_EINVAL, "batch %d < 1", trees->batch);
  if (trees->cols < 1) return fail(DT_EINVAL, "cols %d < 1", trees->cols);
  if (trees->cols > DT_MAX_BUDGET + 1)
    return fail(DT_EUNSUPPORTED, "cols %d > %d", trees->cols, DT_MAX_BUDGET + 1);
  if (!trees->parents || !trees->depths || !trees->n_nodes) return fail(DT_EINVAL, "NULL parents, depths or n_nodes");
  if (!out->mask || !out->positions) return fail(DT_EINVAL, "NULL mask or positions");
  if (out->tokens && !trees->tokens) return fail(DT_EINVAL, "flattened tokens need the trees' tokens");
  HIPCHK(dt::launch_tree_attention(trees->batch, trees->cols, trees->parents, trees->depths, trees->tokens,
                                   trees->n_nodes, trees->prefix_len, trees->anchor, out->mask, out->positions,
                                   out->tokens, out->bad, (hipStream_t)stream));
  return DT_OK;
}

}  // extern "C"
