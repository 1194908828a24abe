// Internal launch interface of the builder's kernels (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// limits shared with include/dominotree.h
#define DT_TOPM_MAX 64
#define DT_TOPM_MAX_CHUNKS 128   // vocab up to 128 * 8192 = 1048576
#define TOPM_CHUNK 8192

namespace dt {

inline int topm_chunks(int V) { return (V + TOPM_CHUNK - 1) / TOPM_CHUNK; }

// ---- per-depth candidates (topm.hip)
// With pA (bf16 [rows, pK]) given, the merge's launch also computes
// pC [rows, pN] = pA pBt^T (pBt bf16 [pN, pK]) in extra blocks: the per-round
// product P = H W1_H beside the candidate selection.
// P = H W1_H in the candidate merge's launch is written as P_KSPLIT partials
// [P_KSPLIT][rows, pN] (pC), which the consumer adds in order
constexpr int P_KSPLIT = 2;
hipError_t launch_topm(const float* logits, int rows, int V, int M, float T, uint64_t* chunk_cand,
                       float4* chunk_stat, int32_t* ids, float* vals, float* lse, float* tail,
                       int32_t* tokrank, int32_t* user_ids, float* user_vals, float* user_lse,
                       hipStream_t stream, const uint16_t* pA = nullptr, const uint16_t* pBt = nullptr,
                       float* pC = nullptr, int pN = 0, int pK = 0);
hipError_t launch_topm_merge(const uint64_t* chunk_cand, const float4* chunk_stat, int rows, int S,
                             int M, float T, int32_t* ids, float* vals, float* lse, float* tail,
                             int32_t* tokrank, int32_t* user_ids, float* user_vals, float* user_lse,
                             hipStream_t stream);
hipError_t launch_nan_scan(const float* x, size_t n, int* flag, hipStream_t stream);

// ---- dense products (gemm.hip)
// C[m, n] = sum_k A[rowsel(m), k] * Bt[n, k] (+ bias[n]); A row-major [*, K],
// Bt row-major [N, K]; rowsel = identity when `rows` is NULL.  fp32 output
// with leading dimension ldc.
hipError_t launch_gemm_bf16(const uint16_t* A, const int32_t* rows, const uint16_t* Bt, const float* bias,
                            float* C, int M, int N, int K, int ldc, hipStream_t stream);
// The same product with Bt pre-tiled by launch_pack_b_tiles (from W = Bt^T,
// [K, N] row-major); needs gemm_b_tiles_ok(N, K) (K a multiple of 64).  The
// tiled copy holds gemm_b_tiles_elems(N, K) bf16.
bool gemm_b_tiles_ok(int N, int K);
size_t gemm_b_tiles_elems(int N, int K);
hipError_t launch_pack_b_tiles(const uint16_t* W, uint16_t* out, int K, int N, hipStream_t stream);
// a_tiles (gemm_a_tiles_elems(M, K) bf16, required): A is first re-laid out
// there in the same tile order, so both operands load as contiguous pieces.
size_t gemm_a_tiles_elems(int M, int K);
hipError_t launch_gemm_bf16_btiled(const uint16_t* A, const uint16_t* Btiled, float* C, int M, int N, int K,
                                   int ldc, uint16_t* a_tiles, hipStream_t stream);
hipError_t launch_gemm_f32(const float* A, const int32_t* rows, const float* Bt, const float* bias,
                           float* C, int M, int N, int K, int ldc, hipStream_t stream);
// The LM head fused with the candidate selection (gemm.hip): the GEMM's
// epilogue writes, per row and per 128 columns, the 8 largest logits as
// (value, id) composites (lists [M, nl, 8]) and (max, sum of exp((x - max)/T))
// (stats [M, nl]), nl = lm_lists_per_row(N); user_logits (optional, [M, N])
// also gets the logits.  lm_select then gives each row's topM candidates,
// their values, the LSE of logits/T, the tail LSE and the token-id ranks, as
// launch_topm does; it reads A (bf16 [M, K]) and Btiled again only to
// recompute a list that may hide candidates.  Needs lm_topm_ok.
int lm_lists_per_row(int N);
bool lm_topm_ok(int M, int N, int K, int topM);
hipError_t launch_lm_topm_gemm(const uint16_t* A, const uint16_t* Btiled, int M, int N, int K, uint16_t* a_tiles,
                               float T, uint64_t* lists, float2* stats, float* user_logits, hipStream_t stream);
hipError_t launch_lm_select(const uint64_t* lists, const float2* stats, int rows, int N, int K, int topM, float T,
                            const uint16_t* hidden, const uint16_t* Btiled, int32_t* ids, float* vals, float* lse,
                            float* tail, int32_t* tokrank, int32_t* user_ids, float* user_vals, float* user_lse,
                            float* user_logits, int* err, hipStream_t stream);

// ---- tree-attention inputs (verify.hip)
constexpr int DT_VERIFY_MAX_COLS = 1025;  // budget + 1 at the largest budget
// One block per tree: the ancestor mask [batch, cols, ceil(cols / 32)] (bit
// j % 32 of word j / 32 of row i set when node j is i or an ancestor of i),
// positions [batch, cols] (prefix + depth), flattened tokens [batch, cols]
// (the anchor at node 0) and a per-tree flag for trees that break the
// builder's invariants.  tokens/flat, prefix_len, anchor and bad may be NULL.
hipError_t launch_tree_attention(int batch, int cols, const int32_t* parents, const int32_t* depths,
                                 const int32_t* tokens, const int32_t* n_nodes, const int32_t* prefix_len,
                                 const int32_t* anchor, uint32_t* mask, int32_t* positions, int32_t* flat,
                                 int32_t* bad, hipStream_t stream);

// ---- greedy chain head over the whole vocabulary (chain.hip)
constexpr int CHAIN_MAX_RANK = 256;
struct ChainArgs {
  int B, D, V, ds, r, bf16;  // bf16: weights and the state operand in bf16
  const void* w2t;      // [V, r] (wdtype)
  const void* w2f;      // bf16 W2^T in MFMA fragment order, or null (then the fp32-FMA kernel)
  const void* wc;       // [3 ds + r, ds] row-major: W_hh rows, then W1_S^T
  const float* G;       // [V, 3 ds] = E W_ih^T + b_ih
  const float* b_hh;    // [3 ds] or null
  const float* base;    // [B, D, V]
  const float* P;       // [B, D, r] = H W1_H
  const float* root;    // [B, ds] or null
  float* gu;            // [B, 3 ds + r] workspace
  float* s;             // [B, ds] workspace (state)
  void* s_op;           // [B, ds] workspace (state as a matrix operand, wdtype)
  uint64_t* part;       // [B, chain_blocks(V)] workspace
  int32_t* tokens;      // [B, D]
  float* logits;        // [B, D] or null
  // sampling: each position's token drawn by the Gumbel-max rule at
  // temperature `temperature`, the noise from Philox4x32-10 under key
  // (key0, key1); 0: the greedy pick
  int sample;
  float temperature;
  uint32_t key0, key1;
};
int chain_blocks(int V);       // blocks of the fp32 correction (one vocabulary row per thread)
int chain_mfma_blocks(int V);  // blocks of the bf16 MFMA correction
size_t chain_w2_frags_elems(int V, int r);
hipError_t launch_pack_w2_frags(const uint16_t* w2t, uint16_t* out, int V, int r, hipStream_t stream);
hipError_t launch_chain(const ChainArgs& c, hipStream_t stream);
// S <- GRU(S, E[t]) over tokens[b, 0..L-1] from c.root (zeros when null),
// written to out [B, ds]; uses c's weights and workspaces (gu, s, s_op).
hipError_t launch_fold(const ChainArgs& c, const int32_t* tokens, int L, float* out, hipStream_t stream);

// ---- weight re-layout (prepack.hip)
// out[c, r] = in[r, c] for a [R, C] matrix of 2- or 4-byte elements
hipError_t launch_transpose(const void* in, void* out, int R, int C, int elem_bytes, hipStream_t stream);
// Tiles of the per-node product [W_hh ; W1_S^T] ([3 ds + r] rows x ds) in the
// builder's LDS order: tile t = rows 16t..16t+15; within a tile, for each
// 32-wide k block, [k group 0..3][row 0..15] x 8 elements.
hipError_t launch_pack_node_tiles(const void* w_hh, const void* w1, int h, int ds, int r, int elem_bytes,
                                  void* out, hipStream_t stream);
hipError_t launch_fill_u32(uint32_t* p, uint32_t v, size_t n, hipStream_t stream);

}  // namespace dt

// the tree builder's arguments, schedule and launch (tree.hip)
#include "tree.h"
