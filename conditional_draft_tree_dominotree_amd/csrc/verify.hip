// Tree-attention inputs of built draft trees: the ancestor mask, position ids
// and flattened tokens that verification needs ("Riassunto Tecnico:
// DominoTree", Componenti Core 5: the tree is verified with the standard tree
// attention of DDTree/SpecInfer, a causal mask built from each node's
// ancestors).
//
// One block per tree.  The tree's parents are staged in LDS; each thread
// builds 32-column words of the mask (node i, word w: walk i's path to the
// root and keep the nodes in columns 32 w .. 32 w + 31), so consecutive
// threads write consecutive words of a row.  Walks follow strictly
// decreasing node indices and stop at the first step that does not, so every
// walk ends; such a tree is reported in `bad`.
#include "common.h"
#include "kernels.h"

namespace dt {

constexpr int VT = 256;

__global__ __launch_bounds__(VT) void tree_attention_kernel(int cols, const int32_t* __restrict__ parents,
                                                            const int32_t* __restrict__ depths,
                                                            const int32_t* __restrict__ tokens,
                                                            const int32_t* __restrict__ n_nodes,
                                                            const int32_t* __restrict__ prefix_len,
                                                            const int32_t* __restrict__ anchor,
                                                            uint32_t* __restrict__ mask, int32_t* __restrict__ positions,
                                                            int32_t* __restrict__ flat, int32_t* __restrict__ bad) {
  __shared__ int32_t par[DT_VERIFY_MAX_COLS];
  __shared__ int flag;
  const int b = blockIdx.x, tid = threadIdx.x;
  const size_t row0 = (size_t)b * cols;
  const int words = (cols + 31) >> 5;
  const int nn = n_nodes[b];
  const int n = min(max(nn, 0), cols - 1);
  if (tid == 0) flag = (nn < 0 || nn > cols - 1) ? 1 : 0;
  for (int i = tid; i < cols; i += VT) par[i] = parents[row0 + i];
  __syncthreads();

  // mask words: (node i, word w) for every row, zero past n
  uint32_t* mrow = mask + row0 * words;
  for (int t = tid; t < cols * words; t += VT) {
    const int i = t / words, w = t - i * words;
    uint32_t bits = 0;
    if (i <= n) {
      int j = i;
      while (true) {
        if ((j >> 5) == w) bits |= 1u << (j & 31);
        const int p = par[j];
        if (j == 0 || !(p >= 0 && p < j)) break;
        j = p;
      }
    }
    mrow[t] = bits;
  }
  // positions, flattened tokens and the tree checks, one thread per node
  const int pre = prefix_len ? prefix_len[b] : 0;
  const int anc = anchor ? anchor[b] : -1;
  for (int i = tid; i < cols; i += VT) {
    int pos = -1, tok = -1;
    if (i <= n) {
      const int d = depths[row0 + i];
      int j = i, steps = 0, ok = 1;
      while (true) {
        const int p = par[j];
        if (j == 0) {
          ok = p == -1;
          break;
        }
        if (!(p >= 0 && p < j)) {
          ok = 0;
          break;
        }
        j = p;
        ++steps;
      }
      if (!ok || steps != d) flag = 1;  // benign race: every writer stores 1
      pos = pre + d;
      tok = i == 0 ? anc : (tokens ? tokens[row0 + i] : -1);
    }
    positions[row0 + i] = pos;
    if (flat) flat[row0 + i] = tok;
  }
  __syncthreads();
  if (tid == 0 && bad) bad[b] = flag;
}

hipError_t launch_tree_attention(int batch, int cols, const int32_t* parents, const int32_t* depths,
                                 const int32_t* tokens, const int32_t* n_nodes, const int32_t* prefix_len,
                                 const int32_t* anchor, uint32_t* mask, int32_t* positions, int32_t* flat,
                                 int32_t* bad, hipStream_t stream) {
  if (batch < 1 || cols < 1 || cols > DT_VERIFY_MAX_COLS) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tree_attention_kernel, dim3(batch), dim3(VT), 0, stream, cols, parents, depths, tokens,
                     n_nodes, prefix_len, anchor, mask, positions, flat, bad);
  return hipGetLastError();
}

}  // namespace dt
