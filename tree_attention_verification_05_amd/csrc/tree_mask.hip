// Ancestor-or-self bitmask of every draft-tree node ("vLLM-TreeEagle" README,
// 核心组件 item 1: the tree attention mask is built at run time; 技术创新点 1:
// irregular trees).
//
// One workgroup per sequence; one thread per node walks from its node up to
// the root.  Parents strictly decrease along the walk, so it ends in at most
// N steps; a parent outside [0, i) marks the tree invalid.
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void tree_mask_kernel(const int32_t* __restrict__ parents,
                                                             int N, uint64_t* __restrict__ mask,
                                                             int32_t* __restrict__ depth,
                                                             int32_t* dev_status) {
  const int b = blockIdx.x;
  const int W = (N + 63) >> 6;
  const int32_t* par = parents + static_cast<size_t>(b) * N;
  __shared__ int s_par[TV_MAX_NODES];
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();

  // validity of the whole tree first, so that every row is either exact or
  // zero; the parents stay in LDS for the walks
  for (int i = threadIdx.x; i < N; i += kThreads) {
    const int p = par[i];
    s_par[i] = p;
    if (i == 0 ? p != -1 : (p < 0 || p >= i)) bad = 1;
  }
  __syncthreads();
  if (bad && threadIdx.x == 0) report(dev_status, TV_DEV_BAD_TREE);

  for (int i = threadIdx.x; i < N; i += kThreads) {
    uint64_t bits[TV_MAX_NODES / 64] = {0, 0, 0, 0};
    int d = 0;
    if (!bad) {
      int c = i;
      bits[c >> 6] |= 1ull << (c & 63);
      while (c != 0) {
        c = s_par[c];
        bits[c >> 6] |= 1ull << (c & 63);
        ++d;
      }
    }
    uint64_t* row = mask + (static_cast<size_t>(b) * N + i) * W;
    for (int w = 0; w < W; ++w) row[w] = bits[w];
    if (depth) depth[static_cast<size_t>(b) * N + i] = d;
  }
}

}  // namespace

hipError_t launch_tree_mask(const int32_t* parents, int B, int N, uint64_t* mask, int32_t* depth,
                            int32_t* dev_status, hipStream_t stream) {
  hipLaunchKernelGGL(tree_mask_kernel, dim3(B), dim3(kThreads), 0, stream, parents, N, mask, depth,
                     dev_status);
  return hipGetLastError();
}

}  // namespace tv
