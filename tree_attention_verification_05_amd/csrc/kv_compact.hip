// In-place compaction of the accepted path's K/V rows ("EAGLE代码实现原理",
// KV缓存优化: copy(indices, prev_length) selects the indexed rows and copies
// them to the rows from prev_length; "P-EAGLE", 技术难点和解决方案: the cache is
// rolled back to the accepted tokens).
//
// One workgroup per sequence.  Each thread owns 16-byte columns of a token's
// K/V (both caches, every KV head; a token's head h sits kv_head_rows rows
// after its head h - 1) and walks the
// path in ascending order, reading source rows before writing destinations.  For a strictly increasing path
// with path[j] >= j, a destination j is never the source of a later step, and
// the source path[j] of step j is rewritten (as destination) only by the later
// step j' = path[j], whose store follows this thread's load of it; so the
// in-order walk gives the same bytes as gathering every source first.
#include "kv_compact_rows.h"

namespace tv {
namespace {

constexpr int kThreads = 256;
static_assert(kThreads >= TV_MAX_NODES, "one path step per thread");

__global__ __launch_bounds__(kThreads) void kv_compact_kernel(CompactArgs a) {
  __shared__ long long s_src[TV_MAX_NODES];  // head-0 cache row of the source of step j
  __shared__ long long s_dst[TV_MAX_NODES];  // head-0 cache row of the destination of step j
  __shared__ int s_bad, s_L;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int N = a.N;
  const int32_t* table = a.block_table + static_cast<size_t>(b) * a.max_blocks;
  const int32_t* path = a.accepted_nodes + static_cast<size_t>(b) * N;
  // step tid's path entries go out together with the lengths (N <= kThreads)
  const int pj_me = tid < N ? path[tid] : 0;
  const int pj_prev = (tid >= 1 && tid < N) ? path[tid - 1] : 0;
  const int P = a.prefix_lens[b];
  const int L = a.accept_len[b] + 1;
  if (tid == 0) {
    s_bad = 0;
    s_L = L;
  }
  __syncthreads();
  int bad = 0;
  if (L < 1 || L > N) bad |= TV_DEV_BAD_TREE;
  if (P < 0 || static_cast<long>(P) + N > static_cast<long>(a.max_blocks) * kBlockSize) bad |= TV_DEV_BAD_CACHE;
  if (!bad) {
    for (int j = tid; j < L; j += kThreads) {
      const int pj = pj_me;
      const bool inc = (j == 0) ? (pj == 0) : (pj > pj_prev && pj < N);
      if (!inc) {
        bad |= TV_DEV_BAD_TREE;
        continue;
      }
      const int ts = P + pj, td = P + j;
      const int bs = table[ts / kBlockSize], bd = table[td / kBlockSize];
      if (bs < 0 || bs >= a.num_blocks || bd < 0 || bd >= a.num_blocks) {
        bad |= TV_DEV_BAD_CACHE;
        continue;
      }
      // the token's row at head 0
      s_src[j] = kv_row(bs, 0, ts % kBlockSize, a.Hkv, a.kv_head_rows, a.kv_slot_rows);
      s_dst[j] = kv_row(bd, 0, td % kBlockSize, a.Hkv, a.kv_head_rows, a.kv_slot_rows);
    }
  }
  if (bad) atomicOr(&s_bad, bad);
  __syncthreads();
  if (s_bad) {
    if (tid == 0) report(a.dev_status, s_bad);
    return;
  }
  if (tid == 0 && a.new_lens) a.new_lens[b] = P + L;

  compact_copy_columns(a, s_src, s_dst, s_L, tid, kThreads);
}

}  // namespace

hipError_t launch_kv_compact(const CompactArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(kv_compact_kernel, dim3(a.B), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tv
