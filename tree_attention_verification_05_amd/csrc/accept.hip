// Greedy verification of a draft tree against the target logits, one launch.
// ("P-EAGLE", 技术原理和实现方式 steps 3-4: the target scores every proposed
// token at once, drafts are accepted while they agree with it; "vLLM EAGLE
// 投机解码实战", 无损性保障: greedy speculative decoding equals greedy decoding.)
//
// Scan kernel (rows x chunks workgroups): one chunk of one logits row is read
// with 16-byte loads, four (two with 1024 threads) in flight per thread; the
// chunk's best (value, index) is packed into a 64-bit key that orders by
// value and then by lower index, and stored in the workspace.  No atomics and no fences: the kernel
// boundary orders the keys before their use.
// Walk kernel (one workgroup per sequence): reduce the chunk keys of the
// sequence's N rows to the target argmax, validate the tree and the draft
// tokens, and find the longest accepted path (smallest node sequence among
// equals).  The workspace needs no initialisation.
// With compaction fused (tv_accept_greedy_compact), the same workgroup then
// moves the accepted path's K/V rows into place: the prefix length and the
// block-table entries of the tree region are loaded with the tree, so once
// the path is known only the row copies remain.
#include <mutex>

#include "kv_compact_rows.h"

namespace tv {
namespace {

constexpr int kThreads = 512;
constexpr int kMinChunk = 8192;      // floats per workgroup at least
// enough workgroups to keep HBM busy: from 512 rows on, twice as many (the
// 70B-shaped chain 101 -> 98 us); below, more chunks per row only add keys
// for the walk to fold (the Llama-3-8B tree 15.5 -> 17.1 us at 2048)
constexpr int kTargetBlocks = 1024;
constexpr int kTargetBlocksManyRows = 2048;
constexpr long kManyRows = 512;

struct Split {
  int chunk;   // floats per chunk (multiple of 4)
  int chunks;  // chunks per row
};

Split split_for(int B, int N, int V) {
  const long rows = static_cast<long>(B) * N;
  const long target = rows >= kManyRows ? kTargetBlocksManyRows : kTargetBlocks;
  long c = (target + rows - 1) / rows;
  const long cmax = (V + kMinChunk - 1) / kMinChunk;
  if (c > cmax) c = cmax;
  if (c < 1) c = 1;
  int chunk = static_cast<int>((V + c - 1) / c);
  chunk = (chunk + 3) & ~3;
  Split s;
  s.chunk = chunk;
  s.chunks = (V + chunk - 1) / chunk;
  return s;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}

template <int kT, int kL>
__global__ __launch_bounds__(kT) void accept_scan_kernel(const float* __restrict__ logits,
                                                               int V, int chunk, int chunks,
                                                               uint64_t* __restrict__ keys) {
  __shared__ uint64_t wbest[kT / 64];
  const long row = blockIdx.x / chunks;
  const int ch = blockIdx.x % chunks;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lo = ch * chunk;
  const int hi = min(V, lo + chunk);
  const float* x = logits + row * V;
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  if ((V & 3) == 0) {
    // four independent 16-byte loads in flight, then compared in index order
    // (each thread visits increasing indices, so strict '>' keeps the first
    // occurrence of its maximum)
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4* x4 = reinterpret_cast<const f32x4*>(x);
    const int lo4 = lo / 4, hi4 = hi / 4;
    for (int j0 = lo4 + tid; j0 < hi4; j0 += kL * kT) {
      f32x4 v[kL];
#pragma unroll
      for (int u = 0; u < kL; ++u) {
        const int j = j0 + u * kT;
        v[u] = j < hi4 ? __builtin_nontemporal_load(x4 + j) : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
#pragma unroll
      for (int u = 0; u < kL; ++u) {
        const int j = j0 + u * kT;
        if (j >= hi4) break;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (v[u][e] > bv || bi == 0x7FFFFFFF) {
            bv = v[u][e];
            bi = 4 * j + e;
          }
      }
    }
  } else {
    for (int j = lo + tid; j < hi; j += kT) {
      const float v = x[j];
      if (v > bv || bi == 0x7FFFFFFF) {
        bv = v;
        bi = j;
      }
    }
  }
  uint64_t key = (bi == 0x7FFFFFFF) ? 0ull : make_key(bv, bi);
  key = wave_max_u64(key);
  if (lane == 0) wbest[wave] = key;
  __syncthreads();
  if (tid == 0) {
    uint64_t k = wbest[0];
    for (int w = 1; w < kT / 64; ++w) k = wbest[w] > k ? wbest[w] : k;
    keys[row * chunks + ch] = k;
  }
}

// kCompact: the fused call (tv_accept_greedy_compact) also compacts
template <bool kCompact>
__global__ __launch_bounds__(kThreads) void accept_walk_kernel(AcceptArgs a, int chunks) {
  __shared__ int s_par[TV_MAX_NODES], s_tok[TV_MAX_NODES], s_am[TV_MAX_NODES];
  __shared__ int s_ok[TV_MAX_NODES], s_dep[TV_MAX_NODES], s_on[TV_MAX_NODES];
  __shared__ int s_bad, s_dmax, s_path[TV_MAX_NODES];
  __shared__ unsigned long long s_key[TV_MAX_NODES];
  // fused compaction: block ids of the tree region, and each step's rows
  __shared__ int s_tab[TV_MAX_NODES / kBlockSize + 2], s_cbad;
  __shared__ long long s_src[TV_MAX_NODES], s_dst[TV_MAX_NODES];

  const int N = a.N, V = a.V;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const CompactArgs& c = a.compact;
  constexpr bool fuse = kCompact;
  const uint64_t* keys = static_cast<const uint64_t*>(a.workspace);
  const size_t base = static_cast<size_t>(b) * N;

  // fused compaction: the tree region's block ids, P_b / 16 .. (P_b + N - 1) / 16
  const int P = fuse ? c.prefix_lens[b] : 0;
  const bool p_ok = P >= 0 && static_cast<long>(P) + N <= static_cast<long>(c.max_blocks) * kBlockSize;
  const int tab0 = P / kBlockSize;
  // compaction of steps 0 .. L-1 of s_path (the fused call only)
  auto compact = [&](int L) __attribute__((always_inline)) {
    int cbad = p_ok ? 0 : TV_DEV_BAD_CACHE;
    if (!cbad) {
      for (int j = tid; j < L; j += kThreads) {
        const int ts = P + s_path[j], td = P + j;
        const int bs = s_tab[ts / kBlockSize - tab0], bd = s_tab[td / kBlockSize - tab0];
        if (bs < 0 || bs >= c.num_blocks || bd < 0 || bd >= c.num_blocks) {
          cbad |= TV_DEV_BAD_CACHE;
          continue;
        }
        s_src[j] = kv_row(bs, 0, ts % kBlockSize, c.Hkv, c.kv_head_rows, c.kv_slot_rows);
        s_dst[j] = kv_row(bd, 0, td % kBlockSize, c.Hkv, c.kv_head_rows, c.kv_slot_rows);
      }
    }
    if (cbad) atomicOr(&s_cbad, cbad);
    __syncthreads();
    if (s_cbad) {  // the sequence is left untouched
      if (tid == 0) report(a.dev_status, s_cbad);
      return;
    }
    if (tid == 0 && c.new_lens) c.new_lens[b] = P + L;
    compact_copy_columns(c, s_src, s_dst, L, tid, kThreads);
  };

  if (N <= 64) {
    // ---- a tree of at most 64 nodes: one wave holds a node per lane and
    // finds the path in registers (shuffles and ballots instead of LDS round
    // trips and barriers); the decisions are those of the general path below ----
    if (tid == 0) s_cbad = 0;
    if (fuse && p_ok)
      for (int i = tid; i <= (P + N - 1) / kBlockSize - tab0; i += kThreads)
        s_tab[i] = c.block_table[static_cast<size_t>(b) * c.max_blocks + tab0 + i];
    if (wave == 0) {
      const bool exists = lane < N;
      int par = -1, tok = 0;
      if (exists) {
        par = a.parents[base + lane];
        tok = a.draft_tokens[base + lane];
      }
      // the target argmax of node `lane`: the largest of its row's chunk
      // keys, sixteen loads in flight at a time
      uint64_t best = 0ull;
      const uint64_t* rk = keys + (base + (exists ? lane : 0)) * chunks;
      for (int c0 = 0; c0 < chunks; c0 += 16) {
        uint64_t kk[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) kk[u] = rk[min(c0 + u, chunks - 1)];
#pragma unroll
        for (int u = 0; u < 16; ++u) best = kk[u] > best ? kk[u] : best;
      }
      const int am = static_cast<int>(key_index(best));
      if (exists && a.target_argmax) a.target_argmax[base + lane] = am;
      int bad = 0;
      if (exists) {
        if (lane == 0 ? par != -1 : (par < 0 || par >= lane)) bad |= TV_DEV_BAD_TREE;
        if (lane > 0 && (tok < 0 || tok >= V)) bad |= TV_DEV_BAD_TOKEN;
      }
      for (int o = 32; o > 0; o >>= 1) bad |= __shfl_xor(bad, o, 64);
      int path_len = 1;
      if (bad) {
        if (lane == 0) report(a.dev_status, bad);
        if (exists) a.accepted_nodes[base + lane] = lane == 0 ? 0 : -1;
        const int am0 = __shfl(am, 0, 64);
        if (lane == 0) {
          a.accept_len[b] = 0;
          a.bonus_token[b] = am0;
          s_path[0] = 0;
        }
      } else {
        // node i is reachable iff every edge on its root path is accepted (the
        // child's token is its parent's target argmax): the AND of those
        // edges and the depth, by pointer jumping up the root path
        const int am_par = __shfl(am, par >= 0 ? par : 0, 64);
        bool ok = exists && (lane == 0 || tok == am_par);
        int dep = (exists && lane > 0) ? 1 : 0;
        int jump = (exists && lane > 0) ? par : -1;
        for (int r = 0; r < 6 && __builtin_amdgcn_ballot_w64(jump >= 0) != 0; ++r) {
          const int src = jump >= 0 ? jump : lane;
          const bool up_ok = __shfl(static_cast<int>(ok), src, 64) != 0;
          const int up_dep = __shfl(dep, src, 64);
          const int up_jump = __shfl(jump, src, 64);
          if (jump >= 0) {
            ok = ok && up_ok;
            dep += up_dep;
            jump = up_jump;
          }
        }
        int dmax = ok ? dep : -1;
        for (int o = 32; o > 0; o >>= 1) dmax = max(dmax, __shfl_xor(dmax, o, 64));
        // every node on some deepest accepted path: the ancestors-or-self of
        // the deepest accepted nodes
        bool not_tree;
        const uint64_t anc = wave_tree_mask(par, N, lane, &not_tree);
        uint64_t on = (ok && dep == dmax) ? anc : 0ull;
        for (int o = 32; o > 0; o >>= 1) on |= __shfl_xor(on, o, 64);
        // descend from the root, taking the lowest-index marked child each
        // step (always there: a marked node's parent is marked)
        int cur = 0, mine = 0;
        for (int k = 1; k <= dmax; ++k) {
          const uint64_t kids = __builtin_amdgcn_ballot_w64(exists && par == cur && ((on >> lane) & 1ull));
          cur = static_cast<int>(__builtin_ctzll(kids));
          if (lane == k) mine = cur;
        }
        if (exists) a.accepted_nodes[base + lane] = lane <= dmax ? mine : -1;
        if (lane <= dmax) s_path[lane] = mine;
        const int bonus = __shfl(am, cur, 64);
        if (lane == 0) {
          a.accept_len[b] = dmax;
          a.bonus_token[b] = bonus;
        }
        path_len = dmax + 1;
      }
      if (lane == 0) s_dmax = path_len;
    }
    __syncthreads();
    if (fuse) compact(s_dmax);
    return;
  }

  // ---- the general path (up to 256 nodes), through LDS ----
  // every (node, chunk) key of the sequence is contiguous in the workspace;
  // the first eight per thread are loaded together with the tree and the
  // draft tokens, so both latencies overlap
  const uint64_t* kb = keys + base * chunks;
  const int nk = N * chunks;
  uint64_t kv[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int k = tid + u * kThreads;
    kv[u] = k < nk ? kb[k] : 0ull;
  }
  for (int i = tid; i < N; i += kThreads) {
    s_par[i] = a.parents[base + i];
    s_tok[i] = a.draft_tokens[base + i];
    s_on[i] = 0;
    s_key[i] = 0ull;
  }
  if (tid == 0) {
    s_bad = 0;
    s_dmax = 0;
    s_cbad = 0;
  }
  if (fuse && p_ok)
    for (int i = tid; i <= (P + N - 1) / kBlockSize - tab0; i += kThreads)
      s_tab[i] = c.block_table[static_cast<size_t>(b) * c.max_blocks + tab0 + i];
  __syncthreads();
  // fold the keys per node with LDS max (further rounds of eight per thread
  // when N * chunks exceeds eight per thread)
  for (int k0 = tid;;) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = k0 + u * kThreads;
      if (k < nk) atomicMax(&s_key[k / chunks], static_cast<unsigned long long>(kv[u]));
    }
    k0 += 8 * kThreads;
    if (k0 >= nk) break;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = k0 + u * kThreads;
      kv[u] = k < nk ? kb[k] : 0ull;
    }
  }
  __syncthreads();
  for (int i = tid; i < N; i += kThreads) {
    const int am = static_cast<int>(key_index(s_key[i]));
    s_am[i] = am;
    if (a.target_argmax) a.target_argmax[base + i] = am;
  }
  __syncthreads();

  int bad = 0;
  for (int i = tid; i < N; i += kThreads) {
    const int p = s_par[i];
    if (i == 0 ? p != -1 : (p < 0 || p >= i)) bad |= TV_DEV_BAD_TREE;
    if (i > 0 && (s_tok[i] < 0 || s_tok[i] >= V)) bad |= TV_DEV_BAD_TOKEN;
  }
  if (bad) atomicOr(&s_bad, bad);
  __syncthreads();
  if (s_bad) {
    if (tid == 0) report(a.dev_status, s_bad);
    for (int i = tid; i < N; i += kThreads) a.accepted_nodes[base + i] = (i == 0) ? 0 : -1;
    if (tid == 0) {
      a.accept_len[b] = 0;
      a.bonus_token[b] = s_am[0];
      s_path[0] = 0;
    }
    if (fuse) {
      __syncthreads();
      compact(1);  // the root alone: nothing moves, the new length is P_b + 1
    }
    return;
  }

  // node i is reachable iff every edge on its root path is accepted
  for (int i = tid; i < N; i += kThreads) {
    int c = i, d = 0, ok = 1;
    while (c != 0) {
      const int p = s_par[c];
      if (s_tok[c] != s_am[p]) { ok = 0; break; }
      c = p;
      ++d;
    }
    s_ok[i] = ok;
    s_dep[i] = d;
    if (ok) atomicMax(&s_dmax, d);
  }
  __syncthreads();
  const int dmax = s_dmax;
  // mark every node on some deepest accepted path
  for (int i = tid; i < N; i += kThreads) {
    if (s_ok[i] && s_dep[i] == dmax) {
      int c = i;
      s_on[c] = 1;
      while (c != 0) {
        c = s_par[c];
        s_on[c] = 1;
      }
    }
  }
  __syncthreads();
  // descend from the root, taking the lowest-index marked child each step
  if (wave == 0) {
    int cur = 0;
    if (lane == 0) s_path[0] = 0;
    for (int k = 1; k <= dmax; ++k) {
      int next = -1;
      for (int c0 = cur + 1; c0 < N && next < 0; c0 += 64) {
        const int c = c0 + lane;
        const bool hit = c < N && s_par[c] == cur && s_on[c];
        const uint64_t m = __ballot(hit);
        if (m) next = c0 + __builtin_ctzll(m);
      }
      if (next >= 0) cur = next;  // always found: a marked node's parent is marked
      if (lane == 0) s_path[k] = cur;
    }
  }
  __syncthreads();
  for (int i = tid; i < N; i += kThreads) a.accepted_nodes[base + i] = (i <= dmax) ? s_path[i] : -1;
  if (tid == 0) {
    a.accept_len[b] = dmax;
    a.bonus_token[b] = s_am[s_path[dmax]];
  }
  if (fuse) compact(dmax + 1);
}

}  // namespace

size_t accept_workspace_bytes(int B, int N, int V) {
  const Split s = split_for(B, N, V);
  return static_cast<size_t>(B) * N * s.chunks * sizeof(uint64_t);
}

hipError_t launch_accept(const AcceptArgs& a, hipStream_t stream) {
  const Split s = split_for(a.B, a.N, a.V);
  const long blocks = static_cast<long>(a.B) * a.N * s.chunks;
  // kT threads with kL 16-byte loads each in flight per pass: from 512 rows
  // on (long chunks, several passes each), 1024 x 2 (the batched workload
  // 70.7 -> 69.7 us, the 70B chain 94.4 -> 94.0 us; 1024 x 4 and 256 x 8
  // slower); below, 512 x 4 (1024 x 2 was 8 % slower on the Llama-3-8B tree)
  if (static_cast<long>(a.B) * a.N >= kManyRows)
    hipLaunchKernelGGL((accept_scan_kernel<1024, 2>), dim3(static_cast<unsigned>(blocks)), dim3(1024), 0, stream,
                       a.logits, a.V, s.chunk, s.chunks, static_cast<uint64_t*>(a.workspace));
  else
    hipLaunchKernelGGL((accept_scan_kernel<kThreads, 4>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                       stream, a.logits, a.V, s.chunk, s.chunks, static_cast<uint64_t*>(a.workspace));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.compact.k_cache)
    hipLaunchKernelGGL(accept_walk_kernel<true>, dim3(a.B), dim3(kThreads), 0, stream, a, s.chunks);
  else
    hipLaunchKernelGGL(accept_walk_kernel<false>, dim3(a.B), dim3(kThreads), 0, stream, a, s.chunks);
  return hipGetLastError();
}

// ---------------- scratch of the allocation-free variant ----------------
// tv_accept_greedy_noalloc keeps its scan keys in this file-scope device
// array instead of a caller workspace.  Every GPU the library runs on holds
// its own copy until the process ends.  In host code `scratch` names a host
// stand-in, not device memory: the device address of each GPU's copy is
// looked up once per device with that device current, and only that address
// is handed to the kernels (as the workspace pointer of launch_accept).  The
// keys need no initial contents (each one a call reads is written earlier in
// the same call), so nothing is cleared between calls.
static __device__ __align__(256) uint64_t scratch[kAcceptScratchBytes / sizeof(uint64_t)];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

hipError_t accept_static_scratch(hipStream_t stream, void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    int cur = 0;
    hipError_t r = hipGetDevice(&cur);
    const bool other = r == hipSuccess && cur != dev;
    if (other) r = hipSetDevice(dev);
    void* p = nullptr;
    if (r == hipSuccess) r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (other) {
      const hipError_t back = hipSetDevice(cur);
      if (r == hipSuccess) r = back;
    }
    g_scratch_ptr[dev] = r == hipSuccess ? p : nullptr;
    g_scratch_err[dev] = r;
  });
  *ptr = g_scratch_ptr[dev];
  return g_scratch_err[dev] != hipSuccess ? g_scratch_err[dev]
                                          : (*ptr ? hipSuccess : hipErrorInvalidSymbol);
}

}  // namespace tv
