// Stochastic verification of a draft tree at temperature T > 0.
// ("P-EAGLE", 技术原理和实现方式 steps 3-4: the target's probabilities of
// the proposed tokens are compared with the drafter's and a sampling rule
// accepts or cuts; "vLLM EAGLE 投机解码实战", 无损性保障: the rejection
// sampler keeps the target distribution.)  The rule: the children of the
// current node are tested in index order, child c (token x, proposal q) is
// accepted iff u_c * q(x) < r(x), a rejection turns r into the normalised
// positive part of r - q, and when every child is rejected the bonus token
// is the largest r[v] / E[v].  Proposals are point masses (deterministic
// top-k trees) or, on chains, dense rows.
//
// Four launches, no atomics between workgroups:
//  1. stats (rows x chunks workgroups): per chunk of a logits row, the max
//     of y = logit * log2(e) / T and the sum of 2^(y - max);
//  2. walk (one workgroup per sequence): merge the chunk stats of every row,
//     gather every node's target and proposal probability of its own token
//     (one latency for the whole tree), then one wavefront walks the tree
//     from LDS and leaves a stop record: the node, its row stats, and what
//     the rejections removed (tokens, or the rejected child's proposal row);
//  3. draw (sequences x chunks workgroups): the best r[v] / E[v] key of one
//     chunk of the stop node's row;
//  4. pick (one thread per sequence): the best key -> bonus token.
// Folding the pick into the draw (the last workgroup of a sequence to
// arrive picks) needs a device-scope fence per workgroup, an L2 write-back
// on this chip, which cost far more than the launch it saves.
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kMinChunk = 8192;       // stats: floats per workgroup at least
constexpr int kTargetBlocks = 1024;   // enough workgroups to keep HBM busy,
constexpr int kTargetBlocksManyRows = 2048;  // twice as many from 512 rows on
constexpr long kManyRows = 512;
constexpr int kDrawMinChunk = 2048;   // draw: floats per workgroup at least
constexpr int kDrawMaxChunk = 16384;  // draw: at most (sizes the LDS bitmap)
constexpr int kPickThreads = 256;   // four sequences per pick workgroup, one per wave
constexpr int kStatsBatch = 16;     // walk: chunk statistics of a row loaded together

struct Split {
  int chunk;   // floats per chunk (multiple of 4)
  int chunks;  // chunks per row
};

Split split_rows(long rows, int V, int min_chunk, int max_chunk) {
  const long target = rows >= kManyRows ? kTargetBlocksManyRows : kTargetBlocks;
  long c = (target + rows - 1) / rows;
  const long cmax = (V + min_chunk - 1) / min_chunk;
  const long cmin = (V + max_chunk - 1) / max_chunk;
  if (c > cmax) c = cmax;
  if (c < cmin) c = cmin;
  if (c < 1) c = 1;
  int chunk = static_cast<int>((V + c - 1) / c);
  chunk = (chunk + 3) & ~3;
  Split s;
  s.chunk = chunk;
  s.chunks = (V + chunk - 1) / chunk;
  return s;
}

Split stats_split(int B, int N, int V) { return split_rows(static_cast<long>(B) * N, V, kMinChunk, 1 << 30); }
Split draw_split(int B, int V) { return split_rows(B, V, kDrawMinChunk, kDrawMaxChunk); }

// Where the walk stopped, for the draw.
struct StopRecord {
  int node;       // stop node u
  int rej_child;  // >= 0: r = max(p_u - q_rej_child, 0) (dense proposal rejected); -1: r = p_u off R
  int n_removed;  // tokens in R (point-mass rejections)
  int pad;
  float m, s;     // stats of row u: p_u(v) = 2^(y_v - m) / s
  float pad2[2];
  int removed[TV_MAX_NODES];
};

struct Layout {
  Split st, dr;
  size_t stats_off, stop_off, keys_off, total;
};

Layout layout_for(int B, int N, int V) {
  Layout l;
  l.st = stats_split(B, N, V);
  l.dr = draw_split(B, V);
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  l.stats_off = 0;
  l.stop_off = up(static_cast<size_t>(B) * N * l.st.chunks * sizeof(float2));
  l.keys_off = l.stop_off + up(static_cast<size_t>(B) * sizeof(StopRecord));
  l.total = l.keys_off + static_cast<size_t>(B) * l.dr.chunks * sizeof(uint64_t);
  return l;
}

// (m, s) pairs: s * 2^m summed.  m = -inf means an empty sum.
__device__ __forceinline__ void merge_ms(float& m, float& s, float m2, float s2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) {
    m = m2;
    s = s2;
    return;
  }
  const float M = fmaxf(m, m2);
  s = s * exp2f(m - M) + s2 * exp2f(m2 - M);
  m = M;
}

__global__ __launch_bounds__(kThreads) void stoch_stats_kernel(const float* __restrict__ logits, int V,
                                                               float k2, int chunk, int chunks,
                                                               float2* __restrict__ stats) {
  __shared__ float2 wpart[kWaves];
  const long row = blockIdx.x / chunks;
  const int ch = blockIdx.x % chunks;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lo = ch * chunk;
  const int hi = min(V, lo + chunk);
  const float* x = logits + row * V;
  float m = -INFINITY, s = 0.f;
  if ((V & 3) == 0) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4* x4 = reinterpret_cast<const f32x4*>(x);
    const int lo4 = lo / 4, hi4 = hi / 4;
    for (int j0 = lo4 + tid; j0 < hi4; j0 += 4 * kThreads) {
      f32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + u * kThreads;
        v[u] = j < hi4 ? __builtin_nontemporal_load(x4 + j) : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
      float gm = -INFINITY;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) gm = fmaxf(gm, v[u][e] * k2);
      if (gm > m) {
        s = (m == -INFINITY) ? 0.f : s * exp2f(m - gm);
        m = gm;
      }
      // the bare v_exp_f32: exp2f adds a scaling for results in the denormal
      // range (six more instructions per entry), and such terms add nothing
      // to a sum whose largest term is 1 (all three calls 2-3 % faster, the
      // same accepted paths and draws)
      if (m != -INFINITY) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) s += __builtin_amdgcn_exp2f(v[u][e] * k2 - m);
      }
    }
  } else {
    for (int j = lo + tid; j < hi; j += kThreads) {
      const float y = x[j] * k2;
      if (y > m) {
        s = (m == -INFINITY) ? 0.f : s * exp2f(m - y);
        m = y;
      }
      if (m != -INFINITY) s += __builtin_amdgcn_exp2f(y - m);
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64);
    const float s2 = __shfl_xor(s, o, 64);
    merge_ms(m, s, m2, s2);
  }
  if (lane == 0) wpart[wave] = make_float2(m, s);
  __syncthreads();
  if (tid == 0) {
    float M = wpart[0].x, S = wpart[0].y;
    for (int w = 1; w < kWaves; ++w) merge_ms(M, S, wpart[w].x, wpart[w].y);
    stats[row * chunks + ch] = make_float2(M, S);
  }
}

__global__ __launch_bounds__(kThreads) void stoch_walk_kernel(StochArgs a, float k2, int chunks,
                                                              const float2* __restrict__ stats,
                                                              StopRecord* __restrict__ stop) {
  __shared__ int s_par[TV_MAX_NODES], s_tok[TV_MAX_NODES], s_path[TV_MAX_NODES];
  __shared__ float s_m[TV_MAX_NODES], s_s[TV_MAX_NODES], s_gl[TV_MAX_NODES];
  __shared__ float s_px[TV_MAX_NODES], s_qx[TV_MAX_NODES], s_u[TV_MAX_NODES];
  __shared__ int s_removed[TV_MAX_NODES];
  __shared__ int s_bad;
  __shared__ int s_stop_node, s_rej, s_nrem, s_len;

  const int N = a.N, V = a.V;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t base = static_cast<size_t>(b) * N;
  const bool dense = a.draft_probs != nullptr;
  if (tid == 0) s_bad = 0;
  __syncthreads();

  // node tid: its parent, token and uniform, then (when they are in range)
  // the target logit of its token in its parent's row and its proposal
  // probability; the row stats merge while those loads are in flight
  int par = 0, tok = 0;
  float gl = 0.f, gq = 1.f, u = 0.f;
  int bad = 0;
  if (tid < N) {
    par = a.parents[base + tid];
    tok = a.draft_tokens[base + tid];
    u = a.uniforms[base + tid];
    if (tid == 0 ? par != -1 : (par < 0 || par >= tid)) bad |= TV_DEV_BAD_TREE;
    if (tid > 0 && (tok < 0 || tok >= V)) bad |= TV_DEV_BAD_TOKEN;
    if (tid > 0 && !(u >= 0.f && u < 1.f)) bad |= TV_DEV_BAD_RANDOM;
    if (dense && tid > 0 && par != tid - 1) bad |= TV_DEV_UNSUPPORTED;
    if (tid > 0 && par >= 0 && par < tid && tok >= 0 && tok < V) {
      gl = a.logits[(base + par) * V + tok];
      if (dense) gq = a.draft_probs[(base + tid) * V + tok];
    }
  }
  for (int i = tid; i < N; i += kThreads) {
    const float2* st = stats + (base + i) * chunks;
    float m = -INFINITY, s = 0.f;
    // sixteen chunk statistics at a time, all in flight together (from
    // clamped indices, so no load is conditional), then merged in chunk order
    for (int c0 = 0; c0 < chunks; c0 += kStatsBatch) {
      float2 v[kStatsBatch];
#pragma unroll
      for (int k = 0; k < kStatsBatch; ++k) v[k] = st[min(c0 + k, chunks - 1)];
#pragma unroll
      for (int k = 0; k < kStatsBatch; ++k)
        if (c0 + k < chunks) merge_ms(m, s, v[k].x, v[k].y);
    }
    s_m[i] = m;
    s_s[i] = s;
  }
  if (tid < N) {
    s_par[tid] = par;
    s_tok[tid] = tok;
    s_u[tid] = u;
    s_gl[tid] = gl;
    s_qx[tid] = gq;
  }
  if (bad) atomicOr(&s_bad, bad);
  __syncthreads();
  if (tid == 0 && s_bad) report(a.dev_status, s_bad);
  // a malformed tree (or dense proposals off a chain) walks nowhere: the
  // bonus is drawn from the root's distribution
  const bool usable = (s_bad & (TV_DEV_BAD_TREE | TV_DEV_BAD_TOKEN | TV_DEV_UNSUPPORTED)) == 0;
  if (tid > 0 && tid < N && usable) {
    const int p = s_par[tid];
    s_px[tid] = exp2f(s_gl[tid] * k2 - s_m[p]) / s_s[p];
  }
  __syncthreads();

  if (wave == 0) {
    int cur = 0, len = 0, rej = -1, nrem = 0;
    float mass = 1.f;  // mass of p_cur left after the point-mass rejections
    if (lane == 0) s_path[0] = 0;
    while (usable) {
      int next = -1;
      mass = 1.f;
      nrem = 0;
      rej = -1;
      for (int c0 = cur + 1; c0 < N && next < 0; c0 += 64) {
        const int cl = c0 + lane;
        uint64_t kids = __ballot(cl < N && s_par[cl] == cur);
        while (kids) {
          const int c = c0 + __builtin_ctzll(kids);
          kids &= kids - 1;
          const int x = s_tok[c];
          const float px = s_px[c];
          bool accept;
          if (dense) {
            accept = s_u[c] * s_qx[c] < px;
            if (!accept) rej = c;
          } else {
            bool removed = false;
            for (int j0 = 0; j0 < nrem; j0 += 64) {
              const int j = j0 + lane;
              if (__ballot(j < nrem && s_removed[j] == x)) removed = true;
            }
            accept = !removed && s_u[c] * mass < px;
            if (!accept && !removed && mass - px > 0.f) {
              mass -= px;
              if (lane == 0) s_removed[nrem] = x;
              ++nrem;
            }
          }
          if (accept) {
            next = c;
            break;
          }
        }
      }
      if (next < 0) break;
      cur = next;
      ++len;
      if (lane == 0) s_path[len] = cur;
    }
    if (lane == 0) {
      s_stop_node = cur;
      s_rej = rej;
      s_nrem = nrem;
      s_len = len;
    }
  }
  __syncthreads();
  const int len = s_len;
  for (int i = tid; i < N; i += kThreads) a.accepted_nodes[base + i] = (i <= len) ? s_path[i] : -1;
  StopRecord* r = stop + b;
  for (int i = tid; i < s_nrem; i += kThreads) r->removed[i] = s_removed[i];
  if (tid == 0) {
    a.accept_len[b] = len;
    const int u_node = s_stop_node;
    r->node = u_node;
    r->rej_child = s_rej;
    r->n_removed = s_nrem;
    r->m = s_m[u_node];
    r->s = s_s[u_node];
  }
}

__global__ __launch_bounds__(kThreads) void stoch_draw_kernel(StochArgs a, float k2, int chunk, int chunks,
                                                              const StopRecord* __restrict__ stop,
                                                              uint64_t* __restrict__ keys) {
  __shared__ uint32_t s_bits[kDrawMaxChunk / 32];
  __shared__ uint64_t wbest[kWaves];
  __shared__ int s_bad;
  const int b = blockIdx.x / chunks;
  const int ch = blockIdx.x % chunks;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int V = a.V;
  const int lo = ch * chunk;
  const int hi = min(V, lo + chunk);
  const StopRecord* r = stop + b;
  const int node = r->node, rej = r->rej_child, nrem = r->n_removed;
  const float m = r->m, s = r->s;
  for (int w = tid; w < kDrawMaxChunk / 32; w += kThreads) s_bits[w] = 0u;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  for (int i = tid; i < nrem; i += kThreads) {
    const int x = r->removed[i];
    if (x >= lo && x < hi) atomicOr(&s_bits[(x - lo) >> 5], 1u << ((x - lo) & 31));
  }
  __syncthreads();
  const size_t base = static_cast<size_t>(b) * a.N;
  const float* lrow = a.logits + (base + node) * V;
  const float* qrow = rej >= 0 ? a.draft_probs + (base + rej) * V : nullptr;
  const float* erow = a.exponentials + static_cast<size_t>(b) * V;
  const float inv_s = 1.f / s;
  uint64_t best = 0ull;
  bool bad = false;
  // one vocabulary entry: r(v) / E(v) as a key
  auto score = [&](int v, float lg, float e, float q) {
    const float p = __builtin_amdgcn_exp2f(lg * k2 - m) * inv_s;
    float rv;
    if (qrow)
      rv = fmaxf(p - q, 0.f);
    else
      rv = ((s_bits[(v - lo) >> 5] >> ((v - lo) & 31)) & 1u) ? 0.f : p;
    if (!(e > 0.f && e < INFINITY)) bad = true;
    const uint64_t k = make_key(rv / e, v);
    best = k > best ? k : best;
  };
  const bool vec = (V & 3) == 0 && ((reinterpret_cast<uintptr_t>(erow) | reinterpret_cast<uintptr_t>(lrow) |
                                     reinterpret_cast<uintptr_t>(qrow)) & 15u) == 0;
  if (vec) {
    // four 16-byte loads of each row in flight per thread
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4* l4 = reinterpret_cast<const f32x4*>(lrow);
    const f32x4* e4 = reinterpret_cast<const f32x4*>(erow);
    const f32x4* q4 = reinterpret_cast<const f32x4*>(qrow);
    const int lo4 = lo / 4, hi4 = hi / 4;
    for (int j0 = lo4 + tid; j0 < hi4; j0 += 4 * kThreads) {
      f32x4 lv[4], ev[4], qv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + u * kThreads;
        const bool in = j < hi4;
        lv[u] = in ? __builtin_nontemporal_load(l4 + j) : f32x4{0.f, 0.f, 0.f, 0.f};
        ev[u] = in ? __builtin_nontemporal_load(e4 + j) : f32x4{1.f, 1.f, 1.f, 1.f};
        qv[u] = (in && qrow) ? __builtin_nontemporal_load(q4 + j) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + u * kThreads;
        if (j >= hi4) break;
#pragma unroll
        for (int e = 0; e < 4; ++e) score(4 * j + e, lv[u][e], ev[u][e], qv[u][e]);
      }
    }
  } else {
    for (int v = lo + tid; v < hi; v += kThreads) score(v, lrow[v], erow[v], qrow ? qrow[v] : 0.f);
  }
  if (bad) s_bad = 1;
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t w = __shfl_xor(best, o, 64);
    best = w > best ? w : best;
  }
  if (lane == 0) wbest[wave] = best;
  __syncthreads();
  if (tid == 0) {
    uint64_t k = wbest[0];
    for (int w = 1; w < kWaves; ++w) k = wbest[w] > k ? wbest[w] : k;
    if (s_bad) report(a.dev_status, TV_DEV_BAD_RANDOM);
    keys[static_cast<size_t>(b) * chunks + ch] = k;
  }
}

// One wave per sequence: lanes load the chunk keys together, and a wave
// maximum picks the best (the keys order by value, then lower index).
__global__ __launch_bounds__(kPickThreads) void stoch_pick_kernel(int B, int chunks, const uint64_t* __restrict__ keys,
                                                                  int32_t* __restrict__ bonus) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * (kPickThreads / 64) + static_cast<int>(threadIdx.x >> 6);
  if (b >= B) return;  // the whole wave
  uint64_t best = 0ull;
  for (int c = lane; c < chunks; c += 64) {
    const uint64_t k = keys[static_cast<size_t>(b) * chunks + c];
    best = k > best ? k : best;
  }
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t w = __shfl_xor(best, o, 64);
    best = w > best ? w : best;
  }
  if (lane == 0) bonus[b] = static_cast<int>(~static_cast<uint32_t>(best & 0xFFFFFFFFu));
}

}  // namespace

size_t stochastic_workspace_bytes(int B, int N, int V) { return layout_for(B, N, V).total; }

hipError_t launch_accept_stochastic(const StochArgs& a, hipStream_t stream) {
  const Layout l = layout_for(a.B, a.N, a.V);
  char* ws = static_cast<char*>(a.workspace);
  float2* stats = reinterpret_cast<float2*>(ws + l.stats_off);
  StopRecord* stop = reinterpret_cast<StopRecord*>(ws + l.stop_off);
  uint64_t* keys = reinterpret_cast<uint64_t*>(ws + l.keys_off);
  // y = logit / T in base-2 units
  const float k2 = 1.4426950408889634f / a.temperature;
  const long sblocks = static_cast<long>(a.B) * a.N * l.st.chunks;
  hipLaunchKernelGGL(stoch_stats_kernel, dim3(static_cast<unsigned>(sblocks)), dim3(kThreads), 0, stream,
                     a.logits, a.V, k2, l.st.chunk, l.st.chunks, stats);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(stoch_walk_kernel, dim3(a.B), dim3(kThreads), 0, stream, a, k2, l.st.chunks,
                     static_cast<const float2*>(stats), stop);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long dblocks = static_cast<long>(a.B) * l.dr.chunks;
  hipLaunchKernelGGL(stoch_draw_kernel, dim3(static_cast<unsigned>(dblocks)), dim3(kThreads), 0, stream, a, k2,
                     l.dr.chunk, l.dr.chunks, static_cast<const StopRecord*>(stop), keys);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int kPickSeqs = kPickThreads / 64;
  hipLaunchKernelGGL(stoch_pick_kernel, dim3((a.B + kPickSeqs - 1) / kPickSeqs), dim3(kPickThreads), 0,
                     stream, a.B, l.dr.chunks, static_cast<const uint64_t*>(keys), a.bonus_token);
  return hipGetLastError();
}

}  // namespace tv
