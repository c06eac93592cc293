// Draft-tree construction from the drafter's scores: top-k expansion level by
// level and a global rerank by cumulative log-probability.
// ("EAGLE代码实现原理", 树结构缓冲: branch prediction proposes likely
// continuations ahead and level pruning keeps the high-probability paths;
// "vLLM-TreeEagle" README, 核心组件 item 3: multi-level candidate generation
// with path pruning.)
//
// Chunk kernel (rows x chunks workgroups of 256 threads): one chunk of one
// score row (8192 entries, or 4096 when a batch has fewer than 1024 of the
// larger ones, so that loads and the selection of different workgroups
// overlap) is held in registers after one pass of 16-byte loads.  It
// yields the chunk's maximum, its sum of exp(x - max), and its topk best
// entries as 64-bit keys (value, then lower index).  The topk selection cuts
// first: T = the topk-th largest of the 32 maxima of 8-lane groups bounds the
// chunk's topk-th entry from below, and only entries at or above T (all of
// them in at most topk groups, usually a few more than topk) are ranked.
// If more than kCandCap pass the cut, topk block-wide max rounds take over.
//
// Row kernel (one wave per row): merges the chunks of each row into its
// log-sum-exp and its topk best keys (the same cut-then-rank selection over
// the chunk lists), all rows of all sequences at once.
//
// Build kernel (one 1024-thread workgroup per sequence): walks the levels:
// candidate (j, r) of level l scores F_j + x - lse, where F_j is the score of
// the j-th best node of level l - 1; every level's candidates are ranked in
// full.  The kept nodes of a level are a prefix of its ranked list (the
// global order restricted to one level is that level's order), so the global
// top N - 1 is found by counting, per candidate, the better candidates of
// every other level with a binary search, and node labels follow as level
// offsets plus ranks.
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kChunkThreads = 256;
constexpr int kBigPer4 = 8;                             // 16-byte loads per thread: 8192-entry chunks
constexpr int kSmallPer4 = 4;                           // 4096-entry chunks for small batches
constexpr int kSmallBatchUnits = 1024;                  // below this many 8192-entry chunks, halve them
constexpr int kGroups = kChunkThreads / 8;              // 8-lane groups per chunk workgroup
constexpr int kCandCap = 512;                           // ranked candidates per chunk
constexpr int kRowWaves = 4;                            // rows per row-merge workgroup
constexpr int kBuildThreads = 1024;
constexpr int kMaxK = TV_DRAFT_MAX_TOPK;
constexpr int kMaxCand = kMaxK * kMaxK;                 // candidates of one level
constexpr int kMaxRows = 1 + (TV_DRAFT_MAX_DEPTH - 1) * kMaxK;
constexpr int kMinChunk = kChunkThreads * kSmallPer4 * 4;
constexpr int kMaxChunks = (TV_DRAFT_MAX_VOCAB + kMinChunk - 1) / kMinChunk;
static_assert(kMaxChunks <= 64, "one lane per chunk in the row merge");

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  for (int o = 32; o > 0; o >>= 1) v = max_u64(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(v & 0xFFFFFFFFu), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(v >> 32), lane);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Number of keys in a[q0, q1) greater than k.  a is 16-byte aligned and q0
// even: keys come in pairs from 16-byte LDS reads, eight keys per round trip.
__device__ __forceinline__ int count_greater(const uint64_t* a, int q0, int q1, uint64_t k) {
  const ulonglong2* a2 = reinterpret_cast<const ulonglong2*>(a);
  int cnt = 0, q = q0;
  for (; q + 8 <= q1; q += 8) {
    const ulonglong2 x0 = a2[q >> 1], x1 = a2[(q >> 1) + 1], x2 = a2[(q >> 1) + 2], x3 = a2[(q >> 1) + 3];
    cnt += (x0.x > k) + (x0.y > k) + (x1.x > k) + (x1.y > k) + (x2.x > k) + (x2.y > k) + (x3.x > k) +
           (x3.y > k);
  }
  for (; q + 2 <= q1; q += 2) {
    const ulonglong2 x0 = a2[q >> 1];
    cnt += (x0.x > k) + (x0.y > k);
  }
  if (q < q1) cnt += a[q] > k;
  return cnt;
}

// Row r of a sequence: r = 0 is the root's row (level 0, slot 0); r >= 1 is
// level 1 + (r - 1) / topk, slot (r - 1) % topk.
__device__ __forceinline__ int row_level(int r, int topk) { return r == 0 ? 0 : 1 + (r - 1) / topk; }
__device__ __forceinline__ int row_slot(int r, int topk) { return r == 0 ? 0 : (r - 1) % topk; }

// Six waves per SIMD: the 8192-entry variant fits in 80 registers (a
// 12-byte spill) instead of 82, so six workgroups instead of five share a
// compute unit and more loads are in flight (batched workload 146 -> 137 us,
// chain 111 -> 101 us; seven waves spill 40 bytes and lose 10 %).
template <bool kVec, int kPer4>
__global__ __launch_bounds__(kChunkThreads) __attribute__((amdgpu_waves_per_eu(6))) void dtree_chunk_kernel(
    const float* __restrict__ logits, int depth, int topk, int V, int R, int C,
    float2* __restrict__ stats, uint64_t* __restrict__ keys) {
  __shared__ float s_m[kChunkThreads / 64], s_s[kChunkThreads / 64];
  __shared__ uint64_t s_grp[kGroups];
  __shared__ __attribute__((aligned(16))) uint64_t s_cand[kCandCap];
  __shared__ uint64_t s_wk[kChunkThreads / 64];
  __shared__ uint64_t s_T;
  __shared__ int s_n;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long sr = blockIdx.x / C;  // (sequence, row) index
  const int c = static_cast<int>(blockIdx.x - sr * C);
  const long b = sr / R;
  const int r = static_cast<int>(sr - b * R);
  const float* row = logits + ((b * depth + row_level(r, topk)) * topk + row_slot(r, topk)) * static_cast<long>(V);
  constexpr int kChunk = kChunkThreads * kPer4 * 4;
  const int lo = c * kChunk, hi = min(V, lo + kChunk);
  // entry x[4u + e] of this thread is lo + 4 (u * 256 + tid) + e: indices
  // increase with (u, e)
  float x[4 * kPer4];
  if (kVec) {
    const f32x4* r4 = reinterpret_cast<const f32x4*>(row + lo);
    const int n4 = (hi - lo) >> 2;
#pragma unroll
    for (int u = 0; u < kPer4; ++u) {
      const int q = u * kChunkThreads + tid;
      const f32x4 v = q < n4 ? __builtin_nontemporal_load(r4 + q)
                             : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * u + e] = v[e];
    }
  } else {
#pragma unroll
    for (int u = 0; u < kPer4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = lo + 4 * (u * kChunkThreads + tid) + e;
        x[4 * u + e] = idx < hi ? row[idx] : -INFINITY;
      }
  }
  if (tid == 0) {
    s_n = 0;
    s_T = 0ull;
  }

  // this thread's best entry (strict '>' keeps the lowest index of equals),
  // which is also its maximum; entries past the row end are -inf
  float bv = -INFINITY;
  int bi = -1;
#pragma unroll
  for (int u = 0; u < kPer4; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = lo + 4 * (u * kChunkThreads + tid) + e;
      if (idx < hi && (bi < 0 || x[4 * u + e] > bv)) {
        bv = x[4 * u + e];
        bi = idx;
      }
    }
  uint64_t gk = bi < 0 ? 0ull : make_key(bv, static_cast<uint32_t>(bi));
  gk = max_u64(gk, __shfl_xor(gk, 1, 64));
  gk = max_u64(gk, __shfl_xor(gk, 2, 64));
  gk = max_u64(gk, __shfl_xor(gk, 4, 64));
  if ((tid & 7) == 0) s_grp[tid >> 3] = gk;
  // sum of exp(x - thread max), then rescaled to the wave maximum; the chunk
  // combines the waves at the end
  float s = 0.f;
  if (bi >= 0) {
#pragma unroll
    for (int i = 0; i < 4 * kPer4; ++i) s += __expf(x[i] - bv);
  }
  const float mw = wave_max(bv);
  s = wave_sum(bi >= 0 ? s * __expf(bv - mw) : 0.f);
  if (lane == 0) {
    s_m[wave] = mw;
    s_s[wave] = s;
  }
  __syncthreads();
  // cut: the topk-th largest group maximum (0 when fewer than topk groups
  // hold an entry: then every entry passes)
  if (tid < kGroups) {
    const uint64_t mine = s_grp[tid];
    int rank = 0;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) rank += s_grp[g] > mine;
    if (mine != 0ull && rank == topk - 1) s_T = mine;
  }
  __syncthreads();
  const uint64_t T = s_T;
  const float tval = T == 0ull ? -INFINITY : key_value(T);
#pragma unroll
  for (int u = 0; u < kPer4; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = lo + 4 * (u * kChunkThreads + tid) + e;
      if (idx < hi && x[4 * u + e] >= tval) {
        const uint64_t k = make_key(x[4 * u + e], static_cast<uint32_t>(idx));
        if (k >= T) {
          const int pos = atomicAdd(&s_n, 1);
          if (pos < kCandCap) s_cand[pos] = k;
        }
      }
    }
  __syncthreads();
  const int n = s_n;
  uint64_t* out = keys + (sr * C + c) * topk;
  if (n <= kCandCap) {
    for (int p = tid; p < n; p += kChunkThreads) {
      const uint64_t k = s_cand[p];
      const int rank = count_greater(s_cand, 0, n, k);
      if (rank < topk) out[rank] = k;
    }
    for (int q = n + tid; q < topk; q += kChunkThreads) out[q] = 0ull;
  } else {
    // many entries at or above the cut: topk rounds of "largest key below
    // the previous one" over the whole chunk
    uint64_t prev = ~0ull;
    for (int q = 0; q < topk; ++q) {
      uint64_t best = 0ull;
#pragma unroll
      for (int u = 0; u < kPer4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int idx = lo + 4 * (u * kChunkThreads + tid) + e;
          if (idx < hi) {
            const uint64_t k = make_key(x[4 * u + e], static_cast<uint32_t>(idx));
            if (k < prev && k > best) best = k;
          }
        }
      best = wave_max_u64(best);
      if (lane == 0) s_wk[wave] = best;
      __syncthreads();
      best = max_u64(max_u64(s_wk[0], s_wk[1]), max_u64(s_wk[2], s_wk[3]));
      if (tid == 0) out[q] = best;
      prev = best;
      __syncthreads();
    }
  }
  if (tid == 0) {
    const float m = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
    float ss = 0.f;
#pragma unroll
    for (int w = 0; w < kChunkThreads / 64; ++w)
      if (s_m[w] > -INFINITY) ss += s_s[w] * __expf(s_m[w] - m);
    stats[sr * C + c] = make_float2(m, ss);
  }
}

// Row merge (one wave per row, one lane per chunk): the row's log-sum-exp
// and its topk best keys, by the same cut-then-rank selection over the chunk
// lists (descending): T = the topk-th largest chunk maximum (0 with fewer
// than topk chunks); only lists whose maximum is at or above T hold keys at or
// above T, so at most topk^2 keys are ranked.
__global__ __launch_bounds__(64 * kRowWaves) void dtree_row_kernel(
    const float2* __restrict__ stats, const uint64_t* __restrict__ keys, int topk, int C, long rows,
    uint64_t* __restrict__ row_top, float* __restrict__ row_lse) {
  __shared__ __attribute__((aligned(16))) uint64_t s_scr[kRowWaves][kMaxCand];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long r = static_cast<long>(blockIdx.x) * kRowWaves + wave;
  const bool active = r < rows;
  uint64_t* scratch = s_scr[wave];
  int n = 0;
  if (active) {
    const long rc = r * C;
    const bool has = lane < C;
    uint64_t kk[kMaxK];
#pragma unroll
    for (int q = 0; q < kMaxK; ++q) kk[q] = (has && q < topk) ? keys[(rc + lane) * topk + q] : 0ull;
    const float2 st = has ? stats[rc + lane] : make_float2(-INFINITY, 0.f);
    const float M = wave_max(st.x);
    const float S = wave_sum(has ? st.y * __expf(st.x - M) : 0.f);
    const uint64_t head = kk[0];
    int rank = 0;
    for (int q = 0; q < C; ++q) rank += readlane_u64(head, q) > head;
    const unsigned long long hit = __ballot(has && rank == topk - 1);
    const uint64_t T = hit ? readlane_u64(head, __ffsll(static_cast<long long>(hit)) - 1) : 0ull;
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < kMaxK; ++q) cnt += (kk[q] != 0ull && kk[q] >= T);
    int incl = cnt;
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    n = min(__shfl(incl, 63, 64), kMaxCand);
    int pos = incl - cnt;
#pragma unroll
    for (int q = 0; q < kMaxK; ++q)
      if (kk[q] != 0ull && kk[q] >= T && pos < kMaxCand) scratch[pos++] = kk[q];
    if (lane == 0) row_lse[r] = M + __logf(S);
  }
  __syncthreads();
  if (active) {
    for (int p = lane; p < n; p += 64) {
      const uint64_t k = scratch[p];
      const int rk = count_greater(scratch, 0, n, k);
      if (rk < topk) row_top[r * topk + rk] = k;
    }
  }
}

// Number of entries of a descending list of distinct keys that exceed k.
__device__ __forceinline__ int count_above(const uint64_t* list, int n, uint64_t k) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (list[mid] > k) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// The level l < depth with off[l] <= p < off[l + 1], for nondecreasing
// offsets held in registers (unrolled compares, no indexed access).
__device__ __forceinline__ int level_of(int p, const int (&off)[TV_DRAFT_MAX_DEPTH + 1], int depth) {
  int l = 0;
#pragma unroll
  for (int q = 1; q < TV_DRAFT_MAX_DEPTH; ++q) l += (q < depth && off[q] <= p);
  return l;
}

__global__ __launch_bounds__(kBuildThreads) void dtree_build_kernel(
    const uint64_t* __restrict__ row_top, const float* __restrict__ row_lse, int depth, int topk, int R,
    int N, const int32_t* __restrict__ root_tokens, int32_t* __restrict__ parents,
    int32_t* __restrict__ tokens, float* __restrict__ scores) {
  __shared__ float s_lse[kMaxRows];
  __shared__ uint64_t s_top[kMaxRows * kMaxK];        // row r's best keys at r * topk + rank
  __shared__ uint64_t s_list[TV_DRAFT_MAX_DEPTH * kMaxCand];  // level l ranked at l * kMaxCand
  __shared__ __attribute__((aligned(16))) uint64_t s_tmp[kMaxCand];
  __shared__ int s_rank[kMaxCand];
  __shared__ int s_grank[TV_DRAFT_MAX_DEPTH * kMaxCand];  // global rank of each level's leading entries
  __shared__ int s_kept[TV_DRAFT_MAX_DEPTH];

  const int tid = threadIdx.x;
  const long b = blockIdx.x;
  const long seq_rows = b * R;
  for (int e = tid; e < R * topk; e += kBuildThreads) s_top[e] = row_top[seq_rows * topk + e];
  for (int e = tid; e < R; e += kBuildThreads) s_lse[e] = row_lse[seq_rows + e];
  __syncthreads();

  // ---- levels: score and rank every candidate; the rank of candidate c
  // is counted in kBuildThreads / nc parts and summed in LDS ----
  const int K2 = topk * topk;
  for (int l = 0; l < depth; ++l) {
    const int nc = l == 0 ? topk : K2;
    const uint32_t gbase = l == 0 ? 0u : static_cast<uint32_t>(topk + (l - 1) * K2);
    if (tid < nc) {
      const int j = tid / topk, rr = tid - j * topk;
      const int row = l == 0 ? 0 : 1 + (l - 1) * topk + j;
      const uint64_t tk = s_top[row * topk + rr];
      const float F = l == 0 ? 0.f : key_value(s_list[(l - 1) * kMaxCand + j]);
      const float sc = F + (key_value(tk) - s_lse[row]);
      s_tmp[tid] = make_key(sc, gbase + tid);
      s_rank[tid] = 0;
    }
    __syncthreads();
    {
      const int parts = kBuildThreads / nc;
      const int part = tid / nc, c = tid - part * nc;
      const int span = (((nc + parts - 1) / parts) + 1) & ~1;  // even: pairs of keys
      const int q0 = part * span;
      if (part < parts && q0 < nc) {
        const int cnt = count_greater(s_tmp, q0, min(nc, q0 + span), s_tmp[c]);
        if (cnt) atomicAdd(&s_rank[c], cnt);
      }
    }
    __syncthreads();
    if (tid < nc) s_list[l * kMaxCand + s_rank[tid]] = s_tmp[tid];
    __syncthreads();
  }

  // ---- global top N - 1: a prefix of every level's ranked list.  Only the
  // first m_l = min(n_l, N - 1) entries of level l can be kept; the global
  // rank of one of them is its rank in its level plus, for every other level,
  // the number of entries there that are better (one binary search per
  // (entry, other level) pair, summed in LDS).  Pair p of level l is entry
  // p - moff[l] of that level; every thread keeps the level offsets in
  // registers ----
  const int need = N - 1;
  int moff[TV_DRAFT_MAX_DEPTH + 1];
  {
    int acc = 0;
#pragma unroll
    for (int l = 0; l <= TV_DRAFT_MAX_DEPTH; ++l) {
      moff[l] = acc;
      if (l < depth) acc += min(l == 0 ? topk : K2, need);
    }
  }
  const int npairs = moff[depth < TV_DRAFT_MAX_DEPTH ? depth : TV_DRAFT_MAX_DEPTH];
  if (tid < depth) s_kept[tid] = 0;
  for (int p = tid; p < npairs; p += kBuildThreads) s_grank[p] = p - moff[level_of(p, moff, depth)];
  __syncthreads();
  if (depth > 1) {
    const int nitems = npairs * (depth - 1);
    for (int it = tid; it < nitems; it += kBuildThreads) {
      // consecutive threads take different entries against one list: their
      // LDS atomics hit different words
      int l2 = it / npairs;
      const int p = it - l2 * npairs;
      const int l = level_of(p, moff, depth);
      if (l2 >= l) ++l2;
      const uint64_t k = s_list[l * kMaxCand + (p - moff[l])];
      // entries past the first N - 1 of a level only matter as "N - 1 or more"
      const int c = count_above(s_list + l2 * kMaxCand, moff[l2 + 1] - moff[l2], k);
      if (c) atomicAdd(&s_grank[p], c);
    }
    __syncthreads();
  }
  for (int p = tid; p < npairs; p += kBuildThreads) {
    if (s_grank[p] >= need) continue;
    const int l = level_of(p, moff, depth);
    atomicMax(&s_kept[l], p - moff[l] + 1);
  }
  __syncthreads();
  // labels: level by level (level offsets base[l] = 1 + kept nodes of the
  // levels above), rank order within a level
  int base[TV_DRAFT_MAX_DEPTH + 1];
  {
    int acc = 1;
#pragma unroll
    for (int l = 0; l <= TV_DRAFT_MAX_DEPTH; ++l) {
      base[l] = acc;
      if (l < depth) acc += s_kept[l];
    }
  }

  const long ob = b * N;
  if (tid == 0) {
    parents[ob] = -1;
    tokens[ob] = root_tokens ? root_tokens[b] : 0;
    if (scores) scores[ob] = 0.f;
  }
  for (int p = tid; p < need; p += kBuildThreads) {
    const int label = 1 + p;
    const int l = level_of(label, base, depth);
    const int rho = label - base[l];
    const uint64_t k = s_list[l * kMaxCand + rho];
    const uint32_t gbase = l == 0 ? 0u : static_cast<uint32_t>(topk + (l - 1) * K2);
    const int i = static_cast<int>(key_index(k) - gbase);
    if (i < 0 || i >= (l == 0 ? topk : K2)) continue;  // only non-finite scores get here
    const int j = i / topk, rr = i - j * topk;
    const int row = l == 0 ? 0 : 1 + (l - 1) * topk + j;
    if (row >= R) continue;
    parents[ob + label] = l == 0 ? 0 : base[l - 1] + j;
    tokens[ob + label] = static_cast<int32_t>(key_index(s_top[row * topk + rr]));
    if (scores) scores[ob + label] = key_value(k);
  }
}

struct Layout {
  int R, C, per4;
  size_t units;        // (sequence, row, chunk) triples
  size_t off_keys, off_top, off_lse, bytes;
};
Layout layout_for(int B, int depth, int topk, int V) {
  Layout s;
  s.R = 1 + (depth - 1) * topk;
  const int big = kChunkThreads * kBigPer4 * 4;
  const long big_units = static_cast<long>(B) * s.R * ((V + big - 1) / big);
  s.per4 = big_units < kSmallBatchUnits ? kSmallPer4 : kBigPer4;
  const int chunk = kChunkThreads * s.per4 * 4;
  s.C = (V + chunk - 1) / chunk;
  s.units = static_cast<size_t>(B) * s.R * s.C;
  const size_t rows = static_cast<size_t>(B) * s.R;
  s.off_keys = s.units * sizeof(float2);
  s.off_top = s.off_keys + s.units * topk * sizeof(uint64_t);
  s.off_lse = s.off_top + rows * topk * sizeof(uint64_t);
  s.bytes = s.off_lse + rows * sizeof(float);
  return s;
}

}  // namespace

size_t draft_tree_workspace_bytes(int B, int depth, int topk, int V) {
  return layout_for(B, depth, topk, V).bytes;
}

hipError_t launch_draft_tree(const DraftTreeArgs& a, hipStream_t stream) {
  const Layout s = layout_for(a.B, a.depth, a.topk, a.V);
  char* ws = static_cast<char*>(a.workspace);
  float2* stats = reinterpret_cast<float2*>(ws);
  uint64_t* keys = reinterpret_cast<uint64_t*>(ws + s.off_keys);
  uint64_t* top = reinterpret_cast<uint64_t*>(ws + s.off_top);
  float* lse = reinterpret_cast<float*>(ws + s.off_lse);
  const dim3 grid1(static_cast<unsigned>(s.units));
  const bool vec = (a.V & 3) == 0;
  if (s.per4 == kSmallPer4) {
    if (vec)
      hipLaunchKernelGGL((dtree_chunk_kernel<true, kSmallPer4>), grid1, dim3(kChunkThreads), 0, stream,
                         a.draft_logits, a.depth, a.topk, a.V, s.R, s.C, stats, keys);
    else
      hipLaunchKernelGGL((dtree_chunk_kernel<false, kSmallPer4>), grid1, dim3(kChunkThreads), 0, stream,
                         a.draft_logits, a.depth, a.topk, a.V, s.R, s.C, stats, keys);
  } else {
    if (vec)
      hipLaunchKernelGGL((dtree_chunk_kernel<true, kBigPer4>), grid1, dim3(kChunkThreads), 0, stream,
                         a.draft_logits, a.depth, a.topk, a.V, s.R, s.C, stats, keys);
    else
      hipLaunchKernelGGL((dtree_chunk_kernel<false, kBigPer4>), grid1, dim3(kChunkThreads), 0, stream,
                         a.draft_logits, a.depth, a.topk, a.V, s.R, s.C, stats, keys);
  }
  const long rows = static_cast<long>(a.B) * s.R;
  hipLaunchKernelGGL(dtree_row_kernel, dim3(static_cast<unsigned>((rows + kRowWaves - 1) / kRowWaves)),
                     dim3(64 * kRowWaves), 0, stream, stats, keys, a.topk, s.C, rows, top, lse);
  hipLaunchKernelGGL(dtree_build_kernel, dim3(a.B), dim3(kBuildThreads), 0, stream, top, lse, a.depth,
                     a.topk, s.R, a.N, a.root_tokens, a.parents, a.tokens, a.scores);
  return hipGetLastError();
}

}  // namespace tv
