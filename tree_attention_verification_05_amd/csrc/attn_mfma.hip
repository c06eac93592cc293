// Tree-masked paged attention on the gfx950 matrix cores (bf16 in, fp32
// accumulate).  ("vLLM-TreeEagle" README, 核心组件 item 1 and 技术创新点 1: all
// candidate paths are verified in one pass under a tree attention mask;
// "EAGLE代码实现原理", 树结构缓冲: the common prefix is shared; "P-EAGLE",
// 技术原理和实现方式 step 3.)
//
// Work unit: a segment is (sequence b, KV head kh, row chunk).  The query
// rows of a KV head are its g = Hq/Hkv heads times the N tree nodes (row r =
// node * g + head-in-group), so one K/V tile read from HBM serves every node
// and every query head of the group.  Each of the NW waves owns 32 rows
// (waves past the last row only help load tiles).  Sequences differ in
// length, so the tiles of all segments are laid end to end and every
// workgroup takes an equal share of that flat range (see balanced_start).
// A segment cut between workgroups is merged by the workgroup that finishes
// its last piece, or, where segments are cut into many pieces, by a second
// kernel.
//
// Memory pipeline: 32-key tiles stream from HBM straight into LDS with
// buffer_load_dwordx4 ... lds (each lane's 16 bytes land at the wave's LDS
// base + 16 * lane; no registers are staged), through a ring of kStages LDS
// buffers.  Iteration t computes the scores of tile t + 1 while it runs the
// softmax and the PV product of tile t, so two buffers are being read and
// kStages - 2 tiles are in flight.  Each wave waits only for its own copies
// of tile t + 1 (s_waitcnt vmcnt with the number of copies it has issued
// since), then one s_barrier makes every wave's copies visible and frees the
// buffer of tile t - 1.  The block ids of a tile are two wave-uniform table
// entries read with scalar loads one tile ahead; a copy's source is that
// block's base plus a per-thread offset.
//
// Per tile, with lanes l and l+32 sharing query row l % 32:
//   S^T (32 keys x rows)  = K (keys x D) * Q^T (D x rows)   v_mfma_f32_32x32x16_bf16
//   O^T (D x rows)       += V^T (D x keys) * P^T (keys x rows)
// In the transposed form every accumulator a lane holds belongs to one row,
// so softmax rescaling is a per-lane scalar, and the score accumulators are
// already the B operand of the PV product.  The V^T operand is read from the
// row-major V tile with ds_read_b64_tr_b16 (inline assembly, waited for
// explicitly; see ds_read_tr16_b64): in each 16-lane group, lane j
// receives element j % 4 of the 8 bytes addressed by lanes j/4, j/4+4,
// j/4+8 and j/4+12; pointing lanes 4k..4k+3 of a group at key k (four dims
// each) hands every lane four keys of its own dim, in the key order of P^T.
//
// LDS layouts (bf16 elements, one buffer = K tile then V tile, [key][D]):
//   K: 16-byte chunk c of key k stored at chunk c ^ (k % 8)
//   V: 16-byte chunk c of key k stored at chunk c ^ (2 * (k % 4))
// The K swizzle spreads the QK operand reads (8 keys, one chunk) and the V
// swizzle the transpose reads (4 keys x 2 chunks per 16 lanes) over all
// banks.  The copies realise a swizzle by choosing which global chunk each
// lane fetches.
//
// Softmax: scores stay raw; p = exp2(s * scale*log2(e) - m) with one FMA and
// one v_exp_f32.  The running maximum m is only raised when a row's new tile
// maximum exceeds it by more than 2^8 (so p <= 256 otherwise); rescaling the
// output accumulators is then rare and happens under a wave-uniform branch.
// The result is the same softmax: numerator and denominator use the same m.
// Prefix tiles need no mask; tiles that reach the tree slots select -inf for
// keys outside the row's ancestor set (branch-free).  A segment shared by
// several workgroups leaves per piece its row maxima and sums (fp32) and its
// normalised output (bf16: the final output is bf16, and the merge is a
// convex combination of these), merged with the log-sum-exp rule.
#include <type_traits>

#include "tv_internal.h"

namespace tv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 32;             // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyRescale = 8.0f;  // log2 units a row maximum may grow before rescaling

template <int D, int NW>
struct Cfg {
  static constexpr int kThreads = NW * 64;
  static constexpr int kChunks = D / 8;                   // 16-byte chunks per key row
  static constexpr int kKeysPerCopy = 64 / kChunks;       // keys one wave copy instruction covers
  static constexpr int kCopiesPerTile = kTile / kKeysPerCopy;  // wave copies per K (or V) tile
  static constexpr int kCopiesPerWave = kCopiesPerTile / NW;
  static constexpr int kKs = D / 16;  // k-steps of the QK product
  static constexpr int kDb = D / 32;  // 32-dim output blocks
  static constexpr int kTileElems = kTile * D;             // one K (or V) tile
  static constexpr int kStageElems = 2 * kTileElems;       // K + V
  static constexpr int kRows = NW * 32;                    // rows per workgroup
  static constexpr int kDmaPerTile = 2 * kCopiesPerWave;   // copies per wave per tile (K and V)
  // LDS buffers (kStages - 2 tiles in flight): 4 (64 KB at D = 128) lets two
  // 4-wave workgroups share a compute unit.  (Six buffers for a grid of one
  // workgroup per unit measured no faster: a lone wave's per-tile latency,
  // not the copies in flight, sets its pace.)
  static constexpr int kStages = 4;
  static_assert(kCopiesPerTile % NW == 0, "every wave issues the same number of copies");
};

struct MfmaParams {
  int grid;        // workgroups launched (G)
  int balanced;    // 1: equal shares of the flat tile range; 0: fixed pieces per segment
  int T;           // fixed: tiles per piece; balanced: smallest share
  int pieces;      // fixed: pieces per segment
  int row_chunks;  // row chunks per KV head
  int waves;       // waves per workgroup (32 rows each)
  int fused_merge; // balanced: the last piece of a cut segment merges it (else a second kernel)
  int merge_split; // balanced, second kernel: merge workgroups per cut record
};

// workspace: kMaxCounters arrival counters (int32; fused balanced merges use
// one per share and lane; zero between calls, since the last arrival of a
// cut sequence resets its counter); balanced shares: a header for the second
// merge kernel (flat positions S, the share boundaries' pair length Tp and
// first-share length Te, then one cut record of four int32 per share); then
// the partial slots (2G balanced, G fixed) of kRows rows each.  The counters
// have the same place and size for every shape, so one workspace,
// zero-filled once, serves calls of any shape.
constexpr int kMaxCounters = 512;
constexpr size_t kCounterBytes = kMaxCounters * sizeof(int);
__host__ __device__ constexpr size_t header_bytes(int shares) {
  return (16 + 16 * static_cast<size_t>(shares) + 255) / 256 * 256;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Partial states after the header: normalised outputs O / l as bf16,
// [slot][D/4][row] with 8 bytes per four dims, then the row maxima m (log2
// units, scaled) and row sums l, [slot][row] fp32.  nslots counts slot rows.
struct PartialView {
  u32x2* o;
  float* m;
  float* l;
};
template <int D>
__device__ __forceinline__ PartialView partial_view_at(void* ws, size_t hbytes, size_t nslots) {
  char* base = static_cast<char*>(ws) + hbytes;
  PartialView v;
  v.o = reinterpret_cast<u32x2*>(base);
  v.m = reinterpret_cast<float*>(base + nslots * D * 2);
  v.l = v.m + nslots;
  return v;
}
template <int D>
__device__ __forceinline__ PartialView partial_view(const AttnArgs& a, const MfmaParams& mp, int G) {
  const size_t nslots = static_cast<size_t>(mp.balanced ? 2 * G : G) * (mp.waves * 32);
  const size_t hbytes = mp.balanced ? header_bytes(G / (a.Hkv * mp.row_chunks)) : 0;
  return partial_view_at<D>(a.workspace, kCounterBytes + hbytes, nslots);
}

// v_cvt_pk_bf16_f32: round to nearest even
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

// Partial states that a workgroup on another XCD merges within the same
// kernel (balanced shares) are stored and loaded at agent scope: the stores
// write through this XCD's L2 (sc1) and the loads bypass the reader's (sc1),
// so no L2 write-back or invalidation of the whole cache is needed (agent
// fences cost both, on every workgroup).
__device__ __forceinline__ void store_agent(u32x2* p, u32x2 v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32x2 load_agent(u32x2* p) {
  return __builtin_bit_cast(u32x2, __hip_atomic_load(reinterpret_cast<uint64_t*>(p), __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ float load_agent(float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The log-sum-exp fold of one item (four dims of one row) over a group of
// kGroup pieces: row maxima m (log2 units, scaled), row sums l and the
// normalised outputs ov (bf16 pairs).  The running state (M, L, o) starts at
// (-inf, 0, 0); a piece without visible keys (or an empty one) has m = -inf
// and contributes nothing, whatever its other values.
template <int kGroup>
__device__ __forceinline__ void fold_pieces(float& M, float& L, float (&o)[4], const float (&m)[kGroup],
                                            const float (&l)[kGroup], const u32x2 (&ov)[kGroup]) {
  float Mn = M;
#pragma unroll
  for (int j = 0; j < kGroup; ++j) Mn = fmaxf(Mn, m[j]);
  if (Mn == -INFINITY) return;  // no visible key in any piece so far
  const float sc = exp2_fast(M - Mn);  // 0 while M is -inf
  L *= sc;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] *= sc;
#pragma unroll
  for (int j = 0; j < kGroup; ++j) {
    const bool use = m[j] != -INFINITY;
    const float w = use ? exp2_fast(m[j] - Mn) * l[j] : 0.f;
    L += w;
    const float x0 = __uint_as_float(ov[j][0] << 16), x1 = __uint_as_float(ov[j][0] & 0xFFFF0000u);
    const float x2 = __uint_as_float(ov[j][1] << 16), x3 = __uint_as_float(ov[j][1] & 0xFFFF0000u);
    o[0] += use ? w * x0 : 0.f;
    o[1] += use ? w * x1 : 0.f;
    o[2] += use ? w * x2 : 0.f;
    o[3] += use ? w * x3 : 0.f;
  }
  M = Mn;
}

// bf16 output of one item: four dims of chunk row r (row r = node * g + head
// in group) of KV head kh
__device__ __forceinline__ void store_item(const AttnArgs& a, int D, int b, int kh, int r, int q, const float (&o)[4],
                                           float L) {
  const int g = a.Hq / a.Hkv;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const int node = r / g, hg = r % g;
  uint16_t* op = static_cast<uint16_t*>(a.out) + ((static_cast<size_t>(b) * a.N + node) * a.Hq + kh * g + hg) * D + 4 * q;
  u32x2 w;
  w[0] = pack_bf16x2(o[0] * inv, o[1] * inv);
  w[1] = pack_bf16x2(o[2] * inv, o[3] * inv);
  *reinterpret_cast<u32x2*>(op) = w;
}

// op(x[l], x[l ^ 32]) for every lane l, with one v_permlane32_swap
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ds_read_b64_tr_b16 issued as inline assembly, at a byte address plus an
// immediate offset.  The compiler cannot tell this LDS read from the
// in-flight LDS copies and would drain them all (vmcnt(0)) before it; the
// caller instead waits with lds_wait_operands, which the copies into other
// buffers never block.
// The destination is an output bound to the caller's register (no value is
// returned, so no temporary stands between the read and the wait).
template <int OFF>
__device__ __forceinline__ void ds_read_tr16_b64(u32x2& dst, uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(dst) : "v"(addr), "i"(OFF));
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// s_waitcnt lgkmcnt(0) taking the transpose-read destinations themselves as
// operands, so that no use of them is scheduled above the wait.  The asm
// reads' outputs are bound to exactly these registers and nothing is built
// from them before the wait: the compiler takes an asm output as written when
// the asm statement ends, so any copy or repacking of a destination placed
// before the wait would read the register before the LDS data arrived.
// (device-only: the register constraints do not exist on the host side of
// the compilation)
__device__ __forceinline__ void lds_wait_operands(u32x2 (&v)[2][4][2]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(v[0][0][0]), "+v"(v[0][0][1]), "+v"(v[0][1][0]), "+v"(v[0][1][1]),
                 "+v"(v[0][2][0]), "+v"(v[0][2][1]), "+v"(v[0][3][0]), "+v"(v[0][3][1]),
                 "+v"(v[1][0][0]), "+v"(v[1][0][1]), "+v"(v[1][1][0]), "+v"(v[1][1][1]),
                 "+v"(v[1][2][0]), "+v"(v[1][2][1]), "+v"(v[1][3][0]), "+v"(v[1][3][1]));
}
__device__ __forceinline__ void lds_wait_operands(u32x2 (&v)[2][2][2]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(v[0][0][0]), "+v"(v[0][0][1]), "+v"(v[0][1][0]), "+v"(v[0][1][1]),
                 "+v"(v[1][0][0]), "+v"(v[1][0][1]), "+v"(v[1][1][0]), "+v"(v[1][1][1]));
}

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
}

// Visibility of the 64 keys starting at logical position tb, for a row whose
// node has ancestor-or-self bits mw: bit k is set iff position tb + k is in
// the prefix or is a tree slot of one of those nodes.  Bits of nodes >= N are
// zero in mw, so positions past the end are hidden.  Every condition depends
// only on (tb, P) and is uniform across the wave.
__device__ __forceinline__ uint64_t tile_visibility(const uint64_t (&mw)[4], int tb, int P) {
  const int npre = P - tb;
  uint64_t vis = npre >= 64 ? ~0ull : (npre <= 0 ? 0ull : ((1ull << npre) - 1ull));
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int pos = P + 64 * k - tb;  // position (relative to tb) of tree node 64k
    if (pos >= 0 && pos < 64)
      vis |= mw[k] << pos;
    else if (pos < 0 && pos > -64)
      vis |= mw[k] >> (-pos);
  }
  return vis;
}

// ---------------- block-wide integer helpers ----------------
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int w = __shfl_up(v, o, 64);
    if (lane >= o) v += w;
  }
  return v;
}

__device__ __forceinline__ int clamp_prefix(const AttnArgs& a, int P) {
  return P < 0 ? 0 : (P > a.max_prefix_len ? a.max_prefix_len : P);
}
// tiles of a sequence with prefix length P: prefix plus tree slots, 32 keys each
__device__ __forceinline__ int tiles_of(const AttnArgs& a, int P) { return (P + a.N + kTile - 1) / kTile; }

// Work decomposition.  A segment is (sequence b, KV head kh, row chunk rc),
// numbered ((b * Hkv) + kh) * row_chunks + rc; a segment of sequence b has
// tiles_of(P_b) tiles.
//
// Fixed pieces (one sequence): every segment is cut into `pieces` pieces of
// T tiles (sized for the longest prefix); workgroup u runs piece u % pieces
// of segment u / pieces and, unless that piece is the whole segment, leaves
// its partial state in slot u.
//
// Balanced shares (several sequences, whose lengths only the device knows):
// a lane is (KV head kh, row chunk rc), and the G workgroups split into
// G / lanes shares per lane, workgroup u taking lane u % lanes and share
// v = u / lanes, so the workgroups that run at the same time stream the same
// blocks for every head.  Within a lane the tiles of all sequences, in order,
// form one flat range of S tiles, cut into shares of T = max(minimum,
// ceil(S / shares)) tiles.  Workgroup u runs every sequence its share
// [v T, v T + T) touches: a sequence inside the share is written straight to
// `out`, and one cut by a share boundary leaves its partial state in slot u
// (the share's first sequence) or G + u (its last).  Workgroup 0 stores S and
// T in the workspace header, and lane 0 of every share the cut at its start.
//
// Workgroup placement: the hardware hands workgroups to the 8 XCDs round
// robin (u % 8).  With several row chunks per KV head, the chunks of one
// (share, KV head) are given to workgroups u, u + 8, ... of one XCD, which
// start together and share the K/V tiles through that XCD's L2.
// Every sequence also carries kSeqCostTiles positions before its tiles in
// the flat range: a share pays for each sequence boundary it crosses (the
// piece's epilogue stores, the next piece's query loads and its pipeline
// refill), measured at 7-9 us, about six tiles, per extra piece on the
// batched and 70B-chain workloads.  Shares stay equal in positions, so one
// that crosses more boundaries gets fewer tiles and all end together.
constexpr int kSeqCostTiles = 6;

// Share boundaries in the flat range: shares come in pairs of Tp positions,
// the first share of a pair Te long.  Equal shares: Tp = 2 T, Te = T.
struct ShareSplit {
  int Tp, Te;
  __device__ int start(int k) const { return (k >> 1) * Tp + ((k & 1) ? Te : 0); }
  __device__ int share_of(int y) const { return 2 * (y / Tp) + ((y % Tp) >= Te ? 1 : 0); }
};

// Odd-numbered XCDs ran the attention main kernel 3-8 % slower than
// even-numbered ones on every MI355X measured (per-workgroup timestamps and
// HW_REG_XCC_ID; the same XCDs stay slow when the KV heads are moved to other
// XCDs).  With 8 lanes of one row chunk, workgroups are placed so that the
// even shares of every lane run on even XCDs and the odd shares on odd XCDs,
// and an even share takes kEvenShare / kShareWeight of each pair.
constexpr int kEvenShare = 103;
constexpr int kShareWeight = 200;

struct Start {
  int S;           // flat positions (tiles plus per-sequence cost)
  ShareSplit sp;   // share boundaries
  int b, base;     // sequence holding the share's first position (-1: none), and its first position
  int ntiles;      // tiles of sequence b (its tiles start at base + kSeqCostTiles)
};

template <int NW>
__device__ Start balanced_start(const AttnArgs& a, int shares, int share_idx, int min_tiles, bool xcd_weighted,
                               int* red, int* found) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  Start st;
  // pass 1: tiles of one lane (and the prefix-length check)
  int local = 0;
  for (int b = tid; b < a.B; b += NW * 64) {
    const int P = a.prefix_lens[b];
    if (P < 0 || P > a.max_prefix_len) report(a.dev_status, TV_DEV_BAD_CACHE);
    local += kSeqCostTiles + tiles_of(a, clamp_prefix(a, P));
  }
  local = wave_sum(local);
  if (lane == 0) red[wave] = local;
  __syncthreads();
  int tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) tot += red[w];
  __syncthreads();
  st.S = tot;
  if (xcd_weighted) {
    const int pair = (2 * st.S + shares - 1) / shares;
    st.sp.Tp = pair > 2 * min_tiles ? pair : 2 * min_tiles;
    st.sp.Te = (st.sp.Tp * kEvenShare + kShareWeight - 1) / kShareWeight;
  } else {
    const int even = (st.S + shares - 1) / shares;
    const int T = even > min_tiles ? even : min_tiles;
    st.sp.Tp = 2 * T;
    st.sp.Te = T;
  }
  const int j0 = st.sp.start(share_idx);
  if (j0 >= st.S) {
    st.b = -1;
    return st;
  }
  // pass 2: the sequence whose tiles hold j0
  int running = 0;
  for (int c = 0; c < a.B; c += NW * 64) {
    const int b = c + tid;
    const int v = b < a.B ? kSeqCostTiles + tiles_of(a, clamp_prefix(a, a.prefix_lens[b])) : 0;
    const int incl = wave_inclusive_scan(v, lane);
    if (lane == 63) red[wave] = incl;
    __syncthreads();
    int before = 0, chunk = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int x = red[w];
      before += w < wave ? x : 0;
      chunk += x;
    }
    const int start = running + before + incl - v;
    if (b < a.B && start <= j0 && j0 < start + v) {
      found[0] = b;
      found[1] = start;
      found[2] = v;
    }
    running += chunk;
    __syncthreads();
  }
  st.b = found[0];
  st.base = found[1];
  st.ntiles = found[2] - kSeqCostTiles;
  return st;
}

// POLICY: the cache policy of the K/V copies (kNonTemporal when each tile is
// read by one workgroup only, i.e. one row chunk per KV head).
template <int D, int NW, int POLICY>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_mfma_kernel(AttnArgs a, MfmaParams mp) {
  using C = Cfg<D, NW>;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  __shared__ int red[NW];
  __shared__ int found[3];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the wave index is uniform across the wave; saying so keeps block bases,
  // buffer descriptors and LDS destinations in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5;   // which half of the key set this lane holds
  const int col = lane & 31;  // query row within the wave's 32 rows
  const int g = a.Hq / a.Hkv;
  const int R = g * a.N;
  const int W = (a.N + 63) >> 6;
  const int segs = a.Hkv * mp.row_chunks;  // segments per sequence
  const int G = static_cast<int>(gridDim.x);
  const int u = blockIdx.x;
  const char* kcb = static_cast<const char*>(a.k_cache);
  const char* vcb = static_cast<const char*>(a.v_cache);
  const float c = a.scale * kLog2e;
  const long block_stride = static_cast<long>(kBlockSize) * a.Hkv * D;  // elements per block

  // ---------------- per-thread parts of the copy and read addresses ----------------
  // Wave copy i of a K (or V) tile covers keys i*kKeysPerCopy .. +kKeysPerCopy-1
  // (all in one 16-token block); lane l writes chunk position l % kChunks of
  // key i*kKeysPerCopy + l / kChunks.  The source address is a wave-uniform
  // block-and-head base plus a per-thread offset fixed for the whole kernel.
  // (byte offsets from the block's row of head kh at slot 0; the block and
  // head go into the buffer descriptor, and consecutive slots of a head are
  // kv_slot_rows rows apart)
  int off_k[C::kCopiesPerWave], off_v[C::kCopiesPerWave];
  {
    const int ckey = lane / C::kChunks, cpos = lane % C::kChunks;
#pragma unroll
    for (int jj = 0; jj < C::kCopiesPerWave; ++jj) {
      const int key = (jj * NW + wave) * C::kKeysPerCopy + ckey;
      const int row = (key & 15) * a.kv_slot_rows * D;
      off_k[jj] = (row + (cpos ^ (key & 7)) * 8) * 2;
      off_v[jj] = (row + (cpos ^ (2 * (key & 3))) * 8) * 2;
    }
  }
  // LDS read addresses: a per-lane base plus a compile-time offset (stage,
  // k-step, key chunk, dim block).  K: chunk c = 2 kk + hh of key `col` sits at
  // c ^ (col % 8), which is (2 (kk % 4) + hh) ^ (col % 8) plus 8 (kk / 4).
  // V^T: in each 16-lane group, lanes 4k..4k+3 point at key row
  // 4 hh + k (+ 16 per key chunk, + 8 for its upper 8 keys), dims
  // 8 ((4 db + 2 (lane/16 % 2) + lane/2 % 2) ^ 2 (k % 4)) + 4 (lane % 2);
  // (4 db + x) ^ y with x, y < 8 is (4 (db % 2) + x) ^ y plus 8 (db / 2).
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LDS_AS const void*)lds));
  uint32_t kaddr[4], vaddr[2];
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4) kaddr[k4] = lds0 + 2 * (col * D + (((2 * k4 + hh) ^ (col & 7)) * 8));
  {
    const int tq = lane >> 4, ts = lane & 15;
    const int tr_row = 4 * hh + (ts >> 2);
    const int tr_chunk = 2 * (tq & 1) + ((ts & 3) >> 1);
    const int tr_half = (ts & 1) * 4;
    const int tr_swz = 2 * ((ts >> 2) & 3);
#pragma unroll
    for (int d2 = 0; d2 < 2; ++d2)
      vaddr[d2] = lds0 + 2 * (C::kTileElems + tr_row * D + (((4 * d2 + tr_chunk) ^ tr_swz) * 8) + tr_half);
  }

  // One piece: tiles [t0, t1) of segment (b, kh, rc) whose sequence has
  // prefix length P (raw, checked here).  `whole` pieces write bf16 outputs,
  // the others their partial state into `slot`.
  // ids[2 i], ids[2 i + 1]: block ids of tile t0 + i, i < kStages, when
  // `have_ids` (read by the caller before the prefix length arrived)
  auto run_piece = [&](int b, int kh, int rc, int Praw, int t0, int t1, bool whole, int slot,
                       const int (&ids)[2 * C::kStages], bool have_ids) __attribute__((always_inline)) {
    // ---- this wave's 32 query rows and their mask words (issued first) ----
    const int rl = wave * 32 + col;  // row within the chunk
    const int row0 = rc * C::kRows + wave * 32;
    const bool active = row0 < R;
    const int r_me = row0 + col;
    bf16x8 qreg[C::kKs];
    uint64_t mw[4];
    const int node = (r_me < R ? r_me : R - 1) / g;
    int par_me = -1;  // without masks: this lane's node of the tree (lane < N), its parent
    {
      const int rr = r_me < R ? r_me : R - 1;
      const int hg = rr % g;
      const u32x4* qp = reinterpret_cast<const u32x4*>(
          static_cast<const uint16_t*>(a.q) +
          ((static_cast<size_t>(b) * a.N + node) * a.Hq + kh * g + hg) * D);
#pragma unroll
      for (int kk = 0; kk < C::kKs; ++kk) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r_me < R) v = qp[kk * 2 + hh];
        qreg[kk] = __builtin_bit_cast(bf16x8, v);
      }
      if (a.mask) {
        const uint64_t* mrow = a.mask + (static_cast<size_t>(b) * a.N + node) * W;
#pragma unroll
        for (int w = 0; w < 4; ++w) mw[w] = (w < W) ? mrow[w] : 0ull;
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) mw[w] = 0ull;
        if (lane < a.N) par_me = a.parents[static_cast<size_t>(b) * a.N + lane];
      }
    }

    // ---- block ids: scalar loads through the constant address space, which
    // never wait behind the in-flight tile copies; reads stop at the table
    // row's end, and entries past the sequence's blocks are replaced by 0 ----
    const int32_t* table = a.block_table + static_cast<size_t>(b) * a.max_blocks;
    const CONST_AS int32_t* table_s = (const CONST_AS int32_t*)table;
    const int maxb = a.max_blocks;
    auto fetch_ids = [&](int tile, int& b0, int& b1) __attribute__((always_inline)) {
      const int e0 = tile * 2;  // the tile spans table entries e0 and e0 + 1
      b0 = e0 < maxb ? table_s[e0] : 0;
      b1 = e0 + 1 < maxb ? table_s[e0 + 1] : 0;
    };
    // the ring's first kStages tiles: all loads issued together
    int pid[2 * C::kStages];
#pragma unroll
    for (int i = 0; i < C::kStages; ++i) {
      if (have_ids) {
        pid[2 * i] = ids[2 * i];
        pid[2 * i + 1] = ids[2 * i + 1];
      } else {
        fetch_ids(t0 + i, pid[2 * i], pid[2 * i + 1]);
      }
    }
    int nb0 = pid[2 * (C::kStages - 1)], nb1 = pid[2 * C::kStages - 1];  // the next tile to issue

    const bool bad_len = Praw < 0 || Praw > a.max_prefix_len;
    const int P = clamp_prefix(a, Praw);
    const int nblk = (P + a.N + kBlockSize - 1) / kBlockSize;
    // buffer descriptors per (cache, block): base = the block's row of head
    // kh at slot 0; the range ends with that head's last slot row, so a stray
    // offset reads zeros
    const long block_bytes = block_stride * 2;
    const long head_bytes = static_cast<long>(kh) * a.kv_head_rows * D * 2;
    const int range = ((kBlockSize - 1) * a.kv_slot_rows + 1) * D * 2;
    auto issue_tile = [&](int stage, int tile, int b0, int b1) __attribute__((always_inline)) {
      const int e0 = tile * 2;
      b0 = e0 < nblk ? b0 : 0;
      b1 = e0 + 1 < nblk ? b1 : 0;
      // an id outside the cache is reported and replaced by block 0 (finite values)
      if (b0 < 0 || b0 >= a.num_blocks || b1 < 0 || b1 >= a.num_blocks) {
        if (tid == 0) report(a.dev_status, TV_DEV_BAD_CACHE);
        b0 = (b0 >= 0 && b0 < a.num_blocks) ? b0 : 0;
        b1 = (b1 >= 0 && b1 < a.num_blocks) ? b1 : 0;
      }
      uint16_t* kst = lds + stage * C::kStageElems;
      uint16_t* vst = kst + C::kTileElems;
#pragma unroll
      for (int jj = 0; jj < C::kCopiesPerWave; ++jj) {
        const int copy = jj * NW + wave;
        const int blk = copy * C::kKeysPerCopy < kBlockSize ? b0 : b1;
        const long src = blk * block_bytes + head_bytes;
        copy_to_lds<POLICY>(kcb + src, range, off_k[jj], kst + copy * 512);
        copy_to_lds<POLICY>(vcb + src, range, off_v[jj], vst + copy * 512);
      }
    };

    f32x16 acc[C::kDb];
#pragma unroll
    for (int db = 0; db < C::kDb; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
    float m_c = -INFINITY;  // running maximum, already multiplied by c
    float l_run = 0.f;

    // One tile: softmax of this tile's scores `sc` and O^T += V^T P^T, with
    // the next tile's scores S^T = K Q^T computed into `sn` in the same
    // straight-line block as the exponentials, so that the matrix cores work
    // while the vector unit runs the softmax.
    auto tile_body = [&](auto stage_c, int tile, f32x16& sc, f32x16& sn) __attribute__((always_inline)) {
        constexpr int kStage = decltype(stage_c)::value;
        constexpr int kStageBytes = kStage * C::kStageElems * 2;
        constexpr int kNextBytes = ((kStage + 1) % C::kStages) * C::kStageElems * 2;
        const int tb = tile * kTile;
        // K operands of the next tile
        bf16x8 kop[C::kKs];
    #pragma unroll
        for (int kk = 0; kk < C::kKs; ++kk)
          kop[kk] = *reinterpret_cast<const LDS_AS bf16x8*>(
              static_cast<uintptr_t>(kaddr[kk & 3] + kNextBytes + (kk >> 2) * 128));
        // V^T operands of this tile, read now so the reads overlap the softmax
        // vtr[kc2][db][0 / 1]: keys 16 kc2 .. + 7 / 16 kc2 + 8 .. + 15
        u32x2 vtr[2][C::kDb][2];
        static_for<0, 2>([&](auto kc2_c) {
          constexpr int kc2 = decltype(kc2_c)::value;
          static_for<0, C::kDb>([&](auto db_c) {
            constexpr int db = decltype(db_c)::value;
            // bytes past vaddr: stage, key rows 16 kc2 (+ 8), dim blocks 2 (db / 2)
            constexpr int kLo = kStageBytes + 2 * (16 * kc2 * D + (db >> 1) * 64);
            constexpr int kHi = kLo + 2 * 8 * D;
            // the offset field holds 16 bits: far stages step the base by 64 KB
            constexpr int kLoB = kLo >= 65536 ? 65536 : 0, kHiB = kHi >= 65536 ? 65536 : 0;
            ds_read_tr16_b64<kLo - kLoB>(vtr[kc2][db][0], vaddr[db & 1] + kLoB);
            ds_read_tr16_b64<kHi - kHiB>(vtr[kc2][db][1], vaddr[db & 1] + kHiB);
          });
        });
        if (tb + kTile > P) {  // the tile reaches the tree slots or the end: mask
          const uint64_t vis = tile_visibility(mw, tb, P) >> (4 * hh);
    #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int bit = 8 * (r >> 2) + (r & 3);
            sc[r] = ((vis >> bit) & 1ull) ? sc[r] : -INFINITY;
          }
        }
        float mt = sc[0];
    #pragma unroll
        for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sc[r]);
        mt = pair_max(mt) * c;
        // lazy rescale: raise m only when a row's maximum grew by more than 2^8
        const bool grow = mt > m_c + kLazyRescale;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
          const float mn = grow ? mt : m_c;
          // rows that do not grow keep alpha = 1 (their m may still be -inf)
          const float alpha = grow ? exp2_fast(m_c - mn) : 1.f;  // 0 on the first visible keys
          m_c = mn;
          l_run *= alpha;
    #pragma unroll
          for (int db = 0; db < C::kDb; ++db)
    #pragma unroll
            for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
        }
        const float mcs = (m_c == -INFINITY) ? 0.f : m_c;  // no visible key yet: p = 0
        // the next tile's scores: independent of the softmax below, which the
        // compiler interleaves with these MFMAs
        sn = f32x16{};
    #pragma unroll
        for (int kk = 0; kk < C::kKs; ++kk) sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kk], qreg[kk], sn, 0, 0, 0);
        u32x4 pw[2];
        float lsum0 = 0.f, lsum1 = 0.f;
    #pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = exp2_fast(__builtin_fmaf(sc[r], c, -mcs));
          const float p1 = exp2_fast(__builtin_fmaf(sc[r + 1], c, -mcs));
          lsum0 += p0;
          lsum1 += p1;
          pw[r >> 3][(r >> 1) & 3] = pack_bf16x2(p0, p1);
        }
        l_run += lsum0 + lsum1;
        // the transpose reads above are invisible to the compiler's wait
        // tracking: wait for them here, with their results as operands so that
        // no use can be scheduled above the wait
        lds_wait_operands(vtr);
        // O^T += V^T P^T over the two 16-key chunks of the tile (the V^T
        // operands are assembled from the transpose reads only now)
    #pragma unroll
        for (int kc2 = 0; kc2 < 2; ++kc2) {
          const bf16x8 pb = __builtin_bit_cast(bf16x8, pw[kc2]);
    #pragma unroll
          for (int db = 0; db < C::kDb; ++db) {
            const u32x4 vop = {vtr[kc2][db][0][0], vtr[kc2][db][0][1], vtr[kc2][db][1][0], vtr[kc2][db][1][1]};
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vop), pb, acc[db], 0, 0, 0);
          }
        }
        if constexpr (POLICY != kNonTemporal) {
          // Several row chunks per KV head share each K/V tile through the
          // L2, and the matrix cores, not HBM, set the pace.  A wave issues
          // in order, so the next tile's eight dependent score MFMAs, left
          // back to back, would stall it for their whole latency: interleave
          // three VALU instructions of the softmax after each of them and
          // four after each PV MFMA (the Qwen2 workload 160.0 -> 153.5 us;
          // 6/2, 4/3, 4/4, 2/4, 2/5, 3/3 and exp-first groups measured
          // between 153 and 165 us).  The HBM-bound instance keeps the
          // compiler's order (3-4 % slower on the batched workload there).
          static_for<0, 8>([&](auto) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // three VALU
          });
          static_for<0, 8>([&](auto) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
          });
        }
    };
    // S^T of the piece's first tile
    auto compute_s = [&](auto stage_c, f32x16& sc) __attribute__((always_inline)) {
        constexpr int kStage = decltype(stage_c)::value;
        constexpr int kStageBytes = kStage * C::kStageElems * 2;
        sc = f32x16{};
    #pragma unroll
        for (int kk = 0; kk < C::kKs; ++kk) {
          const bf16x8 av = *reinterpret_cast<const LDS_AS bf16x8*>(
              static_cast<uintptr_t>(kaddr[kk & 3] + kStageBytes + (kk >> 2) * 128));
          sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qreg[kk], sc, 0, 0, 0);
        }
    };

    // wait until this wave's copies of a tile are done: `later` tiles (at
    // most C::kStages - 2) have been issued after it
    auto wait_tile = [&](int later) __attribute__((always_inline)) {
      static_assert(C::kStages >= 3 && C::kStages <= 6, "wait_tile covers 0..4 later tiles");
      if (later >= 4)
        wait_vmcnt<4 * C::kDmaPerTile>();
      else if (later == 3)
        wait_vmcnt<3 * C::kDmaPerTile>();
      else if (later == 2)
        wait_vmcnt<2 * C::kDmaPerTile>();
      else if (later == 1)
        wait_vmcnt<C::kDmaPerTile>();
      else
        wait_vmcnt<0>();
    };

    // ---- tile pipeline ----
    // Iteration `tile` reads K of tile + 1 (its scores are computed ahead,
    // overlapping this tile's softmax) and V of tile, and refills the buffer
    // of tile - 1, so kStages - 2 tiles stay in flight.
    // the ring may still be read by the previous piece's last tile (every
    // wave's LDS reads of it completed before its last MFMAs)
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    if (bad_len && tid == 0) report(a.dev_status, TV_DEV_BAD_CACHE);
#pragma unroll
    for (int i = 0; i < C::kStages - 1; ++i)
      if (t0 + i < t1) issue_tile(i, t0 + i, pid[2 * i], pid[2 * i + 1]);
    if (!a.mask && t1 * kTile > P) {
      // masks from the parents, while the first tiles are in flight (only
      // pieces that reach the tree's keys use them)
      bool bad_tree;
      const uint64_t anc = wave_tree_mask(par_me, a.N, lane, &bad_tree);
      mw[0] = __shfl(anc, node, 64);
      mw[1] = mw[2] = mw[3] = 0ull;
      if (bad_tree && tid == 0) report(a.dev_status, TV_DEV_BAD_TREE);
    }
    // tile t0 (and the query and mask loads issued before it)
    wait_tile(min(C::kStages - 2, t1 - 1 - t0));
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    // scores of two consecutive tiles, by tile parity (kStages is even), so
    // that the next tile's MFMAs never wait for this tile's softmax to read
    // its registers
    f32x16 s_buf[2];
    s_buf[1] = f32x16{};
    if (active) compute_s(std::integral_constant<int, 0>{}, s_buf[0]);
    // the loop body is unrolled over the ring, so that every LDS address is a
    // per-lane base plus a constant
    int tile = t0;
    while (tile < t1) {
      static_for<0, C::kStages>([&](auto stage_c) {
        constexpr int kStage = decltype(stage_c)::value;
        if (tile < t1) {
          const bool has_next = tile + 1 < t1;
          const int nt = tile + C::kStages - 1;
          if (has_next) {
            wait_tile(min(C::kStages - 3, t1 - 2 - tile));
            __asm__ volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();  // tile + 1 landed everywhere; tile - 1 is free
            __asm__ volatile("" ::: "memory");
            if (nt < t1) issue_tile((kStage + C::kStages - 1) % C::kStages, nt, nb0, nb1);
          }
          if (active) {
            // the last tile's "next" scores read a stale buffer and are dropped
            tile_body(stage_c, tile, s_buf[kStage & 1], s_buf[(kStage + 1) & 1]);
          }
          if (nt < t1) fetch_ids(nt + 1, nb0, nb1);  // ready by the next issue
          ++tile;
        }
      });
    }

    // ---- piece epilogue ----
    if (!active) return;
    const float lt = pair_sum(l_run);
    if (r_me >= R) return;
    if (whole) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const int node = r_me / g, hg = r_me % g;
      uint16_t* op = static_cast<uint16_t*>(a.out) +
                     ((static_cast<size_t>(b) * a.N + node) * a.Hq + kh * g + hg) * D;
#pragma unroll
      for (int db = 0; db < C::kDb; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int d = db * 32 + 8 * jj + 4 * hh;
          u32x2 w;
          w[0] = pack_bf16x2(acc[db][4 * jj] * inv, acc[db][4 * jj + 1] * inv);
          w[1] = pack_bf16x2(acc[db][4 * jj + 2] * inv, acc[db][4 * jj + 3] * inv);
          *reinterpret_cast<u32x2*>(op + d) = w;
        }
    } else {
      // the piece's normalised output O / l in bf16 (the merge weighs it by
      // l and the maximum m), [slot][D/4][row] with 8 bytes per four dims so
      // that one store instruction writes two runs of 32 consecutive rows
      const size_t nslots = static_cast<size_t>(mp.balanced ? 2 * G : G) * C::kRows;
      const size_t prow = static_cast<size_t>(slot) * C::kRows + rl;
      const PartialView pv = partial_view<D>(a, mp, G);
      u32x2* po = pv.o + static_cast<size_t>(slot) * (D / 4) * C::kRows + rl;
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
      for (int db = 0; db < C::kDb; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int q = db * 8 + 2 * jj + hh;  // dims 4q .. 4q + 3
          u32x2 w;
          w[0] = pack_bf16x2(acc[db][4 * jj] * inv, acc[db][4 * jj + 1] * inv);
          w[1] = pack_bf16x2(acc[db][4 * jj + 2] * inv, acc[db][4 * jj + 3] * inv);
          if (mp.fused_merge)
            store_agent(po + static_cast<size_t>(q) * C::kRows, w);
          else
            po[static_cast<size_t>(q) * C::kRows] = w;
        }
      (void)nslots;
      if (hh == 0) {
        if (mp.fused_merge) {
          store_agent(pv.m + prow, m_c);
          store_agent(pv.l + prow, lt);
        } else {
          pv.m[prow] = m_c;
          pv.l[prow] = lt;
        }
      }
    }
  };

  // workgroups are spread over the 8 XCDs round-robin (u % 8); the row chunks
  // of one (item) go to consecutive workgroups of the same XCD so that their
  // shared K/V tiles come from that XCD's L2
  int w_item, rc_p;
  {
    const int RC = mp.row_chunks;
    const int G0 = mp.balanced ? G / (8 * RC) * (8 * RC) : 0;
    if (u < G0) {
      const int x = u & 7, k = u >> 3;
      rc_p = k % RC;
      w_item = (k / RC) * 8 + x;
    } else {
      w_item = G0 / RC + (u - G0) / RC;
      rc_p = (u - G0) % RC;
    }
  }
  // 8 lanes of one row chunk and an even share count: XCD x = u % 8 runs
  // lanes x / 2 and x / 2 + 4 at shares of x's parity
  const bool xcd_weighted = mp.balanced && a.Hkv == 8 && mp.row_chunks == 1 && (G / 8) % 2 == 0;
  const int v = !mp.balanced ? ((w_item / mp.pieces) * mp.row_chunks + rc_p) * mp.pieces + w_item % mp.pieces
                : xcd_weighted ? (2 * ((u >> 3) >> 1) + (u & 1)) * 8 + ((u & 7) >> 1) + 4 * ((u >> 3) & 1)
                               : (w_item / a.Hkv) * (a.Hkv * mp.row_chunks) + (w_item % a.Hkv) * mp.row_chunks + rc_p;
  if (!mp.balanced) {
    // ---------------- fixed pieces ----------------
    const int seg_id = v / mp.pieces, piece = v % mp.pieces;
    const int b = seg_id / segs, seg = seg_id % segs;
    const int t0 = piece * mp.T;
    // the block ids of the ring's first tiles do not depend on the prefix
    // length: their loads go out together with it
    int ids[2 * C::kStages];
    {
      const CONST_AS int32_t* trow =
          (const CONST_AS int32_t*)(a.block_table + static_cast<size_t>(b) * a.max_blocks);
#pragma unroll
      for (int i = 0; i < 2 * C::kStages; ++i) {
        const int e = 2 * t0 + i;
        ids[i] = e < a.max_blocks ? trow[e] : 0;
      }
    }
    const int Praw = a.prefix_lens[b];
    const int ntiles = tiles_of(a, clamp_prefix(a, Praw));
    if (t0 >= ntiles) {
      // the sequence is shorter than the longest: an empty piece, whose row
      // maxima of -inf give it no weight in the merge
      if (tid < C::kRows) partial_view<D>(a, mp, G).m[static_cast<size_t>(v) * C::kRows + tid] = -INFINITY;
      return;
    }
    const int t1 = min(ntiles, t0 + mp.T);
    // with several pieces every piece leaves a partial state, so the merge
    // needs no sequence lengths
    run_piece(b, seg / mp.row_chunks, seg % mp.row_chunks, Praw, t0, t1, mp.pieces == 1, v, ids, true);
    return;
  }

  // ---------------- balanced shares ----------------
  const int lanes = a.Hkv * mp.row_chunks;
  const int lane_id = v % lanes, share = v / lanes;
  const int kh = lane_id / mp.row_chunks, rc = lane_id % mp.row_chunks;
  const Start st = balanced_start<NW>(a, G / lanes, share, mp.T, xcd_weighted, red, found);
  if (!mp.fused_merge) {
    // for the second merge kernel: S and the share boundaries, and the cut
    // at this share's start: the sequence it splits, the flat position of
    // that sequence's first tile and its tile count, and the cut's rank
    // among the sequence's cuts (-1: the share starts at or before a
    // sequence's first tile, or past the end)
    int* hdr = reinterpret_cast<int*>(static_cast<char*>(a.workspace) + kCounterBytes);
    if (u == 0 && tid == 0) {
      hdr[0] = st.S;
      hdr[1] = st.sp.Tp;
      hdr[2] = st.sp.Te;
    }
    if (lane_id == 0 && tid == 0) {
      int4 cut = {-1, 0, 0, 0};
      const int first_tile = st.base + kSeqCostTiles;
      if (st.b >= 0 && st.sp.start(share) > first_tile)
        cut = int4{st.b, first_tile, st.ntiles, share - st.sp.share_of(first_tile) - 1};
      reinterpret_cast<int4*>(hdr + 4)[share] = cut;
    }
  }
  if (st.b < 0) return;  // whole workgroup: the lane's tiles ended before this share
  // A sequence cut by share boundaries has one piece in each of the shares
  // f .. l of this lane that its tiles [first_tile, first_tile + nt) touch.
  // Every piece stores its partial state at agent scope, waits until each
  // wave's stores are acknowledged (written through to device-coherent
  // memory), and after a workgroup barrier counts itself in the sequence's
  // arrival counter, number f * lanes + lane (f is the share where the
  // sequence's first tile lies, and no other cut sequence of the lane starts
  // its tiles there).  The workgroup whose count completes the set resets
  // the counter to zero and merges the pieces, loading them at agent scope
  // only after its count returned.  Nothing waits for another workgroup.
  int* counters = static_cast<int*>(a.workspace);
  __shared__ int s_last;
  auto merge_if_last = [&](int bb, int first_tile, int nt) __attribute__((always_inline)) {
    const int f = st.sp.share_of(first_tile);
    const int npieces = st.sp.share_of(first_tile + nt - 1) - f + 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      int* cnt = counters + f * lanes + lane_id;
      const int before = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = before == npieces - 1;
      if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    // piece k runs in share f + k, in slot (f + k) * lanes + lane; the piece
    // in share f is in the share's second slot (G + ...) when the sequence's
    // tiles start inside that share (cut_first).  Thread t takes row
    // t % kRows of the chunk and half t / kRows of its dims, folding the
    // pieces two at a time with every load of a pair in flight together
    // (three at a time, or the merge as a separate function, raised the
    // register count or spilled, and measured slower).
    const bool cut_first = first_tile != st.sp.start(f);
    constexpr int kQ = D / 8;  // 4-dim chunks per thread
    constexpr int kFold = 2;   // pieces whose loads are in flight together
    static_assert(C::kThreads == 2 * C::kRows, "two threads per row");
    const int rl = tid % C::kRows, q0 = (tid / C::kRows) * kQ;
    if (rc * C::kRows + rl >= R) return;
    const PartialView pv = partial_view<D>(a, mp, G);
    float M = -INFINITY, L = 0.f;
    float o[kQ][4];
#pragma unroll
    for (int q = 0; q < kQ; ++q) o[q][0] = o[q][1] = o[q][2] = o[q][3] = 0.f;
    for (int k0 = 0; k0 < npieces; k0 += kFold) {
      float m[kFold], l[kFold];
      u32x2 ov[kQ][kFold];
#pragma unroll
      for (int j = 0; j < kFold; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.f;
#pragma unroll
        for (int q = 0; q < kQ; ++q) ov[q][j] = u32x2{0u, 0u};
        if (k0 + j < npieces) {
          const int vv = (f + k0 + j) * lanes + lane_id;
          const size_t sl = static_cast<size_t>((k0 + j == 0 && cut_first) ? G + vv : vv);
          m[j] = load_agent(pv.m + sl * C::kRows + rl);
          l[j] = load_agent(pv.l + sl * C::kRows + rl);
#pragma unroll
          for (int q = 0; q < kQ; ++q) ov[q][j] = load_agent(pv.o + (sl * (D / 4) + q0 + q) * C::kRows + rl);
        }
      }
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        // (every chunk of the row has the same maxima and sums)
        float Mq = M, Lq = L;
        fold_pieces<kFold>(Mq, Lq, o[q], m, l, ov[q]);
        if (q == kQ - 1) {
          M = Mq;
          L = Lq;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kQ; ++q) store_item(a, D, bb, kh, rc * C::kRows + rl, q0 + q, o[q], L);
  };
  // flat positions [j, j1) of this share; sequence b's tiles occupy
  // [seq_base + kSeqCostTiles, seq_base + kSeqCostTiles + ntiles)
  const int j_share = st.sp.start(share);
  const int j1 = min(st.S, st.sp.start(share + 1));
  int j = j_share;
  int b = st.b, seq_base = st.base;
  int Praw = a.prefix_lens[b];
  int ntiles = tiles_of(a, clamp_prefix(a, Praw));
  const int no_ids[2 * C::kStages] = {};
  for (;;) {
    const int first_tile = seq_base + kSeqCostTiles;
    if (j < first_tile) j = first_tile;  // the sequence's cost positions hold no tiles
    if (j >= j1) break;
    const int t0 = j - first_tile;
    const int t1 = min(ntiles, t0 + (j1 - j));
    // a cut piece leaves its state in slot v when it starts where the share
    // starts (it continues a sequence from the share before, or its sequence
    // starts exactly there), in G + v when its sequence starts inside the share
    const bool whole = t0 == 0 && t1 == ntiles;
    run_piece(b, kh, rc, Praw, t0, t1, whole, j == j_share ? v : G + v, no_ids, false);
    if (!whole && mp.fused_merge) merge_if_last(b, first_tile, ntiles);
    j += t1 - t0;
    if (j >= j1) break;
    // the share continues into the next sequence
    seq_base = first_tile + ntiles;
    ++b;
    Praw = a.prefix_lens[b];
    ntiles = tiles_of(a, clamp_prefix(a, Praw));
  }
}

// Merge the partial states of a sequence cut into fixed pieces (log-sum-exp
// rule) and write bf16 outputs: workgroup (segment, block of 32 rows x 8
// four-dim chunks) with one item (four dims of one row) per thread, rows
// fastest to match the [slot][D/4][row] partial layout, and all `pieces`
// slots of the item in flight together (empty pieces carry maxima of -inf).
template <int D, int NW>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a, MfmaParams mp) {
  using C = Cfg<D, NW>;
  constexpr int kGroup = 16;  // pieces folded at a time
  constexpr int kQBlocks = D / 4 / 8;
  constexpr int kBlocksPerSeg = C::kRows / 32 * kQBlocks;
  const int tid = threadIdx.x;
  const int u = static_cast<int>(blockIdx.x);
  const int RC = mp.row_chunks;
  const int segs = a.Hkv * RC;
  const int R = (a.Hq / a.Hkv) * a.N;
  const int seg_id = u / kBlocksPerSeg, blk = u % kBlocksPerSeg;
  const int b = seg_id / segs, seg = seg_id % segs;
  const int kh = seg / RC, rc = seg % RC;
  const int rows = min(C::kRows, R - rc * C::kRows);
  const int r_lo = (blk / kQBlocks) * 32;
  const int n = min(32, rows - r_lo);
  if (n <= 0 || (tid & 31) >= n) return;
  const int q = (blk % kQBlocks) * 8 + (tid >> 5), rl = r_lo + (tid & 31);
  const PartialView pv = partial_view<D>(a, mp, mp.grid);
  const size_t slot0 = static_cast<size_t>(seg_id) * mp.pieces;
  float M = -INFINITY, L = 0.f;
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < mp.pieces; k0 += kGroup) {
    float m[kGroup], l[kGroup];
    u32x2 ov[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      m[j] = -INFINITY;
      l[j] = 0.f;
      ov[j] = u32x2{0u, 0u};
      if (k0 + j < mp.pieces) {
        const size_t sl = slot0 + k0 + j;
        m[j] = pv.m[sl * C::kRows + rl];
        l[j] = pv.l[sl * C::kRows + rl];
        ov[j] = pv.o[(sl * (D / 4) + q) * C::kRows + rl];
      }
    }
    fold_pieces<kGroup>(M, L, o, m, l, ov);
  }
  store_item(a, D, b, kh, rc * C::kRows + rl, q, o, L);
}

// The second merge kernel of balanced shares (launches whose segments are
// cut into many pieces): merge_split workgroups per share and lane take the
// cut at the start of share v, if any, and of its rows the part given by
// the cut's rank among the sequence's cuts: the sequence's pieces are the
// shares f .. l it touches, and its n = l - f cuts share its rows.  Items are
// (4-dim chunk, row), rows fastest, four per thread, pieces two at a time.
template <int D, int NW>
__global__ __launch_bounds__(256) void attn_merge_cuts_kernel(AttnArgs a, MfmaParams mp) {
  using C = Cfg<D, NW>;
  constexpr int kItems = 4, kGroup = 2, kStep = 256;
  const int tid = threadIdx.x;
  const int u = static_cast<int>(blockIdx.x) / mp.merge_split;
  const int G = mp.grid;
  const int RC = mp.row_chunks;
  const int segs = a.Hkv * RC;
  const int R = (a.Hq / a.Hkv) * a.N;
  const int share = u / segs, lane = u % segs;
  const int* hdr = reinterpret_cast<const int*>(static_cast<const char*>(a.workspace) + kCounterBytes);
  const int4 cut = reinterpret_cast<const int4*>(hdr + 4)[share];
  if (cut.x < 0) return;
  const ShareSplit sp{hdr[1], hdr[2]};
  const int b = cut.x;
  const int f = sp.share_of(cut.y);
  const int npieces = sp.share_of(cut.y + cut.z - 1) - f + 1;
  const int kh = lane / RC, rc = lane % RC;
  // the sequence's tiles start inside share f: its piece there is that
  // share's second slot
  const bool cut_first = cut.y != sp.start(f);
  const int rows = min(C::kRows, R - rc * C::kRows);
  const int parts = (npieces - 1) * mp.merge_split;
  const int part = cut.w * mp.merge_split + static_cast<int>(blockIdx.x) % mp.merge_split;
  const int r_lo = part * rows / parts;
  const int n = (part + 1) * rows / parts - r_lo;
  if (n <= 0) return;
  const PartialView pv = partial_view<D>(a, mp, G);
  const int nitems = n * (D / 4);
  for (int it0 = tid; it0 < nitems; it0 += kItems * kStep) {
    float M[kItems], L[kItems], o[kItems][4];
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      M[i] = -INFINITY;
      L[i] = 0.f;
      o[i][0] = o[i][1] = o[i][2] = o[i][3] = 0.f;
    }
    for (int k0 = 0; k0 < npieces; k0 += kGroup) {
      float m[kItems][kGroup], l[kItems][kGroup];
      u32x2 ov[kItems][kGroup];
#pragma unroll
      for (int i = 0; i < kItems; ++i) {
        const int item = it0 + i * kStep;
        const int q = item / n, rl = r_lo + item % n;
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
          m[i][j] = -INFINITY;
          l[i][j] = 0.f;
          ov[i][j] = u32x2{0u, 0u};
          if (item < nitems && k0 + j < npieces) {
            const int vv = (f + k0 + j) * segs + lane;
            const size_t sl = static_cast<size_t>((k0 + j == 0 && cut_first) ? G + vv : vv);
            m[i][j] = pv.m[sl * C::kRows + rl];
            l[i][j] = pv.l[sl * C::kRows + rl];
            ov[i][j] = pv.o[(sl * (D / 4) + q) * C::kRows + rl];
          }
        }
      }
#pragma unroll
      for (int i = 0; i < kItems; ++i) fold_pieces<kGroup>(M[i], L[i], o[i], m[i], l[i], ov[i]);
    }
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int item = it0 + i * kStep;
      if (item >= nitems) break;
      store_item(a, D, b, kh, rc * C::kRows + r_lo + item % n, item / n, o[i], L[i]);
    }
  }
}

template <int D, int NW>
hipError_t launch_cfg(const AttnArgs& a, const MfmaParams& mp, hipStream_t stream) {
  using C = Cfg<D, NW>;
  const size_t shmem = C::kStages * C::kStageElems * sizeof(uint16_t);
  // with one row chunk per KV head no other workgroup reads a K/V tile
  // again, and its copies go non-temporal (batched workload 144 -> 129 us,
  // 70B-shaped chain 306 -> 286 us); several row chunks share each tile
  // through the L2, where the hint measured 6 % slower
  if (mp.row_chunks == 1)
    hipLaunchKernelGGL((attn_mfma_kernel<D, NW, kNonTemporal>), dim3(static_cast<unsigned>(mp.grid)),
                       dim3(C::kThreads), shmem, stream, a, mp);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<D, NW, 0>), dim3(static_cast<unsigned>(mp.grid)), dim3(C::kThreads),
                       shmem, stream, a, mp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (mp.balanced) {
    // merged in the attention kernel, or nothing to merge with one share per lane
    if (mp.fused_merge || mp.grid == a.Hkv * mp.row_chunks) return e;
    hipLaunchKernelGGL((attn_merge_cuts_kernel<D, NW>), dim3(static_cast<unsigned>(mp.grid * mp.merge_split)),
                       dim3(256), 0, stream, a, mp);
    return hipGetLastError();
  }
  if (mp.pieces == 1) return e;  // no segment is ever shared
  // fixed pieces: one workgroup per (segment, 32 rows x 32 dims)
  const long blocks = static_cast<long>(a.B) * a.Hkv * mp.row_chunks * (C::kRows / 32) * (D / 32);
  hipLaunchKernelGGL((attn_merge_kernel<D, NW>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a, mp);
  return hipGetLastError();
}

// MI355X: 256 compute units.  A 4-wave workgroup takes 64 KB of LDS, so two
// fit on a compute unit (two waves per SIMD).  Two independent workgroups
// per unit drift apart in phase, so one's softmax overlaps the other's
// MFMAs; an 8-wave workgroup (one per unit, in lockstep at every tile
// barrier) measured slower even where it halves the row chunks.
constexpr int kComputeUnits = 256;
// balanced shares: with two or more shares per lane, G = shares * lanes is at
// most one round of resident workgroups; a single share per lane cuts no
// sequence and counts nothing
static_assert(kMaxCounters >= kComputeUnits * 2, "one arrival counter per balanced workgroup");
constexpr int kMinTilesPerPiece = 4;  // balanced shares
// fixed pieces: each cut adds a partial state of kRows rows, written and
// merged; 5 tiles per piece (14 pieces, 224 workgroups) is the measured sweet
// spot for one Llama-3-8B-shaped sequence (2k prefix, 60 nodes): 4 and 6-8
// were 0.5-2 us slower
constexpr int kMinTilesFixed = 5;

// Rows of a KV head go to row chunks of 128 (4 waves).  One
// sequence: fixed pieces of at least kMinTilesFixed tiles, up to one round of
// resident workgroups.  Several sequences: balanced
// shares over one round of resident workgroups, or fewer when the work
// (bounded by max_prefix_len) would give shares under kMinTilesPerPiece.
MfmaParams plan_for(int B, int N, int Hq, int Hkv, int D, int max_prefix_len) {
  const int R = (Hq / Hkv) * N;
  MfmaParams p;
  // the row chunks of a KV head share its K/V tiles through L2
  p.waves = 4;
  p.fused_merge = 0;
  p.merge_split = 1;
  p.row_chunks = (R + p.waves * 32 - 1) / (p.waves * 32);
  const long max_tiles = (static_cast<long>(max_prefix_len) + N + kTile - 1) / kTile;
  const long segments = static_cast<long>(B) * Hkv * p.row_chunks;
  const long resident = static_cast<long>(kComputeUnits) * 2;
  if (B == 1) {
    long pieces = (resident + segments - 1) / segments;
    const long cap = (max_tiles + kMinTilesFixed - 1) / kMinTilesFixed;
    if (pieces > cap) pieces = cap;
    if (pieces < 1) pieces = 1;
    p.balanced = 0;
    p.T = static_cast<int>((max_tiles + pieces - 1) / pieces);
    p.pieces = static_cast<int>((max_tiles + p.T - 1) / p.T);
    p.grid = static_cast<int>(segments * p.pieces);
  } else {
    const long lanes = static_cast<long>(Hkv) * p.row_chunks;
    long shares = (B * max_tiles + kMinTilesPerPiece - 1) / kMinTilesPerPiece;
    if (shares > resident / lanes) shares = resident / lanes;
    if (shares < 1) shares = 1;
    p.balanced = 1;
    p.T = kMinTilesPerPiece;
    // Who merges a cut sequence: with many segments (a sequence at the
    // longest prefix spans fewer than four shares) the workgroup finishing
    // its last piece, in the attention kernel (the batched workload 123 ->
    // 119 us, the 70B-shaped chain 278 -> 266 us); with few, whose cut
    // sequences have eight or more pieces that one workgroup would fold in
    // series, a second kernel with many workgroups per cut (the Qwen2
    // workload: 156 us, against 159 us fused).  Merge workgroups per cut
    // there: three with one row chunk per KV head, two with several.
    p.fused_merge = segments * 4 > resident;
    p.merge_split = p.row_chunks == 1 ? 3 : 2;
    p.pieces = 0;
    p.grid = static_cast<int>(shares * lanes);
  }
  return p;
}

}  // namespace

size_t attention_mfma_workspace_bytes(int B, int N, int Hq, int Hkv, int D, int max_prefix_len) {
  const MfmaParams p = plan_for(B, N, Hq, Hkv, D, max_prefix_len);
  const size_t slots = static_cast<size_t>(p.balanced ? 2 * p.grid : p.grid) * p.waves * 32;
  const size_t hbytes = p.balanced ? header_bytes(p.grid / (Hkv * p.row_chunks)) : 0;
  return kCounterBytes + hbytes + slots * (2 * D + 2 * sizeof(float));
}

hipError_t launch_attention_mfma(const AttnArgs& a, hipStream_t stream) {
  const MfmaParams p = plan_for(a.B, a.N, a.Hq, a.Hkv, a.D, a.max_prefix_len);
  if (a.D == 128) return launch_cfg<128, 4>(a, p, stream);
  return launch_cfg<64, 4>(a, p, stream);
}

}  // namespace tv
