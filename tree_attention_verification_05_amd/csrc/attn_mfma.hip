// Tree-masked paged attention on the gfx950 matrix cores (bf16 in, fp32
// accumulate).  ("vLLM-TreeEagle" README, 核心组件 item 1 and 技术创新点 1: all
// candidate paths are verified in one pass under a tree attention mask;
// "EAGLE代码实现原理", 树结构缓冲: the common prefix is shared; "P-EAGLE",
// 技术原理和实现方式 step 3.)
//
// Work unit: one workgroup per (sequence b, KV head kh, key split s, row
// chunk).  The query rows of a KV head are its g = Hq/Hkv heads times the N
// tree nodes (row r = node * g + head-in-group), so one K/V tile read from HBM
// serves every node and every query head of the group.  Each wave owns QB
// blocks of 32 rows.
//
// Per 64-key tile (double-buffered in LDS, next tile prefetched into
// registers while the current one is computed):
//   S^T (keys x rows)   = K (keys x D)   * Q^T (D x rows)   v_mfma_f32_32x32x16_bf16
//   O^T (D x rows)     += V^T (D x keys) * P^T (keys x rows) v_mfma_f32_32x32x16_bf16
// In the transposed form every accumulator a lane holds belongs to one query
// row (lane % 32), so the softmax rescaling is a per-lane scalar, and the
// score accumulators are already in the B-operand layout of the PV product
// (the MFMA contraction order of the keys is permuted identically in both
// operands).  Lanes l and l+32 share a row and split its keys; they exchange
// the tile maximum once per tile and their denominators once at the end.
//
// LDS layouts (bf16 elements):
//   K  [key][D], 16-byte chunk c of key k stored at chunk c ^ (k % 8)
//   Vt [dim][64 keys], 8-byte key group G of dim r stored at group
//      G ^ ((r % 16) ^ ((r / 8) % 16))
// Both swizzles make the loader's writes and the MFMA operand reads free of
// bank conflicts.
//
// Softmax: scores are kept raw; exponentials use exp2 with the factor
// scale*log2(e) folded into one FMA.  Prefix tiles need no mask; tiles that
// reach the tree slots apply the node's ancestor bitmask.  With several key
// splits, each split writes (max, denominator, unnormalised output) in fp32
// and a second kernel merges them with the log-sum-exp rule.
#include "tv_internal.h"

namespace tv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 64;  // keys per tile
constexpr float kLog2e = 1.4426950408889634f;

template <int D, int NW, int QB>
struct Cfg {
  static constexpr int kThreads = NW * 64;
  static constexpr int kChunks = D / 8;                  // 16-byte chunks per key row
  static constexpr int kKUnits = kTile * kChunks;        // 16-byte loads of a K tile
  static constexpr int kVUnits = (kTile / 4) * kChunks;  // (4 keys x 16 bytes) loads of a V tile
  static constexpr int kKPer = kKUnits / kThreads;
  static constexpr int kVPer = (kVUnits + kThreads - 1) / kThreads;
  static constexpr int kKs = D / 16;  // k-steps of the QK product
  static constexpr int kDb = D / 32;  // 32-dim output blocks
  static constexpr int kStage = kTile * D * 2;  // K + Vt elements per stage
  static constexpr int kRows = NW * QB * 32;    // rows per workgroup
  static_assert(kKUnits % kThreads == 0, "K tile loads must divide evenly");
};

struct MfmaParams {
  int tiles_per_split;
  int nsplit;      // splits per (sequence, KV head); 1 = write the output directly
  int row_chunks;  // workgroups along the rows of one KV head
};

__device__ __forceinline__ int vt_swz(int r) { return (r & 15) ^ ((r >> 3) & 15); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Visibility of the 64 keys of the tile that starts at logical position tb,
// for a row whose node has ancestor-or-self bits mw: bit k is set iff
// position tb + k is in the prefix or is a tree slot of one of those nodes.
// Bits of nodes >= N are zero in mw, so positions past the end are hidden.
// Every condition depends only on (tb, P) and is uniform across the wave.
__device__ __forceinline__ uint64_t tile_visibility(const uint64_t (&mw)[4], int tb, int P) {
  const int npre = P - tb;
  uint64_t vis = npre >= 64 ? ~0ull : (npre <= 0 ? 0ull : ((1ull << npre) - 1ull));
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int pos = P + 64 * k - tb;  // tile position of tree node 64k
    if (pos >= 0 && pos < 64)
      vis |= mw[k] << pos;
    else if (pos < 0 && pos > -64)
      vis |= mw[k] >> (-pos);
  }
  return vis;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

template <int D, int NW, int QB>
__global__ __launch_bounds__(NW * 64) void attn_mfma_kernel(AttnArgs a, MfmaParams mp) {
  using C = Cfg<D, NW, QB>;
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5;   // which half of the key set this lane holds
  const int col = lane & 31;  // query row within a 32-row block

  // blockIdx.x = ((b * Hkv + kh) * nsplit + s) * row_chunks + rc
  int idx = blockIdx.x;
  const int rc = idx % mp.row_chunks;
  idx /= mp.row_chunks;
  const int s = idx % mp.nsplit;
  idx /= mp.nsplit;
  const int kh = idx % a.Hkv;
  const int b = idx / a.Hkv;

  const int g = a.Hq / a.Hkv;
  const int R = g * a.N;
  const int W = (a.N + 63) >> 6;
  int P = a.prefix_lens[b];
  if (P < 0 || P > a.max_prefix_len) {
    if (tid == 0) report(a.dev_status, TV_DEV_BAD_CACHE);
    P = P < 0 ? 0 : a.max_prefix_len;
  }
  const int total = P + a.N;
  const int ntiles = (total + kTile - 1) / kTile;
  const int t0 = s * mp.tiles_per_split;
  const int t1 = min(ntiles, t0 + mp.tiles_per_split);
  if (t0 >= t1) return;  // whole workgroup: this split is past the sequence's end

  const int32_t* table = a.block_table + static_cast<size_t>(b) * a.max_blocks;
  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);
  const float c = a.scale * kLog2e;

  // ---------------- query rows of this wave (B operand of S^T) ----------------
  const int row0 = rc * C::kRows + wave * QB * 32;
  bf16x8 qreg[QB][C::kKs];
  uint64_t mw[QB][4];
  bool qactive[QB];
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    const int r = row0 + q * 32 + col;
    qactive[q] = (row0 + q * 32) < R;
    const int rr = r < R ? r : R - 1;
    const int node = rr / g, hg = rr % g;
    const u32x4* qp = reinterpret_cast<const u32x4*>(
        static_cast<const uint16_t*>(a.q) +
        ((static_cast<size_t>(b) * a.N + node) * a.Hq + kh * g + hg) * D);
#pragma unroll
    for (int ks = 0; ks < C::kKs; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (r < R) v = qp[ks * 2 + hh];
      qreg[q][ks] = __builtin_bit_cast(bf16x8, v);
    }
    const uint64_t* mrow = a.mask + (static_cast<size_t>(b) * a.N + node) * W;
#pragma unroll
    for (int w = 0; w < 4; ++w) mw[q][w] = (w < W) ? mrow[w] : 0ull;
  }

  // ---------------- tile loader ----------------
  u32x4 kreg[C::kKPer];
  u32x4 vreg[C::kVPer][4];

  auto cache_row = [&](int t, bool& ok) -> long {
    ok = false;
    if (t >= total) return 0;
    const int blk = table[t >> 4];
    if (blk < 0 || blk >= a.num_blocks) {
      report(a.dev_status, TV_DEV_BAD_CACHE);
      return 0;
    }
    ok = true;
    return (static_cast<long>(blk) * kBlockSize + (t & 15)) * a.Hkv + kh;
  };

  auto load_tile = [&](int tile) {
    const int tb = tile * kTile;
#pragma unroll
    for (int j = 0; j < C::kKPer; ++j) {
      const int u = tid + j * C::kThreads;
      const int key = u / C::kChunks, ch = u % C::kChunks;
      bool ok;
      const long cr = cache_row(tb + key, ok);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ok) v = *reinterpret_cast<const u32x4*>(kc + cr * D + ch * 8);
      kreg[j] = v;
    }
#pragma unroll
    for (int j = 0; j < C::kVPer; ++j) {
      const int u = tid + j * C::kThreads;
      const int kg = u / C::kChunks, ch = u % C::kChunks;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (u < C::kVUnits) {
          bool ok;
          const long cr = cache_row(tb + kg * 4 + e, ok);
          if (ok) v = *reinterpret_cast<const u32x4*>(vc + cr * D + ch * 8);
        }
        vreg[j][e] = v;
      }
    }
  };

  auto store_tile = [&](int stage) {
    uint16_t* ks = lds + stage * C::kStage;
    uint16_t* vt = ks + kTile * D;
#pragma unroll
    for (int j = 0; j < C::kKPer; ++j) {
      const int u = tid + j * C::kThreads;
      const int key = u / C::kChunks, ch = u % C::kChunks;
      *reinterpret_cast<u32x4*>(ks + key * D + ((ch ^ (key & 7)) * 8)) = kreg[j];
    }
#pragma unroll
    for (int j = 0; j < C::kVPer; ++j) {
      const int u = tid + j * C::kThreads;
      if (u < C::kVUnits) {
        const int kg = u / C::kChunks, ch = u % C::kChunks;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          // dims 2m and 2m+1 of the 4 keys: low and high halves of word m
          const uint32_t w0 = vreg[j][0][m], w1 = vreg[j][1][m];
          const uint32_t w2 = vreg[j][2][m], w3 = vreg[j][3][m];
          u32x2 even, odd;
          even[0] = __builtin_amdgcn_perm(w1, w0, 0x05040100u);
          even[1] = __builtin_amdgcn_perm(w3, w2, 0x05040100u);
          odd[0] = __builtin_amdgcn_perm(w1, w0, 0x07060302u);
          odd[1] = __builtin_amdgcn_perm(w3, w2, 0x07060302u);
          const int r0 = ch * 8 + 2 * m, r1 = r0 + 1;
          *reinterpret_cast<u32x2*>(vt + r0 * kTile + ((kg ^ vt_swz(r0)) * 4)) = even;
          *reinterpret_cast<u32x2*>(vt + r1 * kTile + ((kg ^ vt_swz(r1)) * 4)) = odd;
        }
      }
    }
  };

  // ---------------- per-row softmax state and output accumulators ----------------
  f32x16 acc[QB][C::kDb];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    m_run[q] = -INFINITY;
    l_run[q] = 0.f;
#pragma unroll
    for (int db = 0; db < C::kDb; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[q][db][r] = 0.f;
  }

  auto compute_tile = [&](int stage, int tile) {
    const uint16_t* ks = lds + stage * C::kStage;
    const uint16_t* vt = ks + kTile * D;
    const int tb = tile * kTile;
    const bool masked = tb + kTile > P;  // tile reaches the tree slots or the end
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      if (!qactive[q]) continue;
      // S^T for the two 32-key halves of the tile
      f32x16 sc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 sacc = {};
        const int key = kb * 32 + col;
#pragma unroll
        for (int kk = 0; kk < C::kKs; ++kk) {
          const int ch = kk * 2 + hh;
          const bf16x8 av =
              *reinterpret_cast<const bf16x8*>(ks + key * D + ((ch ^ (key & 7)) * 8));
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qreg[q][kk], sacc, 0, 0, 0);
        }
        sc[kb] = sacc;
      }
      // scores as plain floats; masked tiles select -inf without branches
      float sv[2][16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[kb][r] = sc[kb][r];
      if (masked) {
        const uint64_t vis = tile_visibility(mw[q], tb, P) >> (4 * hh);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int bit = kb * 32 + 8 * (r >> 2) + (r & 3);
            sv[kb][r] = ((vis >> bit) & 1ull) ? sv[kb][r] : -INFINITY;
          }
      }
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sv[kb][r]);
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float mn = fmaxf(m_run[q], mt);
      const float ms = (mn == -INFINITY) ? 0.f : mn;  // nothing visible yet: keep zeros
      const float alpha = exp2_fast((m_run[q] - ms) * c);
      const float mc = ms * c;
      m_run[q] = mn;
      float lsum = 0.f;
      bf16x8 pb[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = exp2_fast(__builtin_fmaf(sv[kb][r], c, -mc));
          lsum += p[r];
        }
#pragma unroll
        for (int kc2 = 0; kc2 < 2; ++kc2) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(p[kc2 * 8 + 2 * e], p[kc2 * 8 + 2 * e + 1]);
          pb[kb][kc2] = __builtin_bit_cast(bf16x8, w);
        }
      }
      l_run[q] = l_run[q] * alpha + lsum;
      // wave-uniform branch: skipped when no row's maximum moved (alpha == 1)
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
        for (int db = 0; db < C::kDb; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[q][db][r] *= alpha;
      }
      // O^T += V^T P^T
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int kc2 = 0; kc2 < 2; ++kc2) {
          const int g1 = kb * 8 + kc2 * 4 + hh, g2 = g1 + 2;
#pragma unroll
          for (int db = 0; db < C::kDb; ++db) {
            const int d = db * 32 + col;
            const int sw = vt_swz(d);
            const u32x2 lo = *reinterpret_cast<const u32x2*>(vt + d * kTile + ((g1 ^ sw) * 4));
            const u32x2 hi = *reinterpret_cast<const u32x2*>(vt + d * kTile + ((g2 ^ sw) * 4));
            u32x4 w;
            w[0] = lo[0];
            w[1] = lo[1];
            w[2] = hi[0];
            w[3] = hi[1];
            acc[q][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w),
                                                                 pb[kb][kc2], acc[q][db], 0, 0, 0);
          }
        }
    }
  };

  // ---------------- main loop ----------------
  load_tile(t0);
  store_tile(0);
  __syncthreads();
  for (int tile = t0; tile < t1; ++tile) {
    const int stage = (tile - t0) & 1;
    const bool more = tile + 1 < t1;
    if (more) load_tile(tile + 1);
    compute_tile(stage, tile);
    if (more) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---------------- epilogue ----------------
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    if (!qactive[q]) continue;
    const int r = row0 + q * 32 + col;
    const float lt = l_run[q] + __shfl_xor(l_run[q], 32, 64);
    if (r >= R) continue;
    const int node = r / g, hg = r % g;
    if (mp.nsplit == 1) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      uint16_t* op = static_cast<uint16_t*>(a.out) +
                     ((static_cast<size_t>(b) * a.N + node) * a.Hq + kh * g + hg) * D;
#pragma unroll
      for (int db = 0; db < C::kDb; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = db * 32 + 8 * j + 4 * hh;
          u32x2 w;
          w[0] = pack_bf16x2(acc[q][db][4 * j] * inv, acc[q][db][4 * j + 1] * inv);
          w[1] = pack_bf16x2(acc[q][db][4 * j + 2] * inv, acc[q][db][4 * j + 3] * inv);
          *reinterpret_cast<u32x2*>(op + d) = w;
        }
    } else {
      // partial state of this split: [B][Hkv][nsplit][R] rows
      const size_t prow = ((static_cast<size_t>(b) * a.Hkv + kh) * mp.nsplit + s) * R + r;
      const size_t nprow = static_cast<size_t>(a.B) * a.Hkv * mp.nsplit * R;
      float* po = static_cast<float*>(a.workspace) + prow * D;
      float* pm = static_cast<float*>(a.workspace) + nprow * D;
      float* pl = pm + nprow;
#pragma unroll
      for (int db = 0; db < C::kDb; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = db * 32 + 8 * j + 4 * hh;
          float4 v;
          v.x = acc[q][db][4 * j];
          v.y = acc[q][db][4 * j + 1];
          v.z = acc[q][db][4 * j + 2];
          v.w = acc[q][db][4 * j + 3];
          *reinterpret_cast<float4*>(po + d) = v;
        }
      if (hh == 0) {
        pm[prow] = m_run[q];
        pl[prow] = lt;
      }
    }
  }
}

// Merge the per-split partial states of every row (log-sum-exp rule) and
// write the bf16 output.  One wavefront per (sequence, KV head, row).
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a, MfmaParams mp) {
  const int lane = threadIdx.x & 63;
  const int g = a.Hq / a.Hkv;
  const int R = g * a.N;
  const long gw = static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (gw >= static_cast<long>(a.B) * a.Hkv * R) return;
  const int r = static_cast<int>(gw % R);
  const int kh = static_cast<int>((gw / R) % a.Hkv);
  const int b = static_cast<int>(gw / (static_cast<long>(R) * a.Hkv));
  int P = a.prefix_lens[b];
  P = P < 0 ? 0 : (P > a.max_prefix_len ? a.max_prefix_len : P);
  const int ntiles = (P + a.N + kTile - 1) / kTile;
  const int ns = min(mp.nsplit, (ntiles + mp.tiles_per_split - 1) / mp.tiles_per_split);
  const float c = a.scale * kLog2e;
  const size_t nprow = static_cast<size_t>(a.B) * a.Hkv * mp.nsplit * R;
  const float* po = static_cast<const float*>(a.workspace);
  const float* pm = po + nprow * D;
  const float* pl = pm + nprow;
  const size_t base = (static_cast<size_t>(b) * a.Hkv + kh) * mp.nsplit * R + r;

  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, pm[base + static_cast<size_t>(s) * R]);
  const float Ms = (M == -INFINITY) ? 0.f : M;
  constexpr int PER = D / 64;
  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  float L = 0.f;
  for (int s = 0; s < ns; ++s) {
    const size_t pr = base + static_cast<size_t>(s) * R;
    const float w = exp2_fast((pm[pr] - Ms) * c);
    L += w * pl[pr];
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] += w * po[pr * D + lane * PER + e];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const int node = r / g, hg = r % g;
  uint16_t* op = static_cast<uint16_t*>(a.out) +
                 ((static_cast<size_t>(b) * a.N + node) * a.Hq + kh * g + hg) * D;
#pragma unroll
  for (int e = 0; e < PER; ++e) op[lane * PER + e] = f32_to_bf16(o[e] * inv);
}

template <int D, int NW, int QB>
hipError_t launch_cfg(const AttnArgs& a, const MfmaParams& mp, hipStream_t stream) {
  using C = Cfg<D, NW, QB>;
  const long blocks = static_cast<long>(a.B) * a.Hkv * mp.nsplit * mp.row_chunks;
  const size_t shmem = 2 * C::kStage * sizeof(uint16_t);
  hipLaunchKernelGGL((attn_mfma_kernel<D, NW, QB>), dim3(static_cast<unsigned>(blocks)),
                     dim3(C::kThreads), shmem, stream, a, mp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || mp.nsplit == 1) return e;
  const long rows = static_cast<long>(a.B) * a.Hkv * (a.Hq / a.Hkv) * a.N;
  hipLaunchKernelGGL((attn_combine_kernel<D>), dim3(static_cast<unsigned>((rows + 3) / 4)),
                     dim3(256), 0, stream, a, mp);
  return hipGetLastError();
}

constexpr int kWaves = 4;
constexpr int kTargetBlocks = 512;
constexpr int kMinTilesPerSplit = 2;

struct Plan {
  int qb;
  MfmaParams mp;
};

Plan plan_for(int B, int N, int Hq, int Hkv, int max_prefix_len) {
  const int R = (Hq / Hkv) * N;
  Plan p;
  p.qb = R > kWaves * 32 ? 2 : 1;
  const int rows_per_wg = kWaves * 32 * p.qb;
  p.mp.row_chunks = (R + rows_per_wg - 1) / rows_per_wg;
  const int max_tiles = (max_prefix_len + N + kTile - 1) / kTile;
  const long base = static_cast<long>(B) * Hkv * p.mp.row_chunks;
  long want = (kTargetBlocks + base - 1) / base;
  const long cap = (max_tiles + kMinTilesPerSplit - 1) / kMinTilesPerSplit;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  p.mp.tiles_per_split = static_cast<int>((max_tiles + want - 1) / want);
  p.mp.nsplit = (max_tiles + p.mp.tiles_per_split - 1) / p.mp.tiles_per_split;
  return p;
}

}  // namespace

size_t attention_mfma_workspace_bytes(int B, int N, int Hq, int Hkv, int D, int max_prefix_len) {
  const Plan p = plan_for(B, N, Hq, Hkv, max_prefix_len);
  if (p.mp.nsplit == 1) return 0;
  const size_t rows = static_cast<size_t>(B) * Hkv * p.mp.nsplit * (Hq / Hkv) * N;
  return rows * (D + 2) * sizeof(float);
}

hipError_t launch_attention_mfma(const AttnArgs& a, hipStream_t stream) {
  const Plan p = plan_for(a.B, a.N, a.Hq, a.Hkv, a.max_prefix_len);
  if (a.D == 128)
    return p.qb == 2 ? launch_cfg<128, kWaves, 2>(a, p.mp, stream)
                     : launch_cfg<128, kWaves, 1>(a, p.mp, stream);
  return p.qb == 2 ? launch_cfg<64, kWaves, 2>(a, p.mp, stream)
                   : launch_cfg<64, kWaves, 1>(a, p.mp, stream);
}

}  // namespace tv
