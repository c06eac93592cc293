// The target's LM head fused with the greedy choice: for every row m (a
// tree node's final hidden state), the lowest v maximising
// sum_h hidden[m][h] * weight[v][h], and that score, without writing the
// [M][V] scores anywhere.  ("P-EAGLE", 技术原理和实现方式 step 3: one target
// pass scores every proposed token; "vLLM EAGLE 投机解码实战", 无损性保障:
// greedy verification compares drafts with the target's greedy choice.)
//
// Score kernel: a workgroup owns 256 vocabulary rows and 64, 128 or 256
// hidden rows (by the row count), split over 4, 8 or 16 waves of 64 x 64.
// Per wave and 16-wide hidden step it runs
//   S^T (32 vocab x 32 rows) += W (32 vocab x 16) * hidden^T (16 x 32 rows)
// with v_mfma_f32_32x32x16_bf16 on 2 x 2 tiles, so every accumulator a lane
// holds belongs to one row (lane % 32) and the row maximum is mostly an
// in-register reduction.  64-wide hidden slices of both operands stream
// from HBM straight into LDS (buffer_load_dwordx4 ... lds, no staging
// registers) through two or three buffers: the copies of the next slices
// are in flight while slice k is multiplied, and within a slice the
// operands of the next 16-wide step are read while the current one
// multiplies.  Each wave waits for its own copies only
// (vmcnt), then one barrier publishes every wave's copies and frees the
// buffer of slice k - 1.  LDS rows are 128 bytes; 16-byte chunk c of row r
// is stored at chunk c ^ (r % 8), so the operand reads of 8 rows at one
// chunk hit all banks; the copies realise the swizzle by choosing which
// global chunk each lane fetches.  Rows past M or V read as zeros (buffer
// range) and past-V columns are kept out of the maximum.
//
// The workgroup's best (score, lowest index) per row is one 64-bit key per
// (row, vocabulary tile) in the workspace; a pick kernel (one wave per row)
// reduces a row's keys.  Workgroups of one vocabulary tile are numbered onto
// one XCD.
#include <type_traits>

#include "tv_internal.h"

namespace tv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBN = 256;  // vocabulary rows per workgroup (64 per vocabulary wave)
constexpr int kPickThreads = 256;

// Each wave owns CW 32-row vocabulary tiles and RW 32-row hidden tiles;
// NWV = 256 / (32 CW) vocabulary groups times NWR row groups of waves;
// hidden slices of BK dims through STAGES LDS buffers.
template <int RW, int CW, int NWR, int BK, int STAGES>
struct LCfg {
  static constexpr int kNWV = kBN / (32 * CW);
  static constexpr int kWaves = kNWV * NWR;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBM = 32 * RW * NWR;           // hidden rows per workgroup
  static constexpr int kRowBytes = 2 * BK;            // one LDS row
  static constexpr int kLanesPerRow = kRowBytes / 16;
  static constexpr int kRowsPerCopy = 64 / kLanesPerRow;  // one 1 KB wave copy
  static constexpr int kAElems = kBM * BK;            // bf16 elements of the hidden slice
  static constexpr int kWElems = kBN * BK;            // of the weight slice
  static constexpr int kStageElems = kAElems + kWElems;
  static constexpr int kWCopies = kBN / kRowsPerCopy / kWaves;  // per wave and slice
  static constexpr int kACopies = kBM / kRowsPerCopy / kWaves;
  static constexpr int kCopies = kWCopies + kACopies;
  static_assert(BK == 32 || BK == 64, "slice width");
  static_assert(kWCopies * kRowsPerCopy * kWaves == kBN && kACopies * kRowsPerCopy * kWaves == kBM,
                "copies split evenly over the waves");
  // 16-byte chunk c of LDS row r is stored at chunk c ^ swz(r): over 8
  // consecutive rows at one chunk, the reads then cover all 32 banks
  __device__ static constexpr int swz(int r) { return BK == 64 ? (r & 7) : ((r >> 1) & 3); }
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ds_read_b128 as inline assembly at a byte address plus an immediate
// offset.  The compiler cannot tell a plain LDS read from the LDS copies in
// flight and would wait for all of them (vmcnt(0)) before it, which would
// drain the prefetch; these reads are instead waited for by wait_operands.
// The destination is an output bound to the caller's register: no value is
// returned, so no temporary (whose copy the compiler could place before the
// wait, reading the register before the data arrived) stands between the
// read and its wait.
template <int OFF>
__device__ __forceinline__ void ds_read_b128(u32x4& dst, uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(dst) : "v"(addr), "i"(OFF));
}

// s_waitcnt lgkmcnt(0) taking the read destinations of one hidden step as
// operands, so no use of them is scheduled above the wait.
template <int CW, int RW>
__device__ __forceinline__ void wait_operands(u32x4 (&w)[CW], u32x4 (&x)[RW]) {
  static_assert((CW == 2 || CW == 4) && (RW == 2 || RW == 4), "operand counts");
  if constexpr (CW == 2 && RW == 2)
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(w[0]), "+v"(w[1]), "+v"(x[0]), "+v"(x[1]));
  else if constexpr (CW == 2)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(w[0]), "+v"(w[1]), "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
  else if constexpr (RW == 2)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]), "+v"(x[0]), "+v"(x[1]));
  else
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]), "+v"(x[0]), "+v"(x[1]), "+v"(x[2]),
                   "+v"(x[3]));
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
}

// WPOL: cache policy of the weight copies (kNonTemporal when one row tile
// reads the weight once; several row tiles share each slab through the L2).
template <int RW, int CW, int NWR, int BK, int STAGES, int WPOL>
__global__ __launch_bounds__((LCfg<RW, CW, NWR, BK, STAGES>::kThreads)) void lmhead_score_kernel(
    LmArgs a, int nmt, int nvt, uint64_t* __restrict__ keys) {
  using C = LCfg<RW, CW, NWR, BK, STAGES>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[STAGES * C::kStageElems];
  __shared__ uint64_t s_key[C::kNWV][C::kBM];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wv = wave % C::kNWV, wr = wave / C::kNWV;  // vocabulary group, row group

  // the hardware deals workgroups to the eight XCDs in turn; tiles are
  // renumbered so that each XCD takes one contiguous run of logical tiles:
  // the row tiles of a vocabulary tile then share one L2, which serves them
  // the slab's weight rows (on the 70B-shaped chain, 3.9 GB of HBM reads
  // per call instead of 13 GB with the row tiles spread over the XCDs), and
  // a single row tile streams contiguous vocabulary runs per XCD
  const int G = gridDim.x, g = blockIdx.x;
  const int xcd = g & 7, per = G >> 3, rem = G & 7;
  const int logical = xcd * per + min(xcd, rem) + (g >> 3);
  const int vt = logical / nmt, mt = logical % nmt;
  const int v0 = vt * kBN, m0 = mt * C::kBM;
  const int H = a.H;
  const char* wbase = static_cast<const char*>(a.weight) + static_cast<size_t>(v0) * H * 2;
  const char* abase = static_cast<const char*>(a.hidden) + static_cast<size_t>(m0) * H * 2;
  const int wrange = min(a.V - v0, kBN) * H * 2;
  const int arange = min(a.M - m0, C::kBM) * H * 2;

  // copy offsets: lane l fills row l / kLanesPerRow of a copy's rows, at
  // physical chunk l % kLanesPerRow, which holds the logical chunk that the
  // swizzle puts there
  const int crow = lane / C::kLanesPerRow;
  const int cchunk = (lane % C::kLanesPerRow) ^ C::swz(crow);
  int voff_w[C::kWCopies], voff_a[C::kACopies];
#pragma unroll
  for (int j = 0; j < C::kWCopies; ++j)
    voff_w[j] = ((wave * C::kWCopies + j) * C::kRowsPerCopy + crow) * H * 2 + cchunk * 16;
#pragma unroll
  for (int i = 0; i < C::kACopies; ++i)
    voff_a[i] = ((wave * C::kACopies + i) * C::kRowsPerCopy + crow) * H * 2 + cchunk * 16;

  auto issue = [&](int kc, int st) __attribute__((always_inline)) {
    uint16_t* sbase = lds + st * C::kStageElems;
    const int kb = kc * BK * 2;
#pragma unroll
    for (int j = 0; j < C::kWCopies; ++j)
      copy_to_lds<WPOL>(wbase, wrange, voff_w[j] + kb, sbase + C::kAElems + (wave * C::kWCopies + j) * 512);
#pragma unroll
    for (int i = 0; i < C::kACopies; ++i)
      copy_to_lds(abase, arange, voff_a[i] + kb, sbase + (wave * C::kACopies + i) * 512);
  };

  // operand reads: row r of a 32-row tile, logical chunk 2 s + lane / 32
  const int orow = lane & 31, ohalf = lane >> 5, oswz = C::swz(orow);
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LDS_AS const void*)lds));
  f32x16 acc[CW][RW];
#pragma unroll
  for (int cw = 0; cw < CW; ++cw)
#pragma unroll
    for (int rw = 0; rw < RW; ++rw) acc[cw][rw] = f32x16{};

  const int nk = H / BK;
#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st)
    if (st < nk) issue(st, st);
  for (int kc = 0; kc < nk; ++kc) {
    // this wave's copies of slice kc have landed once at most those of the
    // later slices already issued are outstanding
    const int later = min(STAGES - 2, nk - 1 - kc);
    if constexpr (STAGES >= 4) {
      if (later >= 2)
        wait_vmcnt<2 * C::kCopies>();
      else if (later == 1)
        wait_vmcnt<C::kCopies>();
      else
        wait_vmcnt<0>();
    } else {
      if (later >= 1)
        wait_vmcnt<C::kCopies>();
      else
        wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();  // slice kc landed everywhere; slice kc - 1 is free
    if (kc + STAGES - 1 < nk) issue(kc + STAGES - 1, (kc + STAGES - 1) % STAGES);
    const uint32_t sb = lds0 + (kc % STAGES) * C::kStageElems * 2;
    const uint32_t wrow = sb + 2 * C::kAElems + (wv * 32 * CW + orow) * C::kRowBytes;
    const uint32_t arow = sb + (wr * RW * 32 + orow) * C::kRowBytes;
    // operands of step s + 1 are read while step s multiplies
    u32x4 wvr[2][CW], xv[2][RW];
    auto read_step = [&](auto s_c) __attribute__((always_inline)) {
      constexpr int s = decltype(s_c)::value;
      const uint32_t ch = ((2 * s + ohalf) ^ oswz) * 16;
      static_for<0, CW>([&](auto cw_c) {
        constexpr int cw = decltype(cw_c)::value;
        ds_read_b128<cw * 32 * C::kRowBytes>(wvr[s & 1][cw], wrow + ch);
      });
      static_for<0, RW>([&](auto rw_c) {
        constexpr int rw = decltype(rw_c)::value;
        ds_read_b128<rw * 32 * C::kRowBytes>(xv[s & 1][rw], arow + ch);
      });
    };
    read_step(std::integral_constant<int, 0>{});
    wait_operands<CW, RW>(wvr[0], xv[0]);
    static_for<0, BK / 16>([&](auto s_c) {
      constexpr int s = decltype(s_c)::value;
      if constexpr (s + 1 < BK / 16) read_step(std::integral_constant<int, s + 1>{});
#pragma unroll
      for (int cw = 0; cw < CW; ++cw)
#pragma unroll
        for (int rw = 0; rw < RW; ++rw)
          acc[cw][rw] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wvr[s & 1][cw]),
                                                                __builtin_bit_cast(bf16x8, xv[s & 1][rw]),
                                                                acc[cw][rw], 0, 0, 0);
      if constexpr (s + 1 < BK / 16) wait_operands<CW, RW>(wvr[(s + 1) & 1], xv[(s + 1) & 1]);
    });
  }

  // row maxima: lane holds row rw * 32 + lane % 32 of its row group and
  // vocabulary rows 8 (k / 4) + 4 (lane / 32) + k % 4 of each 32-row tile
#pragma unroll
  for (int rw = 0; rw < RW; ++rw) {
    uint64_t best = 0ull;
#pragma unroll
    for (int cw = 0; cw < CW; ++cw)
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int v = v0 + wv * 32 * CW + cw * 32 + 8 * (k >> 2) + 4 * ohalf + (k & 3);
        if (v < a.V) {
          const uint64_t key = make_key(acc[cw][rw][k], v);
          best = key > best ? key : best;
        }
      }
    const uint64_t other = __shfl_xor(best, 32, 64);
    best = other > best ? other : best;
    if (lane < 32) s_key[wv][(wr * RW + rw) * 32 + lane] = best;
  }
  __syncthreads();
  for (int t = tid; t < C::kBM; t += C::kThreads) {
    uint64_t k = s_key[0][t];
#pragma unroll
    for (int w = 1; w < C::kNWV; ++w) k = s_key[w][t] > k ? s_key[w][t] : k;
    if (m0 + t < a.M) keys[static_cast<size_t>(m0 + t) * nvt + vt] = k;
  }
}

__global__ __launch_bounds__(kPickThreads) void lmhead_pick_kernel(LmArgs a, int nvt,
                                                                   const uint64_t* __restrict__ keys) {
  const int row = blockIdx.x * (kPickThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.M) return;
  uint64_t best = 0ull;
  for (int c = lane; c < nvt; c += 64) {
    const uint64_t k = keys[static_cast<size_t>(row) * nvt + c];
    best = k > best ? k : best;
  }
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t w = __shfl_xor(best, o, 64);
    best = w > best ? w : best;
  }
  if (lane == 0) {
    a.argmax[row] = static_cast<int>(~static_cast<uint32_t>(best & 0xFFFFFFFFull));
    if (a.max_score) a.max_score[row] = unordered(static_cast<uint32_t>(best >> 32));
  }
}

int vocab_tiles(int V) { return (V + kBN - 1) / kBN; }


template <int RW, int CW, int NWR, int BK, int STAGES>
hipError_t launch_cfg(const LmArgs& a, uint64_t* keys, hipStream_t stream) {
  using C = LCfg<RW, CW, NWR, BK, STAGES>;
  const int nvt = vocab_tiles(a.V);
  const int nmt = (a.M + C::kBM - 1) / C::kBM;
  const long grid = static_cast<long>(nvt) * nmt;
  if (nmt == 1)
    hipLaunchKernelGGL((lmhead_score_kernel<RW, CW, NWR, BK, STAGES, kNonTemporal>), dim3(static_cast<unsigned>(grid)),
                       dim3(C::kThreads), 0, stream, a, nmt, nvt, keys);
  else
    hipLaunchKernelGGL((lmhead_score_kernel<RW, CW, NWR, BK, STAGES, 0>), dim3(static_cast<unsigned>(grid)),
                       dim3(C::kThreads), 0, stream, a, nmt, nvt, keys);
  return hipGetLastError();
}

}  // namespace

size_t lm_head_workspace_bytes(int M, int V) {
  return static_cast<size_t>(M) * vocab_tiles(V) * sizeof(uint64_t);
}

hipError_t launch_lm_head_argmax(const LmArgs& a, hipStream_t stream) {
  uint64_t* keys = static_cast<uint64_t*>(a.workspace);
  // up to 64 rows: one row tile of four waves streams the weight once
  // (HBM-bound); up to 128: eight waves; more: 256 x 256 tiles of sixteen
  // waves of 64 x 64 each (four waves per SIMD hide each other's LDS and
  // copy waits; larger per-wave tiles with fewer waves measured slower)
  const hipError_t e = a.M <= 64    ? launch_cfg<2, 2, 1, 64, 3>(a, keys, stream)
                       : a.M <= 128 ? launch_cfg<2, 2, 2, 64, 3>(a, keys, stream)
                                    : launch_cfg<2, 2, 4, 64, 2>(a, keys, stream);
  if (e != hipSuccess) return e;
  const int per = kPickThreads / 64;
  hipLaunchKernelGGL(lmhead_pick_kernel, dim3((a.M + per - 1) / per), dim3(kPickThreads), 0, stream, a,
                     vocab_tiles(a.V), static_cast<const uint64_t*>(keys));
  return hipGetLastError();
}

}  // namespace tv
