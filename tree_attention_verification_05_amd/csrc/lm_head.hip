// The target's LM head fused with the greedy choice: for every row m (a
// tree node's final hidden state), the lowest v maximising
// sum_h hidden[m][h] * weight[v][h], and that score, without writing the
// [M][V] scores anywhere.  ("P-EAGLE", 技术原理和实现方式 step 3: one target
// pass scores every proposed token; "vLLM EAGLE 投机解码实战", 无损性保障:
// greedy verification compares drafts with the target's greedy choice.)
//
// Score kernel: a workgroup owns 256 vocabulary rows and 32 * RW hidden
// rows (RW = 2 for up to 64 rows, else 4); each of its four waves owns 64
// vocabulary rows.  Per wave and 16-wide hidden step it runs
//   S^T (32 vocab x 32 rows) += W (32 vocab x 16) * hidden^T (16 x 32 rows)
// with v_mfma_f32_32x32x16_bf16, 2 x RW tiles, so every accumulator a lane
// holds belongs to one row (lane % 32) and the row maximum is mostly an
// in-register reduction.  64-wide hidden slices of both operands stream
// from HBM straight into LDS (buffer_load_dwordx4 ... lds, no staging
// registers) through three buffers: the copies of slice k + 2 are in flight
// while slice k is multiplied, and within a slice the operands of the next
// 16-wide step are read while the current one multiplies.  Each wave waits for its own copies only
// (vmcnt), then one barrier publishes every wave's copies and frees the
// buffer of slice k - 1.  LDS rows are 128 bytes; 16-byte chunk c of row r
// is stored at chunk c ^ (r % 8), so the operand reads of 8 rows at one
// chunk hit all banks; the copies realise the swizzle by choosing which
// global chunk each lane fetches.  Rows past M or V read as zeros (buffer
// range) and past-V columns are kept out of the maximum.
//
// The workgroup's best (score, lowest index) per row is one 64-bit key per
// (row, vocabulary tile) in the workspace; a pick kernel (one wave per row)
// reduces a row's keys.  Workgroups of one vocabulary tile are numbered so
// that they land on one XCD, whose L2 then serves the tile's weight rows to
// all of its row tiles.
#include <type_traits>

#include "tv_internal.h"

namespace tv {
namespace {

#define LDS_AS __attribute__((address_space(3)))
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;  // four waves
constexpr int kBN = 256;       // vocabulary rows per workgroup
constexpr int kBK = 64;        // hidden dims per slice (128-byte LDS rows)
constexpr int kStages = 3;
constexpr int kPickThreads = 256;

template <int RW>
struct LCfg {
  static constexpr int kBM = 32 * RW;                 // hidden rows per workgroup
  static constexpr int kAElems = kBM * kBK;           // bf16 elements of the hidden slice
  static constexpr int kWElems = kBN * kBK;           // of the weight slice
  static constexpr int kStageElems = kAElems + kWElems;
  static constexpr int kCopies = kBN / 32 + RW;       // 1 KB copies per wave per slice
};

// Orders floats as unsigned integers; -0.0 and +0.0 map to the same value.
__device__ __forceinline__ uint32_t ordered(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unordered(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
// Larger key = larger score, then lower index.
__device__ __forceinline__ uint64_t make_key(float v, int idx) {
  return (static_cast<uint64_t>(ordered(v)) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(idx));
}

// One wave copies 64 x 16 bytes from a buffer (base, range in bytes; per-lane
// byte offset) into LDS: lane l's bytes land at dst + 16 l.  Reads past the
// range return zeros.
__device__ __forceinline__ void copy_to_lds(const char* base, int range, int voff, uint16_t* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, range, 0x00020000),
      (LDS_AS void*)dst, 16, voff, 0, 0, 0);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ds_read_b128 as inline assembly at a byte address plus an immediate
// offset.  The compiler cannot tell a plain LDS read from the LDS copies in
// flight and would wait for all of them (vmcnt(0)) before it, which would
// drain the prefetch; these reads are instead waited for by wait_operands.
template <int OFF>
__device__ __forceinline__ u32x4 ds_read_b128(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}

// s_waitcnt lgkmcnt(0) taking the operands of one hidden step as operands,
// so no use of them is scheduled above the wait.
template <int RW>
__device__ __forceinline__ void wait_operands(u32x4 (&w)[2], u32x4 (&x)[RW]) {
  if constexpr (RW == 2)
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(w[0]), "+v"(w[1]), "+v"(x[0]), "+v"(x[1]));
  else
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(w[0]), "+v"(w[1]), "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
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

template <int RW>
__global__ __launch_bounds__(kThreads) void lmhead_score_kernel(LmArgs a, int nmt, int nvt,
                                                                uint64_t* __restrict__ keys) {
  using C = LCfg<RW>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[kStages * C::kStageElems];
  __shared__ uint64_t s_key[kThreads / 64][C::kBM];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // workgroup g runs on XCD g % 8; number the tiles so that consecutive
  // logical tiles (the row tiles of one vocabulary tile) share an XCD
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

  // copy offsets: lane l fills row 8 j + l / 8 of its 1 KB block, physical
  // chunk l % 8, which holds logical chunk (l % 8) ^ (l / 8)
  const int crow = lane >> 3;
  const int cchunk = (lane & 7) ^ crow;
  int voff_w[kBN / 32], voff_a[RW];
#pragma unroll
  for (int j = 0; j < kBN / 32; ++j) voff_w[j] = ((wave * (kBN / 32) + j) * 8 + crow) * H * 2 + cchunk * 16;
#pragma unroll
  for (int i = 0; i < RW; ++i) voff_a[i] = ((wave * RW + i) * 8 + crow) * H * 2 + cchunk * 16;

  auto issue = [&](int kc, int st) __attribute__((always_inline)) {
    uint16_t* sbase = lds + st * C::kStageElems;
    const int kb = kc * kBK * 2;
#pragma unroll
    for (int j = 0; j < kBN / 32; ++j)
      copy_to_lds(wbase, wrange, voff_w[j] + kb, sbase + C::kAElems + (wave * (kBN / 32) + j) * 512);
#pragma unroll
    for (int i = 0; i < RW; ++i) copy_to_lds(abase, arange, voff_a[i] + kb, sbase + (wave * RW + i) * 512);
  };

  // operand read offsets (elements within a stage): row r, logical chunk
  // 2 s + lane / 32 stored at chunk (2 s + lane / 32) ^ (r % 8), r % 8 = lane % 8
  const int orow = lane & 31, ohalf = lane >> 5, oswz = lane & 7;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LDS_AS const void*)lds));
  f32x16 acc[2][RW];
#pragma unroll
  for (int cw = 0; cw < 2; ++cw)
#pragma unroll
    for (int rw = 0; rw < RW; ++rw) acc[cw][rw] = f32x16{};

  const int nk = H / kBK;
#pragma unroll
  for (int st = 0; st < kStages - 1; ++st)
    if (st < nk) issue(st, st);
  for (int kc = 0; kc < nk; ++kc) {
    if (kc + 1 < nk)
      wait_vmcnt<C::kCopies>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();  // slice kc landed everywhere; slice kc - 1 is free
    if (kc + kStages - 1 < nk) issue(kc + kStages - 1, (kc + kStages - 1) % kStages);
    const uint32_t sb = lds0 + (kc % kStages) * C::kStageElems * 2;
    const uint32_t wrow = sb + (wave * 64 + orow) * (kBK * 2);
    const uint32_t arow = sb + orow * (kBK * 2);
    // operands of step s + 1 are read while step s multiplies
    u32x4 wv[2][2], xv[2][RW];
    auto read_step = [&](auto s_c) __attribute__((always_inline)) {
      constexpr int s = decltype(s_c)::value;
      const uint32_t ch = ((2 * s + ohalf) ^ oswz) * 16;
      static_for<0, 2>([&](auto cw_c) {
        constexpr int cw = decltype(cw_c)::value;
        wv[s & 1][cw] = ds_read_b128<2 * C::kAElems + cw * 32 * kBK * 2>(wrow + ch);
      });
      static_for<0, RW>([&](auto rw_c) {
        constexpr int rw = decltype(rw_c)::value;
        xv[s & 1][rw] = ds_read_b128<rw * 32 * kBK * 2>(arow + ch);
      });
    };
    read_step(std::integral_constant<int, 0>{});
    wait_operands<RW>(wv[0], xv[0]);
    static_for<0, kBK / 16>([&](auto s_c) {
      constexpr int s = decltype(s_c)::value;
      if constexpr (s + 1 < kBK / 16) read_step(std::integral_constant<int, s + 1>{});
#pragma unroll
      for (int cw = 0; cw < 2; ++cw)
#pragma unroll
        for (int rw = 0; rw < RW; ++rw)
          acc[cw][rw] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wv[s & 1][cw]),
                                                                __builtin_bit_cast(bf16x8, xv[s & 1][rw]),
                                                                acc[cw][rw], 0, 0, 0);
      if constexpr (s + 1 < kBK / 16) wait_operands<RW>(wv[(s + 1) & 1], xv[(s + 1) & 1]);
    });
  }

  // row maxima: lane holds row rw * 32 + lane % 32 and vocabulary rows
  // 8 (k / 4) + 4 (lane / 32) + k % 4 of each 32-row tile
#pragma unroll
  for (int rw = 0; rw < RW; ++rw) {
    uint64_t best = 0ull;
#pragma unroll
    for (int cw = 0; cw < 2; ++cw)
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int v = v0 + wave * 64 + cw * 32 + 8 * (k >> 2) + 4 * ohalf + (k & 3);
        if (v < a.V) {
          const uint64_t key = make_key(acc[cw][rw][k], v);
          best = key > best ? key : best;
        }
      }
    const uint64_t other = __shfl_xor(best, 32, 64);
    best = other > best ? other : best;
    if (lane < 32) s_key[wave][rw * 32 + lane] = best;
  }
  __syncthreads();
  for (int t = tid; t < C::kBM; t += kThreads) {
    uint64_t k = s_key[0][t];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) k = s_key[w][t] > k ? s_key[w][t] : k;
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

template <int RW>
hipError_t launch_rw(const LmArgs& a, uint64_t* keys, hipStream_t stream) {
  const int nvt = vocab_tiles(a.V);
  const int nmt = (a.M + LCfg<RW>::kBM - 1) / LCfg<RW>::kBM;
  const long grid = static_cast<long>(nvt) * nmt;
  hipLaunchKernelGGL(lmhead_score_kernel<RW>, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream, a, nmt,
                     nvt, keys);
  return hipGetLastError();
}

}  // namespace

size_t lm_head_workspace_bytes(int M, int V) {
  return static_cast<size_t>(M) * vocab_tiles(V) * sizeof(uint64_t);
}

hipError_t launch_lm_head_argmax(const LmArgs& a, hipStream_t stream) {
  uint64_t* keys = static_cast<uint64_t*>(a.workspace);
  const hipError_t e = a.M <= 64 ? launch_rw<2>(a, keys, stream) : launch_rw<4>(a, keys, stream);
  if (e != hipSuccess) return e;
  const int per = kPickThreads / 64;
  hipLaunchKernelGGL(lmhead_pick_kernel, dim3((a.M + per - 1) / per), dim3(kPickThreads), 0, stream, a,
                     vocab_tiles(a.V), static_cast<const uint64_t*>(keys));
  return hipGetLastError();
}

}  // namespace tv
