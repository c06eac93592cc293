// Tree-masked paged attention, simple form: one wavefront per
// (sequence, node, query head) row, fp32 arithmetic for fp32 or bf16 inputs.
// ("vLLM-TreeEagle" README, 核心组件 item 1 and 技术创新点 1; "P-EAGLE",
// 技术原理和实现方式 step 3.)
//
// Keys are visited in chunks of 64 (one per lane).  Each lane forms one score,
// the wave keeps a running maximum and denominator (softmax rescaling), and
// the value rows are accumulated with lanes spread over the head dimension.
// This is the fp32 path and the reference shape for the matrix-core kernel.
#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <typename T, int D>
__global__ __launch_bounds__(kWaves * 64) void attn_rowwave_kernel(AttnArgs a) {
  constexpr int R = D / 64;  // dims per lane in the value accumulation
  __shared__ float qs[kWaves][D];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long row = static_cast<long>(blockIdx.x) * kWaves + wave;  // (b*N + i)*Hq + h
  const long rows = static_cast<long>(a.B) * a.N * a.Hq;
  const bool active = row < rows;
  const int h = static_cast<int>(row % a.Hq);
  const int i = static_cast<int>((row / a.Hq) % a.N);
  const int b = static_cast<int>(row / (static_cast<long>(a.Hq) * a.N));
  const int kh = h / (a.Hq / a.Hkv);
  const int W = (a.N + 63) >> 6;
  const T* q = static_cast<const T*>(a.q) + row * D;
  const T* kc = static_cast<const T*>(a.k_cache);
  const T* vc = static_cast<const T*>(a.v_cache);
  T* out = static_cast<T*>(a.out) + row * D;
  const float c = a.scale * kLog2e;  // scores in base-2 units

  if (active)
    for (int d = lane; d < D; d += 64) qs[wave][d] = Elt<T>::load(q + d);
  __syncthreads();
  if (!active) return;  // no barrier below this point

  const uint64_t* mrow = a.mask ? a.mask + (static_cast<size_t>(b) * a.N + i) * W : nullptr;
  uint64_t own = 0;  // without masks: node i's word, built from the parents (N <= 64)
  if (!a.mask) {
    bool bad_tree;
    const int p = lane < a.N ? a.parents[static_cast<size_t>(b) * a.N + lane] : -1;
    own = __shfl(wave_tree_mask(p, a.N, lane, &bad_tree), i, 64);
    if (bad_tree && lane == 0) report(a.dev_status, TV_DEV_BAD_TREE);
  }
  const int P = a.prefix_lens[b];
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  if (P < 0 || P > a.max_prefix_len) {
    if (lane == 0) report(a.dev_status, TV_DEV_BAD_CACHE);
#pragma unroll
    for (int r = 0; r < R; ++r) Elt<T>::store(out + lane + 64 * r, 0.f);
    return;
  }
  const int32_t* table = a.block_table + static_cast<size_t>(b) * a.max_blocks;
  const int total = P + a.N;
  float m = -INFINITY, l = 0.f;

  for (int t0 = 0; t0 < total; t0 += 64) {
    const int t = t0 + lane;
    float s = -INFINITY;
    long long crow = -1;  // cache row (D elements) of this lane's key in head kh
    if (t < total) {
      bool vis = true;
      if (t >= P) {
        const int j = t - P;
        vis = ((mrow ? mrow[j >> 6] : own) >> (j & 63)) & 1ull;
      }
      const int blk = table[t / kBlockSize];
      if (blk < 0 || blk >= a.num_blocks) {
        report(a.dev_status, TV_DEV_BAD_CACHE);
        vis = false;
      }
      if (vis) {
        crow = kv_row(blk, kh, t % kBlockSize, a.Hkv, a.kv_head_rows, a.kv_slot_rows);
        const long long base = crow * D;
        float dot = 0.f;
        for (int d = 0; d < D; ++d) dot += qs[wave][d] * Elt<T>::load(kc + base + d);
        s = dot * c;
      }
    }
    const float cmax = wave_max(s);
    if (cmax == -INFINITY) continue;  // nothing visible in this chunk
    const float mn = fmaxf(m, cmax);
    const float alpha = exp2f(m - mn);  // 0 on the first visible chunk
    const float p = (crow >= 0) ? exp2f(s - mn) : 0.f;
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] *= alpha;
    m = mn;
    for (int j = 0; j < 64; ++j) {
      const float pj = __shfl(p, j, 64);
      const long long cj = __shfl(crow, j, 64);
      if (cj < 0) continue;
      const long long bj = cj * D;
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] += pj * Elt<T>::load(vc + bj + lane + 64 * r);
    }
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int r = 0; r < R; ++r) Elt<T>::store(out + lane + 64 * r, acc[r] * inv);
}

template <typename T>
hipError_t launch_typed(const AttnArgs& a, hipStream_t stream) {
  const long rows = static_cast<long>(a.B) * a.N * a.Hq;
  const dim3 grid(static_cast<unsigned>((rows + kWaves - 1) / kWaves));
  if (a.D == 64)
    hipLaunchKernelGGL((attn_rowwave_kernel<T, 64>), grid, dim3(kWaves * 64), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_rowwave_kernel<T, 128>), grid, dim3(kWaves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_rowwave(const AttnArgs& a, tv_dtype dtype, hipStream_t stream) {
  return dtype == TV_F32 ? launch_typed<float>(a, stream) : launch_typed<uint16_t>(a, stream);
}

}  // namespace tv
