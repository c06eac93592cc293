// Tree K/V write with rotary positions ("EAGLE代码实现原理", KV缓存优化: cat()
// appends the step's new rows after the current length inside the
// preallocated cache; "P-EAGLE", 技术难点和解决方案: the block manager appends
// the proposed tokens to the paged cache).  Node i of sequence b is rotated
// to position P_b + depth(i): siblings share a position, and every
// root-to-leaf path carries consecutive positions, as if decoded alone.
//
// One workgroup per (sequence, node).  The D/2 rotation angles of the node
// are formed in fp64 (positions reach tens of thousands of radians) and
// reduced to fp32 (cos, sin) in LDS; each thread then turns four (x[j],
// x[j + D/2]) pairs of one head at a time, reading both halves before
// writing them, so q_out may alias q.  The rotated key and the value go to
// logical position P_b + i of the paged cache (either layout).
// The step is a stream of small rows: HBM-bound.
#include <math.h>

#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kThreads = 256;

template <typename T>
struct Vec4;
template <>
struct Vec4<float> {
  typedef float4 raw;  // four elements as loaded
  __device__ static raw load_raw(const float* p) { return *reinterpret_cast<const float4*>(p); }
  __device__ static void unpack(const raw& v, float (&x)[4]) {
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  }
  __device__ static void load(const float* p, float (&x)[4]) { unpack(load_raw(p), x); }
  __device__ static void store(float* p, const float (&x)[4]) {
    *reinterpret_cast<float4*>(p) = float4{x[0], x[1], x[2], x[3]};
  }
};
template <>
struct Vec4<uint16_t> {
  typedef uint2 raw;  // four elements as loaded
  __device__ static raw load_raw(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }
  __device__ static void unpack(const raw& v, float (&x)[4]) {
    x[0] = __uint_as_float(v.x << 16);
    x[1] = __uint_as_float(v.x & 0xFFFF0000u);
    x[2] = __uint_as_float(v.y << 16);
    x[3] = __uint_as_float(v.y & 0xFFFF0000u);
  }
  __device__ static void load(const uint16_t* p, float (&x)[4]) { unpack(load_raw(p), x); }
  __device__ static void store(uint16_t* p, const float (&x)[4]) {
    uint2 v;
    v.x = static_cast<uint32_t>(f32_to_bf16(x[0])) | (static_cast<uint32_t>(f32_to_bf16(x[1])) << 16);
    v.y = static_cast<uint32_t>(f32_to_bf16(x[2])) | (static_cast<uint32_t>(f32_to_bf16(x[3])) << 16);
    *reinterpret_cast<uint2*>(p) = v;
  }
};

template <typename T>
__global__ __launch_bounds__(kThreads) void tree_kv_write_kernel(KvWriteArgs a) {
  __shared__ float s_cos[64], s_sin[64];
  const int node = blockIdx.x % a.N, b = blockIdx.x / a.N;
  const int tid = threadIdx.x;
  const int D = a.D, h = D / 2;
  const size_t nidx = static_cast<size_t>(b) * a.N + node;
  // the chain that fixes where and how the rows go starts first
  const int P = a.prefix_lens[b];
  int d = a.depth[nidx];
  // D is 64 or 128: items decode with shifts
  const int quads = h / 4;  // groups of four pairs per head row
  const int qsh = __builtin_ctz(quads), csh = qsh + 1;  // log2 of quads and of D / 4
  const T* q = static_cast<const T*>(a.q) + nidx * a.Hq * D;
  T* qo = static_cast<T*>(a.q_out) + nidx * a.Hq * D;
  const T* kn = static_cast<const T*>(a.k_new) + nidx * a.Hkv * D;
  const T* vn = static_cast<const T*>(a.v_new) + nidx * a.Hkv * D;
  // items: Hq query rows, then Hkv key rows (rotated), then Hkv value rows (copied)
  const int rot_items = (a.Hq + a.Hkv) * quads;
  const int items = rot_items + a.Hkv * (D / 4);
  // the inputs of an item as loaded: the two halves r1, r2 of a rotated
  // row, or r1 of a value row
  using Raw = typename Vec4<T>::raw;
  // Both loads are unconditional, from addresses that are always inside the
  // inputs (a value row loads its one address twice; past the last item, q's
  // first four elements), so no branch merges loaded values and nothing
  // waits for a load before its item is finished.
  auto fetch = [&](int it, Raw& r1, Raw& r2) __attribute__((always_inline)) {
    const T* src = q;
    const T* src2 = q;
    if (it < rot_items) {
      const int row = it >> qsh;
      src = (row < a.Hq ? q + row * D : kn + (row - a.Hq) * D) + (it & (quads - 1)) * 4;
      src2 = src + h;
    } else if (it < items) {
      const int v_it = it - rot_items;
      src = vn + (v_it >> csh) * D + (v_it & ((D / 4) - 1)) * 4;
      src2 = src;
    }
    r1 = Vec4<T>::load_raw(src);
    r2 = Vec4<T>::load_raw(src2);
  };
  // The rows do not depend on the prefix length, depth or block table: this
  // thread's first four items are loaded before those, so their latencies
  // overlap (the rest of a large row set follows the same loop later).
  Raw p1a, p2a, p1b, p2b, p1c, p2c, p1d, p2d;
  fetch(tid, p1a, p2a);
  fetch(tid + kThreads, p1b, p2b);
  fetch(tid + 2 * kThreads, p1c, p2c);
  fetch(tid + 3 * kThreads, p1d, p2d);

  // where the node's K/V rows go: logical position P + node
  const long t = static_cast<long>(P) + node;
  int blk = -1;
  if (P >= 0 && t < static_cast<long>(a.max_blocks) * kBlockSize) blk = a.block_table[static_cast<size_t>(b) * a.max_blocks + t / kBlockSize];
  if (tid == 0) {
    if (d < 0 || d >= a.N) report(a.dev_status, TV_DEV_BAD_TREE);
    if (blk < 0 || blk >= a.num_blocks) report(a.dev_status, TV_DEV_BAD_CACHE);
  }
  d = (d < 0 || d >= a.N) ? 0 : d;
  const double pos = static_cast<double>(P < 0 ? 0 : P) + d;
  if (tid < h) {
    // pos * theta^(-2 j / D) in fp64, then fp32 cos and sin of it
    const double ang = pos * pow(static_cast<double>(a.theta), -2.0 * tid / D);
    double sn, cs;
    sincos(ang, &sn, &cs);
    s_cos[tid] = static_cast<float>(cs);
    s_sin[tid] = static_cast<float>(sn);
  }
  __syncthreads();

  const bool write_cache = blk >= 0 && blk < a.num_blocks;
  const int slot = static_cast<int>(t % kBlockSize);
  T* kc = static_cast<T*>(a.k_cache);
  T* vc = static_cast<T*>(a.v_cache);
  // rotate (or copy) an item whose inputs are loaded, and store it
  auto finish = [&](int it, const Raw& r1, const Raw& r2) __attribute__((always_inline)) {
    float x1[4], x2[4];
    Vec4<T>::unpack(r1, x1);
    Vec4<T>::unpack(r2, x2);
    if (it < rot_items) {
      const int row = it >> qsh, j = (it & (quads - 1)) * 4;
      const bool is_q = row < a.Hq;
      if (!is_q && !write_cache) return;
      float y1[4], y2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float c = s_cos[j + e], s = s_sin[j + e];
        y1[e] = x1[e] * c - x2[e] * s;
        y2[e] = x2[e] * c + x1[e] * s;
      }
      T* dst = is_q ? qo + row * D
                    : kc + kv_row(blk, row - a.Hq, slot, a.Hkv, a.kv_head_rows, a.kv_slot_rows) * D;
      Vec4<T>::store(dst + j, y1);
      Vec4<T>::store(dst + j + h, y2);
    } else if (it < items && write_cache) {
      const int v_it = it - rot_items;
      const int head = v_it >> csh, j = (v_it & ((D / 4) - 1)) * 4;
      Vec4<T>::store(vc + kv_row(blk, head, slot, a.Hkv, a.kv_head_rows, a.kv_slot_rows) * D + j, x1);
    }
  };
  finish(tid, p1a, p2a);
  finish(tid + kThreads, p1b, p2b);
  finish(tid + 2 * kThreads, p1c, p2c);
  finish(tid + 3 * kThreads, p1d, p2d);
  for (int it = tid + 4 * kThreads; it < items; it += kThreads) {
    Raw r1, r2;
    fetch(it, r1, r2);
    finish(it, r1, r2);
  }
}

}  // namespace

hipError_t launch_tree_kv_write(const KvWriteArgs& a, tv_dtype dtype, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.B * a.N));
  if (dtype == TV_BF16)
    hipLaunchKernelGGL(tree_kv_write_kernel<uint16_t>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(tree_kv_write_kernel<float>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace tv
