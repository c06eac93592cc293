// Moving the accepted rows of one sequence: shared by the compaction kernel
// and the acceptance kernel that compacts as it walks ("EAGLE代码实现原理",
// KV缓存优化: copy(indices, prev_length) gathers the indexed rows and writes
// them from prev_length).
#pragma once

#include "tv_internal.h"

namespace tv {

// Steps j = 1 .. L-1 move cache row src[j] to row dst[j] (rows at KV head 0,
// in D-element units; step 0 is the root, which never moves) in K and V, for
// every KV head; steps with src[j] == dst[j] are skipped.  The workgroup's
// nthreads threads (this one is tid) share the 16-byte columns of a token.
// src and dst are the workgroup's LDS arrays.
__device__ __forceinline__ void compact_copy_columns(const CompactArgs& a, const long long* s_src,
                                                     const long long* s_dst, int s_L, int tid, int nthreads) {
  // 16-byte columns of a token: dq per head row (D elements), Hkv heads.
  // Steps go in batches of 8: all sources of a batch are loaded before its
  // stores.  A batch's sources path[j] >= j are never an earlier
  // destination, and a destination j that is the source of an earlier step
  // of the batch is stored after that load, so batches keep
  // gather-before-write.
  const int dq = a.D * a.elt_bytes / 16;
  const int cols = a.Hkv * dq;
  for (int c = tid; c < 2 * cols; c += nthreads) {
    int4* base = reinterpret_cast<int4*>(c < cols ? a.k_cache : a.v_cache);
    const int cc = c < cols ? c : c - cols;
    // head cc / dq sits (cc / dq) * kv_head_rows rows after head 0
    const long long col = static_cast<long long>(cc / dq) * a.kv_head_rows * dq + cc % dq;
    for (int j0 = 1; j0 < s_L; j0 += 8) {
      // every lane loads eight rows (steps past L or without a move read
      // column col of block 0, head 0, slot 0, which is in bounds), so the
      // batch stays in registers; only real moves are stored
      const int L = s_L;
      int4 v0, v1, v2, v3, v4, v5, v6, v7;
      long long d0, d1, d2, d3, d4, d5, d6, d7;  // destination index, -1: no move
      auto load = [&](int j, int4& v, long long& d) __attribute__((always_inline)) {
        const bool mv = j < L && s_src[j] != s_dst[j];
        v = base[(mv ? s_src[j] * dq : 0) + col];
        d = mv ? s_dst[j] * dq + col : -1;
      };
      load(j0 + 0, v0, d0);
      load(j0 + 1, v1, d1);
      load(j0 + 2, v2, d2);
      load(j0 + 3, v3, d3);
      load(j0 + 4, v4, d4);
      load(j0 + 5, v5, d5);
      load(j0 + 6, v6, d6);
      load(j0 + 7, v7, d7);
      if (d0 >= 0) base[d0] = v0;
      if (d1 >= 0) base[d1] = v1;
      if (d2 >= 0) base[d2] = v2;
      if (d3 >= 0) base[d3] = v3;
      if (d4 >= 0) base[d4] = v4;
      if (d5 >= 0) base[d5] = v5;
      if (d6 >= 0) base[d6] = v6;
      if (d7 >= 0) base[d7] = v7;
    }
  }
}

}  // namespace tv
