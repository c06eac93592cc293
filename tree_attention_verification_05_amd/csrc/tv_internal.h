// Internal declarations shared by the host API and the kernel translation
// units of libtv (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tv.h"

namespace tv {

constexpr int kBlockSize = 16;   // tokens per paged-cache block

// Paged-cache layout.  A block holds kBlockSize slots of Hkv heads, each a
// row of D elements; the row of (block, head, slot) is
//   block * kBlockSize * Hkv + head * head_rows + slot * slot_rows.
// Head-major blocks ([block][head][slot][D], the default) keep one head's
// slots together: head_rows = kBlockSize, slot_rows = 1.  Token-major blocks
// ([block][slot][head][D]) keep one slot's heads together: head_rows = 1,
// slot_rows = Hkv.
struct KvLayout {
  int head_rows;
  int slot_rows;
};
inline KvLayout kv_layout(bool token_major, int Hkv) {
  return token_major ? KvLayout{1, Hkv} : KvLayout{kBlockSize, 1};
}
__host__ __device__ __forceinline__ long long kv_row(long long block, int head, int slot, int Hkv, int head_rows,
                                                     int slot_rows) {
  return block * kBlockSize * Hkv + static_cast<long long>(head) * head_rows +
         static_cast<long long>(slot) * slot_rows;
}

// ---- bf16 helpers (storage is the raw 16-bit pattern) ----
__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}
// round to nearest even; inputs are finite
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T> struct Elt;
template <> struct Elt<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};
template <> struct Elt<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void store(uint16_t* p, float v) { *p = f32_to_bf16(v); }
};

__device__ __forceinline__ void report(int32_t* dev_status, int bits) {
  if (dev_status) atomicOr(dev_status, bits);
}

// Ancestor-or-self bits of every node of one tree of N <= 64 nodes, computed
// by a whole wave ("vLLM-TreeEagle" README, 核心组件 item 1 and 技术创新点 1:
// the mask follows the tree, whatever its shape).  Lane l passes node l's
// parent (anything for l >= N).  Six rounds of pointer jumping: each node ORs
// in the bits of the node its jump pointer names and then jumps to that
// node's jump target, so after round r it holds its ancestors up to 2^r - 1
// edges up, and after six every depth a 64-node tree can have.  Lane l gets
// node l's word (0 for l >= N).  When the parents are not a tree
// (parent[0] != -1, or parent[i] outside [0, i)) every lane gets 0 and *bad
// is set, as the mask kernel leaves such a sequence.  Every lane of the wave
// must call it.
__device__ __forceinline__ uint64_t wave_tree_mask(int p, int N, int lane, bool* bad) {
  const bool exists = lane < N;
  const bool ok = !exists || (lane == 0 ? p == -1 : (p >= 0 && p < lane));
  const bool any_bad = __builtin_amdgcn_ballot_w64(!ok) != 0;
  uint64_t anc = exists ? (1ull << lane) : 0ull;
  int jump = (exists && lane > 0 && ok) ? p : -1;
  // (rounds stop early once no node has an ancestor left to add: a tree of
  // depth d needs ceil(log2(d + 1)) of them)
  for (int r = 0; r < 6 && __builtin_amdgcn_ballot_w64(jump >= 0) != 0; ++r) {
    const int src = jump >= 0 ? jump : lane;
    const uint64_t up = __shfl(anc, src, 64);
    const int up_jump = __shfl(jump, src, 64);
    if (jump >= 0) {
      anc |= up;
      jump = up_jump;
    }
  }
  *bad = any_bad;
  return any_bad ? 0ull : anc;
}

// ---- ordered 64-bit selection keys (one definition for every kernel that
// picks a maximum with the lowest index winning ties) ----
// Orders floats as unsigned integers; -0.0 and +0.0 map to the same value.
__device__ __forceinline__ uint32_t ordered(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unordered(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
// Larger key = larger value, then lower index.  Every key of a finite value
// is nonzero, so 0 can mark "none".
__device__ __forceinline__ uint64_t make_key(float v, uint32_t idx) {
  return (static_cast<uint64_t>(ordered(v)) << 32) | static_cast<uint32_t>(~idx);
}
__device__ __forceinline__ uint32_t key_index(uint64_t k) { return ~static_cast<uint32_t>(k & 0xFFFFFFFFu); }
__device__ __forceinline__ float key_value(uint64_t k) { return unordered(static_cast<uint32_t>(k >> 32)); }

// ---- LDS copies straight from a buffer (gfx950 buffer_load ... lds) ----
#define LDS_AS __attribute__((address_space(3)))
#define CONST_AS __attribute__((address_space(4)))
constexpr int kNonTemporal = 2;  // cache-policy bit of a buffer access (gfx950: nt)

// One wave copies 64 x 16 bytes from a buffer (base, range in bytes;
// per-lane byte offset) into LDS: lane l's bytes land at dst + 16 l.  Reads
// past the range return zeros.  POLICY is the copy's cache policy: 0, or
// kNonTemporal for data that no other workgroup reads again.  (A plain
// device function: lambdas would also be compiled for the host, which has no
// buffer resources.)
template <int POLICY = 0>
__device__ __forceinline__ void copy_to_lds(const char* base, int range, int voff, uint16_t* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, range, 0x00020000),
      (LDS_AS void*)dst, 16, voff, 0, 0, POLICY);
}

// ---- launchers (each defined in its kernel translation unit) ----
hipError_t launch_tree_mask(const int32_t* parents, int B, int N, uint64_t* mask, int32_t* depth,
                            int32_t* dev_status, hipStream_t stream);

struct AttnArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  int num_blocks;
  const int32_t* block_table;
  int max_blocks;
  const int32_t* prefix_lens;
  int max_prefix_len;
  const uint64_t* mask;     // ancestor masks, or NULL:
  const int32_t* parents;   // the masks are built from the parents (N <= 64)
  void* out;
  int B, N, Hq, Hkv, D;
  int kv_head_rows, kv_slot_rows;  // cache layout (KvLayout)
  float scale;
  void* workspace;
  int32_t* dev_status;
};

// fp32 path: one wavefront per (sequence, node, query head) row.
hipError_t launch_attention_rowwave(const AttnArgs& a, tv_dtype dtype, hipStream_t stream);

// bf16 path: matrix-core split-KV kernel (+ split merge when the key range is split).
size_t attention_mfma_workspace_bytes(int B, int N, int Hq, int Hkv, int D, int max_prefix_len);
hipError_t launch_attention_mfma(const AttnArgs& a, hipStream_t stream);

struct CompactArgs {
  void* k_cache;
  void* v_cache;
  int num_blocks;
  const int32_t* block_table;
  int max_blocks;
  const int32_t* prefix_lens;
  const int32_t* accepted_nodes;
  const int32_t* accept_len;
  int B, N, Hkv, D;
  int kv_head_rows, kv_slot_rows;  // cache layout (KvLayout)
  int elt_bytes;
  int32_t* new_lens;
  int32_t* dev_status;
};
struct AcceptArgs {
  const float* logits;
  const int32_t* draft_tokens;
  const int32_t* parents;
  int B, N, V;
  int32_t* accept_len;
  int32_t* accepted_nodes;
  int32_t* bonus_token;
  int32_t* target_argmax;
  void* workspace;
  int32_t* dev_status;
  // compaction of the accepted path by the walking workgroup (k_cache NULL:
  // walk only)
  CompactArgs compact;
};
size_t accept_workspace_bytes(int B, int N, int V);
hipError_t launch_accept(const AcceptArgs& a, hipStream_t stream);
// the allocation-free variant's static scratch: its size, and the device
// address of the copy on the device of `stream` (looked up on first use)
constexpr size_t kAcceptScratchBytes = TV_ACCEPT_NOALLOC_SCRATCH_BYTES;
hipError_t accept_static_scratch(hipStream_t stream, void** ptr);

struct StochArgs {
  const float* logits;
  const float* draft_probs;  // NULL: point-mass proposals
  const int32_t* draft_tokens;
  const int32_t* parents;
  const float* uniforms;
  const float* exponentials;
  int B, N, V;
  float temperature;
  int32_t* accept_len;
  int32_t* accepted_nodes;
  int32_t* bonus_token;
  void* workspace;
  int32_t* dev_status;
};
size_t stochastic_workspace_bytes(int B, int N, int V);
hipError_t launch_accept_stochastic(const StochArgs& a, hipStream_t stream);

struct LmArgs {
  const void* hidden;  // [M][H] bf16
  const void* weight;  // [V][H] bf16
  int M, H, V;
  int32_t* argmax;
  float* max_score;    // may be NULL
  void* workspace;
};
size_t lm_head_workspace_bytes(int M, int V);
hipError_t launch_lm_head_argmax(const LmArgs& a, hipStream_t stream);

struct DraftTreeArgs {
  const float* draft_logits;  // [B][depth][topk][V]
  int B, depth, topk, V, N;
  const int32_t* root_tokens;  // may be NULL
  int32_t* parents;
  int32_t* tokens;
  float* scores;               // may be NULL
  void* workspace;
};
size_t draft_tree_workspace_bytes(int B, int depth, int topk, int V);
hipError_t launch_draft_tree(const DraftTreeArgs& a, hipStream_t stream);

hipError_t launch_kv_compact(const CompactArgs& a, hipStream_t stream);

struct KvWriteArgs {
  const void* q;
  const void* k_new;
  const void* v_new;
  const int32_t* depth;
  void* q_out;
  void* k_cache;
  void* v_cache;
  int num_blocks;
  const int32_t* block_table;
  int max_blocks;
  const int32_t* prefix_lens;
  int B, N, Hq, Hkv, D;
  int kv_head_rows, kv_slot_rows;  // cache layout (KvLayout)
  float theta;
  int32_t* dev_status;
};
hipError_t launch_tree_kv_write(const KvWriteArgs& a, tv_dtype dtype, hipStream_t stream);

}  // namespace tv
