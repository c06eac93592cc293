// Host side of the C ABI declared in tv.h: argument checks, workspace sizing
// and kernel launches on the caller's stream.  Nothing here allocates or
// keeps state between calls.
#include <math.h>

#include "tv_internal.h"

using namespace tv;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

tv_status launched(hipError_t e) { return e == hipSuccess ? TV_OK : TV_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char* tv_status_string(tv_status s) {
  switch (s) {
    case TV_OK: return "TV_OK";
    case TV_ERR_NULL: return "TV_ERR_NULL: a required pointer is NULL";
    case TV_ERR_SHAPE: return "TV_ERR_SHAPE: sizes are inconsistent or out of range";
    case TV_ERR_DTYPE: return "TV_ERR_DTYPE: dtype must be TV_F32 or TV_BF16 (with TV_KV_TOKEN_MAJOR only where a cache is taken)";
    case TV_ERR_UNSUPPORTED: return "TV_ERR_UNSUPPORTED: D must be 64 or 128, block_size 16, and H a multiple of 64";
    case TV_ERR_ALIGN: return "TV_ERR_ALIGN: a tensor pointer is not 16-byte aligned";
    case TV_ERR_WORKSPACE: return "TV_ERR_WORKSPACE: workspace missing or too small";
    case TV_ERR_LAUNCH: return "TV_ERR_LAUNCH: kernel launch failed";
    case TV_ERR_TOO_LARGE: return "TV_ERR_TOO_LARGE: the sizes need more scratch than the static buffer holds";
  }
  return "unknown tv_status";
}

int tv_version(void) { return 100; }

tv_status tv_build_tree_mask(const int32_t* parents, int32_t B, int32_t N, uint64_t* mask,
                             int32_t* depth, int32_t* dev_status, hipStream_t stream) {
  if (!parents || !mask) return TV_ERR_NULL;
  if (B <= 0 || N <= 0 || N > TV_MAX_NODES) return TV_ERR_SHAPE;
  return launched(launch_tree_mask(parents, B, N, mask, depth, dev_status, stream));
}

size_t tv_tree_attention_workspace_size(int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                        int32_t max_prefix_len) {
  // the bf16 path's need; the fp32 path needs none
  if (B <= 0 || N <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || max_prefix_len < 0 || (D != 64 && D != 128))
    return 0;
  return attention_mfma_workspace_bytes(B, N, Hq, Hkv, D, max_prefix_len);
}

}  // extern "C"

// tv_tree_attention and tv_tree_attention_parents: the same checks and
// launch, with the masks given (mask) or built from the parents in the
// attention kernels (parents, N <= 64)
static tv_status tree_attention(const void* q, const void* k_cache, const void* v_cache, int32_t num_blocks,
                                const int32_t* block_table, int32_t max_blocks, int32_t block_size,
                                const int32_t* prefix_lens, int32_t max_prefix_len, const uint64_t* mask,
                                const int32_t* parents, void* out, int32_t B, int32_t N, int32_t Hq, int32_t Hkv,
                                int32_t D, float scale, tv_dtype dtype, void* workspace, size_t workspace_bytes,
                                int32_t* dev_status, hipStream_t stream) {
  if (!q || !k_cache || !v_cache || !block_table || !prefix_lens || !(mask || parents) || !out) return TV_ERR_NULL;
  const bool token_major = (dtype & TV_KV_TOKEN_MAJOR) != 0;
  dtype = static_cast<tv_dtype>(dtype & ~TV_KV_TOKEN_MAJOR);
  if (dtype != TV_F32 && dtype != TV_BF16) return TV_ERR_DTYPE;
  if (B <= 0 || N <= 0 || N > TV_MAX_NODES || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 ||
      num_blocks <= 0 || max_blocks <= 0 || max_prefix_len < 0)
    return TV_ERR_SHAPE;
  if (D != 64 && D != 128) return TV_ERR_UNSUPPORTED;
  if (block_size != kBlockSize) return TV_ERR_UNSUPPORTED;
  if (!mask && N > 64) return TV_ERR_UNSUPPORTED;  // one wave builds the masks
  if (static_cast<long>(max_prefix_len) + N > static_cast<long>(max_blocks) * block_size)
    return TV_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return TV_ERR_ALIGN;
  const size_t need = dtype == TV_BF16 ? tv_tree_attention_workspace_size(B, N, Hq, Hkv, D, max_prefix_len) : 0;
  if (need > 0 && (!workspace || workspace_bytes < need)) return TV_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return TV_ERR_ALIGN;

  AttnArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_blocks = num_blocks;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.prefix_lens = prefix_lens;
  a.max_prefix_len = max_prefix_len;
  a.mask = mask;
  a.parents = mask ? nullptr : parents;
  a.out = out;
  a.B = B;
  a.N = N;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  const KvLayout lay = kv_layout(token_major, Hkv);
  a.kv_head_rows = lay.head_rows;
  a.kv_slot_rows = lay.slot_rows;
  a.scale = scale > 0.f ? scale : 1.f / sqrtf(static_cast<float>(D));
  a.workspace = workspace;
  a.dev_status = dev_status;
  if (dtype == TV_BF16) return launched(launch_attention_mfma(a, stream));
  return launched(launch_attention_rowwave(a, dtype, stream));
}

extern "C" {

tv_status tv_tree_attention(const void* q, const void* k_cache, const void* v_cache,
                            int32_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                            int32_t block_size, const int32_t* prefix_lens, int32_t max_prefix_len,
                            const uint64_t* mask, void* out, int32_t B, int32_t N, int32_t Hq,
                            int32_t Hkv, int32_t D, float scale, tv_dtype dtype, void* workspace,
                            size_t workspace_bytes, int32_t* dev_status, hipStream_t stream) {
  if (!mask) return TV_ERR_NULL;
  return tree_attention(q, k_cache, v_cache, num_blocks, block_table, max_blocks, block_size, prefix_lens,
                        max_prefix_len, mask, nullptr, out, B, N, Hq, Hkv, D, scale, dtype, workspace,
                        workspace_bytes, dev_status, stream);
}

tv_status tv_tree_attention_parents(const void* q, const void* k_cache, const void* v_cache,
                                    int32_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                                    int32_t block_size, const int32_t* prefix_lens, int32_t max_prefix_len,
                                    const int32_t* parents, void* out, int32_t B, int32_t N, int32_t Hq,
                                    int32_t Hkv, int32_t D, float scale, tv_dtype dtype, void* workspace,
                                    size_t workspace_bytes, int32_t* dev_status, hipStream_t stream) {
  if (!parents) return TV_ERR_NULL;
  return tree_attention(q, k_cache, v_cache, num_blocks, block_table, max_blocks, block_size, prefix_lens,
                        max_prefix_len, nullptr, parents, out, B, N, Hq, Hkv, D, scale, dtype, workspace,
                        workspace_bytes, dev_status, stream);
}

size_t tv_accept_greedy_workspace_size(int32_t B, int32_t N, int32_t V) {
  if (B <= 0 || N <= 0 || V <= 0) return 0;
  return accept_workspace_bytes(B, N, V);
}

tv_status tv_accept_greedy(const float* logits, const int32_t* draft_tokens, const int32_t* parents,
                           int32_t B, int32_t N, int32_t V, int32_t* accept_len,
                           int32_t* accepted_nodes, int32_t* bonus_token, int32_t* target_argmax,
                           void* workspace, size_t workspace_bytes, int32_t* dev_status,
                           hipStream_t stream) {
  if (!logits || !draft_tokens || !parents || !accept_len || !accepted_nodes || !bonus_token)
    return TV_ERR_NULL;
  if (B <= 0 || N <= 0 || N > TV_MAX_NODES || V <= 0) return TV_ERR_SHAPE;
  if (!aligned16(logits)) return TV_ERR_ALIGN;
  if (!workspace || workspace_bytes < accept_workspace_bytes(B, N, V)) return TV_ERR_WORKSPACE;
  AcceptArgs a{};  // no compaction
  a.logits = logits;
  a.draft_tokens = draft_tokens;
  a.parents = parents;
  a.B = B;
  a.N = N;
  a.V = V;
  a.accept_len = accept_len;
  a.accepted_nodes = accepted_nodes;
  a.bonus_token = bonus_token;
  a.target_argmax = target_argmax;
  a.workspace = workspace;
  a.dev_status = dev_status;
  return launched(launch_accept(a, stream));
}

tv_status tv_accept_greedy_noalloc(const float* logits, const int32_t* draft_tokens, const int32_t* parents,
                                   int32_t B, int32_t N, int32_t V, int32_t* accept_len,
                                   int32_t* accepted_nodes, int32_t* bonus_token, int32_t* target_argmax,
                                   int32_t* dev_status, hipStream_t stream) {
  if (!logits || !draft_tokens || !parents || !accept_len || !accepted_nodes || !bonus_token)
    return TV_ERR_NULL;
  if (B <= 0 || N <= 0 || N > TV_MAX_NODES || V <= 0) return TV_ERR_SHAPE;
  if (!aligned16(logits)) return TV_ERR_ALIGN;
  if (accept_workspace_bytes(B, N, V) > kAcceptScratchBytes) return TV_ERR_TOO_LARGE;
  void* scratch = nullptr;
  if (accept_static_scratch(stream, &scratch) != hipSuccess) return TV_ERR_LAUNCH;
  AcceptArgs a{};  // no compaction
  a.logits = logits;
  a.draft_tokens = draft_tokens;
  a.parents = parents;
  a.B = B;
  a.N = N;
  a.V = V;
  a.accept_len = accept_len;
  a.accepted_nodes = accepted_nodes;
  a.bonus_token = bonus_token;
  a.target_argmax = target_argmax;
  a.workspace = scratch;
  a.dev_status = dev_status;
  return launched(launch_accept(a, stream));
}

size_t tv_accept_stochastic_workspace_size(int32_t B, int32_t N, int32_t V) {
  if (B <= 0 || N <= 0 || N > TV_MAX_NODES || V <= 0) return 0;
  return stochastic_workspace_bytes(B, N, V);
}

tv_status tv_accept_stochastic(const float* logits, const float* draft_probs, const int32_t* draft_tokens,
                               const int32_t* parents, const float* uniforms, const float* exponentials,
                               int32_t B, int32_t N, int32_t V, float temperature, int32_t* accept_len,
                               int32_t* accepted_nodes, int32_t* bonus_token, void* workspace,
                               size_t workspace_bytes, int32_t* dev_status, hipStream_t stream) {
  if (!logits || !draft_tokens || !parents || !uniforms || !exponentials || !accept_len || !accepted_nodes ||
      !bonus_token)
    return TV_ERR_NULL;
  if (B <= 0 || N <= 0 || N > TV_MAX_NODES || V <= 0 || !(temperature > 0.f && temperature < INFINITY))
    return TV_ERR_SHAPE;
  if (!aligned16(logits) || (draft_probs && !aligned16(draft_probs))) return TV_ERR_ALIGN;
  if (!workspace || workspace_bytes < stochastic_workspace_bytes(B, N, V)) return TV_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TV_ERR_ALIGN;
  StochArgs a;
  a.logits = logits;
  a.draft_probs = draft_probs;
  a.draft_tokens = draft_tokens;
  a.parents = parents;
  a.uniforms = uniforms;
  a.exponentials = exponentials;
  a.B = B;
  a.N = N;
  a.V = V;
  a.temperature = temperature;
  a.accept_len = accept_len;
  a.accepted_nodes = accepted_nodes;
  a.bonus_token = bonus_token;
  a.workspace = workspace;
  a.dev_status = dev_status;
  return launched(launch_accept_stochastic(a, stream));
}

size_t tv_lm_head_argmax_workspace_size(int32_t M, int32_t H, int32_t V) {
  if (M <= 0 || H <= 0 || V <= 0) return 0;
  return lm_head_workspace_bytes(M, V);
}

tv_status tv_lm_head_argmax(const void* hidden, const void* weight, int32_t M, int32_t H, int32_t V,
                            tv_dtype dtype, int32_t* argmax, float* max_score, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (!hidden || !weight || !argmax) return TV_ERR_NULL;
  if (dtype != TV_BF16) return TV_ERR_DTYPE;
  // the score kernel addresses one 256-row slab of the weight with 32-bit offsets
  if (M <= 0 || H <= 0 || V <= 0 || H > 1 << 20) return TV_ERR_SHAPE;
  if (H % 64 != 0) return TV_ERR_UNSUPPORTED;
  if (!aligned16(hidden) || !aligned16(weight)) return TV_ERR_ALIGN;
  if (!workspace || workspace_bytes < lm_head_workspace_bytes(M, V)) return TV_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TV_ERR_ALIGN;
  LmArgs a;
  a.hidden = hidden;
  a.weight = weight;
  a.M = M;
  a.H = H;
  a.V = V;
  a.argmax = argmax;
  a.max_score = max_score;
  a.workspace = workspace;
  return launched(launch_lm_head_argmax(a, stream));
}

static bool draft_tree_shape_ok(int32_t B, int32_t depth, int32_t topk, int32_t V) {
  return B > 0 && depth >= 1 && depth <= TV_DRAFT_MAX_DEPTH && topk >= 1 && topk <= TV_DRAFT_MAX_TOPK &&
         topk <= V && V <= TV_DRAFT_MAX_VOCAB;
}

size_t tv_build_draft_tree_workspace_size(int32_t B, int32_t depth, int32_t topk, int32_t V) {
  if (!draft_tree_shape_ok(B, depth, topk, V)) return 0;
  return draft_tree_workspace_bytes(B, depth, topk, V);
}

tv_status tv_build_draft_tree(const float* draft_logits, int32_t B, int32_t depth, int32_t topk, int32_t V,
                              int32_t N, const int32_t* root_tokens, int32_t* parents, int32_t* tokens,
                              float* scores, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!draft_logits || !parents || !tokens) return TV_ERR_NULL;
  if (!draft_tree_shape_ok(B, depth, topk, V) || N < 1 || N > TV_MAX_NODES) return TV_ERR_SHAPE;
  const long generated = topk + static_cast<long>(depth - 1) * topk * topk;
  if (N - 1 > generated) return TV_ERR_SHAPE;
  if (!aligned16(draft_logits)) return TV_ERR_ALIGN;
  if (!workspace || workspace_bytes < draft_tree_workspace_bytes(B, depth, topk, V)) return TV_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TV_ERR_ALIGN;
  DraftTreeArgs a;
  a.draft_logits = draft_logits;
  a.B = B;
  a.depth = depth;
  a.topk = topk;
  a.V = V;
  a.N = N;
  a.root_tokens = root_tokens;
  a.parents = parents;
  a.tokens = tokens;
  a.scores = scores;
  a.workspace = workspace;
  return launched(launch_draft_tree(a, stream));
}

}  // extern "C"

// Host checks of a compaction's cache arguments, and its argument record
// (tv_kv_compact and the fused acceptance call).
static tv_status make_compact_args(void* k_cache, void* v_cache, int32_t num_blocks, const int32_t* block_table,
                                   int32_t max_blocks, int32_t block_size, const int32_t* prefix_lens, int32_t B,
                                   int32_t N, int32_t Hkv, int32_t D, tv_dtype dtype, int32_t* new_lens,
                                   int32_t* dev_status, CompactArgs* out) {
  if (!k_cache || !v_cache || !block_table || !prefix_lens) return TV_ERR_NULL;
  const bool token_major = (dtype & TV_KV_TOKEN_MAJOR) != 0;
  dtype = static_cast<tv_dtype>(dtype & ~TV_KV_TOKEN_MAJOR);
  if (dtype != TV_F32 && dtype != TV_BF16) return TV_ERR_DTYPE;
  if (B <= 0 || N <= 0 || N > TV_MAX_NODES || Hkv <= 0 || num_blocks <= 0 || max_blocks <= 0)
    return TV_ERR_SHAPE;
  if (D != 64 && D != 128) return TV_ERR_UNSUPPORTED;
  if (block_size != kBlockSize) return TV_ERR_UNSUPPORTED;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return TV_ERR_ALIGN;
  CompactArgs& a = *out;
  a = CompactArgs{};
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_blocks = num_blocks;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.prefix_lens = prefix_lens;
  a.B = B;
  a.N = N;
  a.Hkv = Hkv;
  a.D = D;
  const KvLayout lay = kv_layout(token_major, Hkv);
  a.kv_head_rows = lay.head_rows;
  a.kv_slot_rows = lay.slot_rows;
  a.elt_bytes = dtype == TV_F32 ? 4 : 2;
  a.new_lens = new_lens;
  a.dev_status = dev_status;
  return TV_OK;
}

extern "C" {

tv_status tv_kv_compact(void* k_cache, void* v_cache, int32_t num_blocks, const int32_t* block_table,
                        int32_t max_blocks, int32_t block_size, const int32_t* prefix_lens,
                        const int32_t* accepted_nodes, const int32_t* accept_len, int32_t B,
                        int32_t N, int32_t Hkv, int32_t D, tv_dtype dtype, int32_t* new_lens,
                        int32_t* dev_status, hipStream_t stream) {
  if (!accepted_nodes || !accept_len) return TV_ERR_NULL;
  CompactArgs a;
  const tv_status st = make_compact_args(k_cache, v_cache, num_blocks, block_table, max_blocks, block_size,
                                         prefix_lens, B, N, Hkv, D, dtype, new_lens, dev_status, &a);
  if (st != TV_OK) return st;
  a.accepted_nodes = accepted_nodes;
  a.accept_len = accept_len;
  return launched(launch_kv_compact(a, stream));
}

tv_status tv_accept_greedy_compact(const float* logits, const int32_t* draft_tokens, const int32_t* parents,
                                   int32_t B, int32_t N, int32_t V, int32_t* accept_len, int32_t* accepted_nodes,
                                   int32_t* bonus_token, int32_t* target_argmax, void* workspace,
                                   size_t workspace_bytes, void* k_cache, void* v_cache, int32_t num_blocks,
                                   const int32_t* block_table, int32_t max_blocks, int32_t block_size,
                                   const int32_t* prefix_lens, int32_t Hkv, int32_t D, tv_dtype dtype,
                                   int32_t* new_lens, int32_t* dev_status, hipStream_t stream) {
  if (!logits || !draft_tokens || !parents || !accept_len || !accepted_nodes || !bonus_token)
    return TV_ERR_NULL;
  if (B <= 0 || N <= 0 || N > TV_MAX_NODES || V <= 0) return TV_ERR_SHAPE;
  AcceptArgs a{};
  const tv_status st = make_compact_args(k_cache, v_cache, num_blocks, block_table, max_blocks, block_size,
                                         prefix_lens, B, N, Hkv, D, dtype, new_lens, dev_status, &a.compact);
  if (st != TV_OK) return st;
  if (!aligned16(logits)) return TV_ERR_ALIGN;
  if (!workspace || workspace_bytes < accept_workspace_bytes(B, N, V)) return TV_ERR_WORKSPACE;
  a.logits = logits;
  a.draft_tokens = draft_tokens;
  a.parents = parents;
  a.B = B;
  a.N = N;
  a.V = V;
  a.accept_len = accept_len;
  a.accepted_nodes = accepted_nodes;
  a.bonus_token = bonus_token;
  a.target_argmax = target_argmax;
  a.workspace = workspace;
  a.dev_status = dev_status;
  return launched(launch_accept(a, stream));
}

tv_status tv_tree_kv_write(const void* q, const void* k_new, const void* v_new, const int32_t* depth,
                           void* q_out, void* k_cache, void* v_cache, int32_t num_blocks,
                           const int32_t* block_table, int32_t max_blocks, int32_t block_size,
                           const int32_t* prefix_lens, int32_t B, int32_t N, int32_t Hq, int32_t Hkv,
                           int32_t D, float rope_theta, tv_dtype dtype, int32_t* dev_status,
                           hipStream_t stream) {
  if (!q || !k_new || !v_new || !depth || !q_out || !k_cache || !v_cache || !block_table || !prefix_lens)
    return TV_ERR_NULL;
  const bool token_major = (dtype & TV_KV_TOKEN_MAJOR) != 0;
  dtype = static_cast<tv_dtype>(dtype & ~TV_KV_TOKEN_MAJOR);
  if (dtype != TV_F32 && dtype != TV_BF16) return TV_ERR_DTYPE;
  if (B <= 0 || N <= 0 || N > TV_MAX_NODES || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || num_blocks <= 0 ||
      max_blocks <= 0 || !(rope_theta > 0.f))
    return TV_ERR_SHAPE;
  if (D != 64 && D != 128) return TV_ERR_UNSUPPORTED;
  if (block_size != kBlockSize) return TV_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(q_out) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return TV_ERR_ALIGN;
  KvWriteArgs a;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.depth = depth;
  a.q_out = q_out;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_blocks = num_blocks;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.prefix_lens = prefix_lens;
  a.B = B;
  a.N = N;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  const KvLayout lay = kv_layout(token_major, Hkv);
  a.kv_head_rows = lay.head_rows;
  a.kv_slot_rows = lay.slot_rows;
  a.theta = rope_theta;
  a.dev_status = dev_status;
  return launched(launch_tree_kv_write(a, dtype, stream));
}

}  // extern "C"
