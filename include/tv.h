/*
 * tv.h -- single-pass verification of a draft token tree on AMD Instinct
 * MI355X (gfx950): tree mask, tree-masked paged attention, greedy acceptance
 * and KV compaction.
 *
 * The problem (web pages, cited by title and section):
 *   - "vLLM-TreeEagle: Tree Attention优化的EAGLE3推测解码框架" (README),
 *     核心组件 item 1 TreeAttentionLayer and 技术创新点 1: the target model
 *     verifies every candidate path of a draft tree in one forward pass under a
 *     tree attention mask that is built at run time for any tree shape; the
 *     architecture graph puts this layer on top of PagedAttention.
 *   - "EAGLE代码实现原理：从树结构缓冲到KV缓存优化的技术细节", 树结构缓冲: all
 *     candidate paths share their common prefix; KV缓存优化:
 *     KVCache.copy(indices, prev_length) gathers accepted rows and writes them
 *     contiguously from prev_length.
 *   - "P-EAGLE：vLLM集成并行推测解码加速LLM推理", 技术原理和实现方式 steps 3-4:
 *     the target scores all proposed tokens at once; drafts are accepted while
 *     they agree with the target and the sequence is cut at the first
 *     rejection.
 *   - "vLLM EAGLE 投机解码实战：EAGLE/EAGLE3 草稿模型配置、源码实现与接受率评测",
 *     无损性保障: greedy speculative decoding yields exactly the greedy tokens.
 *
 * Conventions shared by every call
 *   - B sequences, N tree nodes per sequence (node 0 is the root, the last
 *     verified token; 1 <= N <= TV_MAX_NODES), Hq query heads, Hkv KV heads
 *     (Hq % Hkv == 0, query head h reads KV head h / (Hq/Hkv)), head dim D,
 *     vocab V.  W = ceil(N / 64) mask words per node.
 *   - parents[b][0] == -1 and 0 <= parents[b][i] < i for i >= 1.
 *   - Paged K/V cache: k_cache and v_cache are [num_blocks][Hkv][block_size][D]
 *     row-major by default (head-major: within a block, the block_size slots
 *     of KV head 0, then of head 1, ...: one head's keys of a block are one
 *     contiguous run), or [num_blocks][block_size][Hkv][D] (token-major: a
 *     slot's Hkv heads together) when the calls that take a cache get
 *     TV_KV_TOKEN_MAJOR OR'd into their dtype argument.  Both hold the same
 *     rows; head-major lets one copy instruction fetch a head's keys in one
 *     contiguous run.  Logical position t of sequence b lives in block
 *     block_table[b][t / block_size], slot t % block_size.  Sequence b's prefix
 *     is t in [0, prefix_lens[b]); tree node i's key/value sit at
 *     t = prefix_lens[b] + i and must be written before tv_tree_attention.
 *   - All pointers are DEVICE pointers to caller-owned memory; the library
 *     allocates nothing and keeps no global mutable state, except the static
 *     scratch buffer of tv_accept_greedy_noalloc (and the per-device address
 *     of it, looked up once).  Integers are int32 row-major.
 *   - Every call checks its scalar arguments on the host, returns a status
 *     and, on TV_OK, has enqueued its kernels on `stream` (asynchronous; no
 *     host synchronisation).  On any error other than TV_ERR_LAUNCH nothing is
 *     launched.
 *   - dev_status (optional, may be NULL): device int32 that the kernels OR
 *     status bits into for malformed data that only the device can see
 *     (TV_DEV_*).  The caller zeroes it; bits accumulate across calls.  A
 *     sequence that raises a bit gets unspecified (but in-bounds) outputs.
 */
#ifndef TV_H
#define TV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TV_MAX_NODES 256

/* exported symbols of libtv.so */
#define TV_API __attribute__((visibility("default")))

typedef enum {
  TV_OK = 0,
  TV_ERR_NULL = 1,        /* a required pointer is NULL */
  TV_ERR_SHAPE = 2,       /* a size <= 0, Hq % Hkv != 0, N > TV_MAX_NODES, or the
                             block table cannot hold max_prefix_len + N positions */
  TV_ERR_DTYPE = 3,       /* dtype (without TV_KV_TOKEN_MAJOR) is neither TV_F32 nor
                             TV_BF16, or the flag is given to a call without a cache */
  TV_ERR_UNSUPPORTED = 4, /* D not in {64, 128}, block_size != 16, or H % 64 != 0 */
  TV_ERR_ALIGN = 5,       /* q, out, cache, logits or workspace pointer not 16-byte aligned */
  TV_ERR_WORKSPACE = 6,   /* workspace missing or smaller than the queried size */
  TV_ERR_LAUNCH = 7,      /* the HIP runtime reported an error at launch */
  TV_ERR_TOO_LARGE = 8    /* the sizes need more scratch than
                             TV_ACCEPT_NOALLOC_SCRATCH_BYTES (allocation-free
                             variant only) */
} tv_status;

typedef enum { TV_F32 = 0, TV_BF16 = 1 } tv_dtype;

/* Cache-layout flag for the dtype argument of tv_tree_attention (and
 * tv_tree_attention_parents), tv_kv_compact, tv_accept_greedy_compact and
 * tv_tree_kv_write: the caches are token-major
 * [num_blocks][block_size][Hkv][D] instead of head-major
 * [num_blocks][Hkv][block_size][D].  Pass (tv_dtype)(TV_BF16 | TV_KV_TOKEN_MAJOR). */
#define TV_KV_TOKEN_MAJOR 0x100

/* device status bits */
#define TV_DEV_BAD_TREE 1   /* parents[b][0] != -1 or parents[b][i] not in [0, i) */
#define TV_DEV_BAD_CACHE 2  /* a used block id outside [0, num_blocks), or a prefix
                               length outside [0, max_prefix_len] */
#define TV_DEV_BAD_TOKEN 4  /* draft_tokens[b][i] (i >= 1) outside [0, V) */
#define TV_DEV_BAD_RANDOM 8 /* a uniform (i >= 1) outside [0, 1) or an exponential
                               variate of the drawn row outside (0, inf) */
#define TV_DEV_UNSUPPORTED 16 /* proposal rows given for a tree that is not a
                                 chain (parents[b][i] != i - 1) */

/* Name of a status code (static string). */
TV_API const char* tv_status_string(tv_status s);

/* Library version: major * 10000 + minor * 100 + patch. */
TV_API int tv_version(void);

/*
 * tv_build_tree_mask -- ancestor-or-self bitmask and depth of every node.
 * ("vLLM-TreeEagle" README, 核心组件 item 1: the tree attention mask is built
 * dynamically; 技术创新点 1: any tree shape.)
 *
 *   parents  [B][N] int32, device.
 *   mask     [B][N][W] uint64, device, written: bit (j % 64) of word j / 64 of
 *            mask[b][i] is set iff node j is node i or one of its ancestors.
 *   depth    [B][N] int32, device, written (may be NULL): edges from the root.
 *   Errors: TV_ERR_NULL, TV_ERR_SHAPE.  A sequence whose parent array is not
 *   a tree sets TV_DEV_BAD_TREE and gets an all-zero mask and zero depths.
 */
TV_API tv_status tv_build_tree_mask(const int32_t* parents, int32_t B, int32_t N, uint64_t* mask,
                             int32_t* depth, int32_t* dev_status, hipStream_t stream);

/*
 * Workspace bytes tv_tree_attention needs for these sizes, either dtype and
 * either cache layout (the fp32 path uses none).  The workspace holds
 * arrival counters (its first 2048 bytes, the same for every shape) and the
 * partial softmax state of every piece of a split key range (row maxima and
 * sums in fp32, the normalised partial outputs in bf16).  The workgroup that
 * finishes the last piece of a split sequence merges it, found through the
 * counters.  A new workspace must therefore be zero-filled once before its
 * first call (hipMemset, or a zeroed allocation).  Every call leaves the
 * counters at zero again, so the workspace then serves any number of later
 * calls of any shape without clearing.  Calls that share a workspace must be
 * ordered (same stream), and so must a call and any other use of its
 * workspace memory.
 */
TV_API size_t tv_tree_attention_workspace_size(int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                        int32_t max_prefix_len);

/*
 * tv_tree_attention -- tree-masked attention of every draft node over the
 * paged prefix and its own ancestors, in one pass.
 * ("vLLM-TreeEagle" README, 核心组件 item 1 and 技术创新点 1; "EAGLE代码实现原理",
 * 树结构缓冲: each prefix K/V tile is read once and serves every node and every
 * query head of its KV head; "P-EAGLE", 技术原理和实现方式 step 3.)
 *
 * For sequence b, node i, query head h, KV head kh = h / (Hq/Hkv), the visible
 * keys are prefix positions [0, P_b) and tree positions P_b + j for every j
 * whose bit is set in mask[b][i]:
 *   out[b][i][h] = sum_t softmax_t(scale * <q[b][i][h], k[t][kh]>) * v[t][kh].
 *
 *   q            [B][N][Hq][D], dtype, device, 16-byte aligned.
 *   k_cache, v_cache  [num_blocks][Hkv][block_size][D] (or token-major, see
 *                TV_KV_TOKEN_MAJOR), dtype, device, 16-byte aligned; read only.
 *   block_table  [B][max_blocks] int32, device.
 *   prefix_lens  [B] int32, device; every entry <= max_prefix_len (host int).
 *   mask         [B][N][W] uint64, device (as written by tv_build_tree_mask).
 *   out          [B][N][Hq][D], dtype, device, 16-byte aligned, written.
 *   scale        softmax scale; <= 0 selects 1/sqrt(D).
 *   dtype        TV_BF16 (fp32 accumulation, bf16 output rounded to nearest
 *                even) or TV_F32 (fp32 throughout), optionally OR'd with
 *                TV_KV_TOKEN_MAJOR.
 *   workspace    device buffer of at least
 *                tv_tree_attention_workspace_size(...) bytes, 16-byte aligned,
 *                zero-filled before its first use (see above); may be NULL
 *                for the fp32 path.
 * Errors: TV_ERR_NULL, TV_ERR_SHAPE, TV_ERR_DTYPE, TV_ERR_UNSUPPORTED,
 * TV_ERR_ALIGN, TV_ERR_WORKSPACE, TV_ERR_LAUNCH.  Device: TV_DEV_BAD_CACHE.
 */
TV_API tv_status tv_tree_attention(const void* q, const void* k_cache, const void* v_cache,
                            int32_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                            int32_t block_size, const int32_t* prefix_lens, int32_t max_prefix_len,
                            const uint64_t* mask, void* out, int32_t B, int32_t N, int32_t Hq,
                            int32_t Hkv, int32_t D, float scale, tv_dtype dtype, void* workspace,
                            size_t workspace_bytes, int32_t* dev_status, hipStream_t stream);

/*
 * tv_tree_attention_parents -- tv_tree_attention with the tree given as its
 * parent array instead of the masks: each wave of the attention kernels
 * builds the ancestor-or-self masks of the tree's nodes itself, while its
 * first K/V tiles are in flight, so a step needs no tv_build_tree_mask
 * launch before attention.  ("vLLM-TreeEagle" README, 核心组件 item 1 and
 * 技术创新点 1: one pass under a mask built at run time for any tree.)
 *
 *   parents  [B][N] int32, device, as for tv_build_tree_mask; N <= 64.
 *   Every other argument, the output and the workspace are tv_tree_attention's;
 *   the output is bit-identical to tv_build_tree_mask followed by
 *   tv_tree_attention.
 * Errors: those of tv_tree_attention, and TV_ERR_UNSUPPORTED for N > 64.
 * Device: TV_DEV_BAD_CACHE as tv_tree_attention; TV_DEV_BAD_TREE for a
 * parent array that is not a tree (the sequence is then attended with no
 * tree key visible, as with the mask tv_build_tree_mask leaves it).
 */
TV_API tv_status tv_tree_attention_parents(const void* q, const void* k_cache, const void* v_cache,
                                           int32_t num_blocks, const int32_t* block_table, int32_t max_blocks,
                                           int32_t block_size, const int32_t* prefix_lens,
                                           int32_t max_prefix_len, const int32_t* parents, void* out, int32_t B,
                                           int32_t N, int32_t Hq, int32_t Hkv, int32_t D, float scale,
                                           tv_dtype dtype, void* workspace, size_t workspace_bytes,
                                           int32_t* dev_status, hipStream_t stream);

/*
 * Workspace bytes tv_accept_greedy needs (per-chunk partial maxima).  The
 * workspace needs no initialisation; calls that share one workspace must be
 * ordered (same stream).
 */
TV_API size_t tv_accept_greedy_workspace_size(int32_t B, int32_t N, int32_t V);

/*
 * tv_accept_greedy -- target argmax of every tree node and the longest
 * accepted path.
 * ("P-EAGLE", 技术原理和实现方式 steps 3-4; "vLLM EAGLE 投机解码实战", 无损性保障.)
 *
 * am[b][i] = lowest v with logits[b][i][v] == max_u logits[b][i][u] (-0.0 and
 * +0.0 compare equal; NaN rows are unspecified).  An edge parent(c) -> c is
 * accepted iff draft_tokens[b][c] == am[b][parent(c)].  The accepted path is
 * the longest root-started path of accepted edges, the smallest node-index
 * sequence among equally long ones.
 *
 *   logits          [B][N][V] fp32, device, 16-byte aligned; row i holds the
 *                   target's next-token scores after node i.
 *   draft_tokens    [B][N] int32, device (entry 0, the root, is not compared).
 *   parents         [B][N] int32, device.
 *   accept_len      [B] int32, written: accepted draft tokens (root and bonus
 *                   excluded).
 *   accepted_nodes  [B][N] int32, written: the path from the root (node 0
 *                   first), padded with -1.
 *   bonus_token     [B] int32, written: am at the path's last node.
 *   target_argmax   [B][N] int32, written (may be NULL): am.
 * Errors: TV_ERR_NULL, TV_ERR_SHAPE, TV_ERR_ALIGN, TV_ERR_WORKSPACE,
 * TV_ERR_LAUNCH.  Device: TV_DEV_BAD_TREE, TV_DEV_BAD_TOKEN (the sequence then
 * reports accept_len 0, path [0] and bonus am[b][0]).
 */
TV_API tv_status tv_accept_greedy(const float* logits, const int32_t* draft_tokens, const int32_t* parents,
                           int32_t B, int32_t N, int32_t V, int32_t* accept_len,
                           int32_t* accepted_nodes, int32_t* bonus_token, int32_t* target_argmax,
                           void* workspace, size_t workspace_bytes, int32_t* dev_status,
                           hipStream_t stream);

/* Scratch bytes the library holds, per GPU, for tv_accept_greedy_noalloc. */
#define TV_ACCEPT_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)

/*
 * tv_accept_greedy_noalloc -- tv_accept_greedy for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same computation, arguments and
 * outputs, without the workspace argument.  Its per-chunk keys live in a
 * static scratch buffer of TV_ACCEPT_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends (its device address
 * is looked up on the first call for a device; nothing is allocated by any
 * call).  The outputs are bit-identical to tv_accept_greedy's.
 *
 *   stream  selects the GPU (the scratch of that stream's device is used).
 * Calls whose sizes need more than the buffer holds
 * (tv_accept_greedy_workspace_size(B, N, V) > TV_ACCEPT_NOALLOC_SCRATCH_BYTES,
 * i.e. more than 524288 chunk keys: about half a million rows of logits) are
 * refused with TV_ERR_TOO_LARGE.  Every call on one GPU shares that GPU's
 * buffer: calls that may overlap on one GPU (different streams, or different
 * host threads) race on it and must be ordered by the caller; calls on one
 * stream are ordered already.
 * Errors: TV_ERR_NULL, TV_ERR_SHAPE, TV_ERR_ALIGN, TV_ERR_TOO_LARGE,
 * TV_ERR_LAUNCH (also when the buffer's address cannot be looked up).
 * Device: as tv_accept_greedy.
 */
TV_API tv_status tv_accept_greedy_noalloc(const float* logits, const int32_t* draft_tokens,
                                          const int32_t* parents, int32_t B, int32_t N, int32_t V,
                                          int32_t* accept_len, int32_t* accepted_nodes,
                                          int32_t* bonus_token, int32_t* target_argmax,
                                          int32_t* dev_status, hipStream_t stream);

/*
 * Workspace bytes tv_accept_stochastic needs (per-chunk row statistics, one
 * stop record per sequence, per-chunk draw keys); 0 for invalid sizes.  The
 * workspace needs no initialisation; calls that share one must be ordered.
 */
TV_API size_t tv_accept_stochastic_workspace_size(int32_t B, int32_t N, int32_t V);

/*
 * tv_accept_stochastic -- stochastic verification of the draft tree at
 * temperature > 0: accepted path and bonus token.
 * ("P-EAGLE", 技术原理和实现方式 steps 3-4: target and draft probabilities of
 * the proposed tokens are compared, a sampling rule accepts, the sequence is
 * cut at the first rejection; "vLLM EAGLE 投机解码实战", 无损性保障: the
 * rejection sampler keeps the target distribution.)
 *
 * p_i = softmax(logits[b][i] / temperature).  From node u = 0 with r = p_u,
 * the children c of u are tested in increasing index: with x =
 * draft_tokens[b][c] and q_c its proposal (draft_probs[b][c], or the point
 * mass on x when draft_probs is NULL), c is accepted iff
 * uniforms[b][c] * q_c(x) < r(x), and the walk continues at c; a rejection
 * replaces r by max(r - q_c, 0) normalised (kept as is if that has no mass).
 * When every child of u is rejected, or u is a leaf, the bonus token is the
 * v with the largest r(v) / exponentials[b][v] (lowest v among equals).
 * Decisions are taken in fp32 (row sums in a chunked order): a decision
 * within about 1e-5 relative of its threshold may go either way.
 *
 *   logits          [B][N][V] fp32, device, 16-byte aligned; row i holds the
 *                   target's next-token scores after node i.
 *   draft_probs     [B][N][V] fp32, device, 16-byte aligned, or NULL; row c is
 *                   the distribution node c's token was drawn from (row 0
 *                   unused).  Only chains (parents[b][i] == i - 1) are taken
 *                   with it; another tree sets TV_DEV_UNSUPPORTED.
 *   draft_tokens    [B][N] int32, device (entry 0 unused).
 *   parents         [B][N] int32, device.
 *   uniforms        [B][N] fp32, device, in [0, 1) (entry 0 unused).
 *   exponentials    [B][V] fp32, device, Exp(1) variates, in (0, inf).
 *   temperature     > 0 and finite.
 *   accept_len      [B] int32, written: accepted draft tokens.
 *   accepted_nodes  [B][N] int32, written: the path from the root, -1 padded.
 *   bonus_token     [B] int32, written.
 * Errors: TV_ERR_NULL, TV_ERR_SHAPE (also a temperature that is not > 0 and
 * finite), TV_ERR_ALIGN, TV_ERR_WORKSPACE, TV_ERR_LAUNCH.  Device:
 * TV_DEV_BAD_TREE, TV_DEV_BAD_TOKEN, TV_DEV_UNSUPPORTED (the sequence then
 * reports accept_len 0, path [0] and a bonus drawn from p_0), TV_DEV_BAD_RANDOM
 * (results unspecified).
 */
TV_API tv_status tv_accept_stochastic(const float* logits, const float* draft_probs,
                               const int32_t* draft_tokens, const int32_t* parents,
                               const float* uniforms, const float* exponentials, int32_t B,
                               int32_t N, int32_t V, float temperature, int32_t* accept_len,
                               int32_t* accepted_nodes, int32_t* bonus_token, void* workspace,
                               size_t workspace_bytes, int32_t* dev_status, hipStream_t stream);

/*
 * Workspace bytes tv_lm_head_argmax needs (one 64-bit key per row and
 * 256-wide vocabulary tile); 0 for invalid sizes.  No initialisation needed.
 */
TV_API size_t tv_lm_head_argmax_workspace_size(int32_t M, int32_t H, int32_t V);

/*
 * tv_lm_head_argmax -- the target's LM head fused with the greedy choice:
 * per row, the best-scoring vocabulary entry and its score, without
 * writing the [M][V] scores.
 * ("P-EAGLE", 技术原理和实现方式 step 3: one target pass scores every
 * proposed token; "vLLM EAGLE 投机解码实战", 无损性保障: greedy verification
 * compares drafts with the target's greedy choice.)
 *
 * score[m][v] = sum_h hidden[m][h] * weight[v][h] (bf16 products, fp32
 * accumulation); argmax[m] = lowest v among the row's maxima (-0.0 and
 * +0.0 compare equal; NaN rows unspecified).  The scores differ from exact
 * ones by fp32 rounding, so two entries within that rounding of each other
 * may swap.  With rows = B * N tree nodes, argmax is the target_argmax a
 * greedy walk needs.
 *
 *   hidden      [M][H] bf16, device, 16-byte aligned: final hidden states.
 *   weight      [V][H] bf16, device, 16-byte aligned: LM-head rows.
 *   H           a multiple of 64, at most 2^20.
 *   argmax      [M] int32, device, written.
 *   max_score   [M] fp32, device, written (may be NULL).
 *   workspace   device buffer of tv_lm_head_argmax_workspace_size(M, H, V)
 *               bytes, 16-byte aligned.
 * Errors: TV_ERR_NULL, TV_ERR_DTYPE (only TV_BF16), TV_ERR_SHAPE,
 * TV_ERR_UNSUPPORTED (H % 64 != 0), TV_ERR_ALIGN, TV_ERR_WORKSPACE,
 * TV_ERR_LAUNCH.
 */
TV_API tv_status tv_lm_head_argmax(const void* hidden, const void* weight, int32_t M, int32_t H,
                            int32_t V, tv_dtype dtype, int32_t* argmax, float* max_score,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * tv_kv_compact -- move the accepted path's K/V rows into the contiguous
 * positions right after the prefix, in place.
 * ("EAGLE代码实现原理", KV缓存优化: copy(indices, prev_length) selects the
 * indexed rows and then copies them to the rows starting at prev_length;
 * "P-EAGLE", 技术难点和解决方案: the cache is rolled back to the accepted
 * tokens.)
 *
 * With L = accept_len[b] + 1 and path = accepted_nodes[b][0 .. L-1], the rows
 * at logical positions P_b + path[j] are gathered and written to positions
 * P_b + j (j < L), for every KV head, in both caches, with the result of
 * gathering all sources before writing any destination.  All other rows keep
 * their bytes.  The path must be strictly increasing and start at node 0 (as
 * tv_accept_greedy writes it).
 *
 *   k_cache, v_cache  [num_blocks][Hkv][block_size][D] (or token-major with
 *                     TV_KV_TOKEN_MAJOR in dtype), dtype, device, 16-byte
 *                     aligned, updated in place.
 *   new_lens          [B] int32, written (may be NULL): P_b + L.
 * Errors: TV_ERR_NULL, TV_ERR_SHAPE, TV_ERR_DTYPE, TV_ERR_UNSUPPORTED,
 * TV_ERR_ALIGN, TV_ERR_LAUNCH.  Device: TV_DEV_BAD_CACHE (block id out of
 * range), TV_DEV_BAD_TREE (a path that is not strictly increasing from node 0
 * or an accept_len outside [0, N-1]); the sequence is then left untouched.
 */
TV_API tv_status tv_kv_compact(void* k_cache, void* v_cache, int32_t num_blocks, const int32_t* block_table,
                        int32_t max_blocks, int32_t block_size, const int32_t* prefix_lens,
                        const int32_t* accepted_nodes, const int32_t* accept_len, int32_t B,
                        int32_t N, int32_t Hkv, int32_t D, tv_dtype dtype, int32_t* new_lens,
                        int32_t* dev_status, hipStream_t stream);

/*
 * tv_accept_greedy_compact -- tv_accept_greedy followed by tv_kv_compact of
 * its accepted paths, in one call: the workgroup that walks a sequence also
 * moves that sequence's accepted K/V rows, so the step needs one launch
 * fewer.  ("P-EAGLE", 技术原理和实现方式 steps 3-4 and 技术难点和解决方案;
 * "EAGLE代码实现原理", KV缓存优化: copy(indices, prev_length).)
 *
 * Outputs, caches and new_lens are exactly those of tv_accept_greedy and
 * then tv_kv_compact(accepted_nodes, accept_len) on the same arguments: the
 * same bytes, the same device status bits.  Arguments are those of the two
 * calls (workspace: tv_accept_greedy_workspace_size(B, N, V) bytes; dtype
 * and the cache layout flag as for tv_kv_compact).
 * Errors: the union of both calls' host errors.
 */
TV_API tv_status tv_accept_greedy_compact(const float* logits, const int32_t* draft_tokens,
                                          const int32_t* parents, int32_t B, int32_t N, int32_t V,
                                          int32_t* accept_len, int32_t* accepted_nodes, int32_t* bonus_token,
                                          int32_t* target_argmax, void* workspace, size_t workspace_bytes,
                                          void* k_cache, void* v_cache, int32_t num_blocks,
                                          const int32_t* block_table, int32_t max_blocks, int32_t block_size,
                                          const int32_t* prefix_lens, int32_t Hkv, int32_t D, tv_dtype dtype,
                                          int32_t* new_lens, int32_t* dev_status, hipStream_t stream);

/*
 * tv_tree_kv_write -- rotate the step's queries and new keys to their tree
 * positions and append the new K/V rows to the paged cache, before
 * tv_tree_attention.  ("EAGLE代码实现原理", KV缓存优化: cat() appends the new
 * rows after the current length inside the preallocated cache; "P-EAGLE",
 * 技术难点和解决方案: the block manager appends the proposed tokens.  The pages
 * leave the positional encoding open: this is the rotary embedding of the
 * Llama-family targets, at tree positions.)
 *
 * Node i of sequence b takes rotary position pos = P_b + depth[b][i]
 * (siblings share a position; a root-to-leaf path has consecutive ones).
 * Every pair (x[j], x[j + D/2]), j < D/2, of each query head and each new key
 * head turns by the angle pos * rope_theta^(-2j/D):
 *   x'[j] = x[j] cos - x[j + D/2] sin,  x'[j + D/2] = x[j + D/2] cos + x[j] sin
 * (angles formed in fp64, rotation in fp32, bf16 results rounded to nearest
 * even).  The rotated key and the unchanged value of node i are written at
 * logical position P_b + i of the paged cache; no other row changes.
 *
 *   q             [B][N][Hq][D], dtype, device, 16-byte aligned, read.
 *   k_new, v_new  [B][N][Hkv][D], dtype, device, 16-byte aligned, read.
 *   depth         [B][N] int32, device (as written by tv_build_tree_mask).
 *   q_out         [B][N][Hq][D], dtype, device, 16-byte aligned, written;
 *                 may be q itself (in place).
 *   k_cache, v_cache, block_table, prefix_lens: as for tv_tree_attention;
 *                 the caches are updated in place.
 *   dtype         TV_BF16 or TV_F32, optionally OR'd with TV_KV_TOKEN_MAJOR.
 *   rope_theta    rotary base (> 0), e.g. 500000 for Llama 3.
 * Errors: TV_ERR_NULL, TV_ERR_SHAPE (also rope_theta <= 0), TV_ERR_DTYPE,
 * TV_ERR_UNSUPPORTED, TV_ERR_ALIGN, TV_ERR_LAUNCH.  Device: TV_DEV_BAD_TREE
 * (a depth outside [0, N): position P_b is used), TV_DEV_BAD_CACHE (the slot
 * of P_b + i lies outside the table or names a block outside the cache: that
 * node's rows are not written).
 */
TV_API tv_status tv_tree_kv_write(const void* q, const void* k_new, const void* v_new, const int32_t* depth,
                           void* q_out, void* k_cache, void* v_cache, int32_t num_blocks,
                           const int32_t* block_table, int32_t max_blocks, int32_t block_size,
                           const int32_t* prefix_lens, int32_t B, int32_t N, int32_t Hq, int32_t Hkv,
                           int32_t D, float rope_theta, tv_dtype dtype, int32_t* dev_status,
                           hipStream_t stream);

/* limits of tv_build_draft_tree */
#define TV_DRAFT_MAX_DEPTH 16
#define TV_DRAFT_MAX_TOPK 16
#define TV_DRAFT_MAX_VOCAB 262144

/*
 * Workspace bytes tv_build_draft_tree needs (per row chunk: its maximum, its
 * sum of exponentials and its topk best entries); 0 for invalid sizes.  No
 * initialisation needed; calls that share one must be ordered.
 */
TV_API size_t tv_build_draft_tree_workspace_size(int32_t B, int32_t depth, int32_t topk, int32_t V);

/*
 * tv_build_draft_tree -- the draft token tree of N nodes, grown level by
 * level from the drafter's scores: top-k expansion and a global rerank by
 * cumulative log-probability.
 * ("EAGLE代码实现原理", 树结构缓冲: branch prediction proposes likely
 * continuations ahead, level pruning keeps the high-probability paths and
 * cuts the low-probability branches; "vLLM-TreeEagle" README, 核心组件
 * item 3: multi-level candidate generation with path pruning.)
 *
 * A node's score is the sum of the log-probabilities (log softmax of the
 * row it was proposed from) of the tokens on its path; the root's is 0.
 * Level 0: the root proposes the topk most probable tokens of row (0, 0).
 * Level l >= 1: the j-th best candidate of level l - 1 (by score, then
 * generation order) proposes the topk most probable tokens of row (l, j),
 * giving candidates in order (j, rank); within a row, more probable first
 * and the lower token id among equals.  Every candidate of every level is a
 * generated node; the tree is the root plus the N - 1 best generated nodes
 * (score, then level, then generation order), which is ancestor-closed.
 * Nodes are numbered level by level and by that order within a level, so
 * parents[b][i] < i and the output feeds tv_build_tree_mask directly.
 * Scores are computed in fp32 (row log-sum-exp in a chunked order): two
 * candidates whose scores lie within about 1e-5 of each other may swap.
 *
 *   draft_logits  [B][depth][topk][V] fp32, device, 16-byte aligned, finite:
 *                 row (l, j) holds the drafter's next-token scores at the
 *                 j-th best node of level l - 1 (row (0, 0): at the root;
 *                 rows (0, j >= 1) are not read).
 *   depth         1 .. TV_DRAFT_MAX_DEPTH levels of expansion.
 *   topk          1 .. TV_DRAFT_MAX_TOPK, at most V.
 *   V             at most TV_DRAFT_MAX_VOCAB.
 *   N             1 .. TV_MAX_NODES, with N - 1 <= topk + (depth - 1) * topk^2
 *                 (the number of generated nodes).
 *   root_tokens   [B] int32, device, or NULL (then 0): token of node 0.
 *   parents       [B][N] int32, device, written: parents[b][0] = -1.
 *   tokens        [B][N] int32, device, written: draft token of each node.
 *   scores        [B][N] fp32, device, written (may be NULL): node scores.
 *   workspace     device buffer of tv_build_draft_tree_workspace_size(B,
 *                 depth, topk, V) bytes, 16-byte aligned.
 * Errors: TV_ERR_NULL, TV_ERR_SHAPE, TV_ERR_ALIGN, TV_ERR_WORKSPACE,
 * TV_ERR_LAUNCH.
 */
TV_API tv_status tv_build_draft_tree(const float* draft_logits, int32_t B, int32_t depth, int32_t topk,
                              int32_t V, int32_t N, const int32_t* root_tokens, int32_t* parents,
                              int32_t* tokens, float* scores, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TV_H */
