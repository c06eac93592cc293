"""Single-pass verification of a draft token tree on AMD Instinct MI355X.

The calls of libtv (hand-written HIP kernels for gfx950) with the same
names as the C ABI in ``include/tv.h``:

* ``tv_build_tree_mask``  -- ancestor-or-self bitmask of every tree node
* ``tv_tree_attention``   -- tree-masked attention over the paged prefix
* ``tv_accept_greedy``    -- target argmax and the longest accepted path
* ``tv_accept_greedy_noalloc`` -- the same without a workspace, for callers
  that cannot allocate (a static per-GPU scratch buffer serves instead)
* ``tv_accept_stochastic`` -- accepted path and bonus token at temperature
  > 0 (speculative sampling over the tree, random numbers passed in)
* ``tv_kv_compact``       -- move the accepted path's K/V after the prefix
* ``tv_lm_head_argmax``   -- the target's LM head fused with the greedy
  choice (scores never written)
* ``tv_tree_kv_write``    -- rotate q and the new keys to their tree
  positions and append the new K/V rows (runs before ``tv_tree_attention``)
* ``tv_build_draft_tree`` -- grow the draft tree level by level from the
  drafter's scores (top-k expansion, global rerank by cumulative
  log-probability); its parents and tokens feed the calls above

Importing the package loads libtv.so and raises if it has not been built.
"""
from ._lib import (  # noqa: F401
    BLOCK_SIZE,
    TV_BF16,
    TV_DEV_BAD_CACHE,
    TV_DEV_BAD_RANDOM,
    TV_DEV_BAD_TOKEN,
    TV_DEV_BAD_TREE,
    TV_ACCEPT_NOALLOC_SCRATCH_BYTES,
    TV_DEV_UNSUPPORTED,
    TV_ERR_TOO_LARGE,
    TV_F32,
    TV_KV_TOKEN_MAJOR,
    TV_MAX_NODES,
    TVError,
    header_functions,
    lib,
    tv_accept_greedy,
    tv_accept_greedy_compact,
    tv_accept_greedy_noalloc,
    tv_accept_stochastic,
    tv_build_draft_tree,
    tv_build_tree_mask,
    tv_kv_compact,
    tv_lm_head_argmax,
    tv_tree_attention,
    tv_tree_attention_parents,
    tv_tree_attention_workspace_size,
    tv_tree_kv_write,
)
