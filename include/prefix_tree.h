/*
 * prefix_tree.h -- host-side prefix cache for the dual-pool KV cache: a radix
 * tree over token ids whose nodes carry both a Full-pool page index and an
 * SWA segment map, matched under the window-safe rule.
 *
 * The method (web pages cited by title and section):
 *   [YLY]  youleyou.com "小米MiMo首次公开模型推理系统全链路优化降价99%",
 *          section 2 sub-section "KVCache系统重构：让缓存真正省下来": with
 *          sliding-window layers, equal token prefixes no longer imply that
 *          the KV is still there -- a node's SWA KV may survive only as a
 *          tail, or not at all -- so the prefix tree changes in three ways:
 *          the match is cut to the window-safe length; SWA eviction follows
 *          the request's lifecycle, so SWA occupancy stays at window scale;
 *          each node holds a Full segment index and an SWA segment map that
 *          are evicted independently.
 *   [HD9]  blog.hotdry.top 2026-06-09, section "Hybrid SWA：用 1/7 计算量捕获
 *          长程依赖": nodes record the Full index and the SWA window map, and
 *          the match length is clipped to the window.
 *   [HTX]  htx.com news, section 工程三 (window-safe prefix reuse).
 *
 * Model. A request's sequence of token ids is cached as a path from the root.
 * Position p of a cached path has
 *   - a Full page: page index p / page_size of the path holds a page id of the
 *     Full pool (the tree references pages; a page id is owned by the tree
 *     while any node references it);
 *   - an SWA source: the id of a ring (the per-request SWA buffer of W slots,
 *     slot p mod W) that still holds position p, or none.
 * A ring holds positions [len - W, len) of its request, where len is the
 * request's current length, so at most W positions of the tree name one ring
 * (SWA occupancy is O(W) per ring). A ring is either live (its request runs:
 * ha_tree_ring_advance moves its window, ha_tree_ring_release ends it) or
 * owned by the tree (handed over on insert; freed by the tree's SWA eviction
 * or when no position names it any more).
 *
 * Window-safe reuse. ha_tree_match returns, for a request, the longest common
 * prefix m with the cached paths and the SWA validity of each position in
 * [0, m) -- exactly the swa_valid map window_safe_match (hybrid_attn.h)
 * consumes, with the matched tokens as cached_tokens. The reusable length L
 * it returns needs only positions [0, L) of the Full pool (pages [0, L/16],
 * the last one partly) and positions [L - W, L) of the SWA pool.
 *
 * Pages split by a request. Paths are token-granular: a node may start in the
 * middle of a page. Then the page index that straddles the node's start holds
 * a different page id in the node than in its parent; both hold identical KV
 * for the positions before the node's start. A request reusing L positions
 * with L % page_size != 0 must therefore write its own tokens into a copy of
 * the page it borrows for index L / page_size (copy on write), never into the
 * tree's page.
 *
 * Eviction. ha_tree_evict_full frees whole leaves, least recently used first,
 * skipping locked nodes (ha_tree_lock), and returns the page ids whose last
 * reference went away, plus tree-owned rings no position names any more.
 * ha_tree_evict_swa frees tree-owned rings, least recently used first; their
 * positions become invalid while their Full pages stay matchable.
 *
 * Threading and ownership. A tree is a host object; calls on one tree must
 * not overlap. Every array argument is host memory owned by the caller; the
 * tree copies what it keeps. No call touches the GPU.
 *
 * Errors. Every call returns ha_status (hybrid_attn.h). On an error nothing
 * changes and ha_last_error() describes it.
 */
#ifndef PREFIX_TREE_H
#define PREFIX_TREE_H

#include <stdint.h>

#include "hybrid_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ha_prefix_tree ha_prefix_tree;

/* A new, empty tree. window >= 1 (W of the SWA layers), page_size >= 1. */
ha_status ha_tree_create(int32_t window, int32_t page_size, ha_prefix_tree** out_tree);

/* Frees the tree (pages and rings it references are not returned: the
 * caller's pools are released with it). NULL is allowed. */
void ha_tree_destroy(ha_prefix_tree* tree);

/* Caches tokens [0, n) of a request.
 *   pages [ceil(n / page_size)]: the request's Full page ids, page index i
 *     holding positions [i * page_size, (i + 1) * page_size); ids >= 0.
 *   ring_id >= 0 with ring_len >= 0: the request's ring holds positions
 *     [max(0, ring_len - W), ring_len); those below n are recorded as held
 *     by it. ring_id = -1 records no SWA positions.
 *   transfer_ring != 0: the tree takes over the ring (the request ends);
 *     otherwise the ring stays live.
 *   page_kept [ceil(n / page_size)] (out, may be NULL): 1 where the tree now
 *     references pages[i] -- either it was already the tree's page, or it
 *     holds positions the tree did not have -- else 0, and the caller may
 *     free that page.
 *   ring_kept (out, may be NULL): 1 if the tree now names the ring for some
 *     position (and, with transfer_ring, owns it), else 0: the tree holds no
 *     position of it and the caller keeps (or frees) the ring.
 * The positions already cached keep their pages; positions past the longest
 * cached prefix are added as a new leaf with the caller's pages, which must
 * not be pages the tree references (a page holding new positions is the
 * request's own: a borrowed page is copied before the request writes to it).
 * A ring that already held positions keeps only its window at ring_len. A
 * position keeps its existing source ring unless that ring is live and this
 * one is handed over. */
ha_status ha_tree_insert(ha_prefix_tree* tree, const int32_t* tokens, int64_t n, const int32_t* pages,
                         int32_t ring_id, int64_t ring_len, int32_t transfer_ring, uint8_t* page_kept,
                         int32_t* ring_kept);

/* Longest cached prefix of tokens [0, n) and its maps. Outputs (host):
 *   *out_matched = m;
 *   swa_valid [n]: 1 where position p < m is held by some ring, else 0;
 *   swa_ring [n] (may be NULL): that ring's id, else -1;
 *   pages [ceil(n / page_size)] (may be NULL): the page ids of page indices
 *     [0, ceil(m / page_size)) along the path (for a page index split by a
 *     node start, the page of the node that holds position
 *     min(m, (i + 1) * page_size) - 1), -1 beyond.
 * Marks the matched nodes and rings as used for LRU eviction. */
ha_status ha_tree_match(ha_prefix_tree* tree, const int32_t* tokens, int64_t n, int64_t* out_matched,
                        uint8_t* swa_valid, int32_t* swa_ring, int32_t* pages);

/* Adds delta (+1 or -1) to the lock count of the nodes holding positions
 * [0, n) of the path of tokens; n must not exceed the cached prefix. Locked
 * nodes are never evicted. Locking first splits a node that n ends inside,
 * so an unlock with the same tokens and n undoes it exactly. */
ha_status ha_tree_lock(ha_prefix_tree* tree, const int32_t* tokens, int64_t n, int32_t delta);

/* A live ring's request has grown to new_len tokens: positions below
 * new_len - W are no longer held by it. */
ha_status ha_tree_ring_advance(ha_prefix_tree* tree, int32_t ring_id, int64_t new_len);

/* A live ring is released (its request ended without handing it over): none
 * of its positions stays valid. Unknown ids are ignored. */
ha_status ha_tree_ring_release(ha_prefix_tree* tree, int32_t ring_id);

/* Evicts unlocked leaves, least recently used first, until at least
 * want_pages page ids have been freed or nothing is evictable. Freed page ids
 * go to freed_pages [page_cap], tree-owned rings left without positions to
 * freed_rings [ring_cap]; a leaf whose frees would not fit is not evicted. */
ha_status ha_tree_evict_full(ha_prefix_tree* tree, int64_t want_pages, int32_t* freed_pages, int64_t page_cap,
                             int64_t* out_pages, int32_t* freed_rings, int64_t ring_cap, int64_t* out_rings);

/* Frees up to want_rings tree-owned rings, least recently used first, into
 * freed_rings [ring_cap]. Their positions become invalid. */
ha_status ha_tree_evict_swa(ha_prefix_tree* tree, int64_t want_rings, int32_t* freed_rings, int64_t ring_cap,
                            int64_t* out_rings);

/* Counts: out[0] nodes (root excluded), out[1] distinct page ids referenced,
 * out[2] positions with an SWA source, out[3] tree-owned rings, out[4] live
 * rings with positions, out[5] the most positions held by one ring. */
ha_status ha_tree_stats(const ha_prefix_tree* tree, int64_t out[6]);

#ifdef __cplusplus
}
#endif

#endif /* PREFIX_TREE_H */
