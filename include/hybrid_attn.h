/*
 * hybrid_attn.h -- C ABI of the hybrid sliding-window / full GQA attention
 * library for AMD Instinct MI355X (gfx950).
 *
 * The method (web pages cited by title and section):
 *   [HTX]  htx.com news "Xiaomi MiMo's 99% price cut is not marketing -- Luo Fuli
 *          posts ...", sections 工程一 (60 of 70 layers use a 128-token window,
 *          10 attend to everything), 工程二 (two separate KV pools), 工程三
 *          (window-safe prefix reuse).
 *   [YLY]  youleyou.com "小米MiMo首次公开模型推理系统全链路优化降价99%",
 *          section 1 "为什么选择 Hybrid SWA 架构" and section 2 sub-section
 *          "KVCache系统重构：让缓存真正省下来" (Full pool grows on demand and is
 *          long-lived; SWA pool is a ring buffer sized by the window, O(W);
 *          the Full index is authoritative; window-safe length rule).
 *   [HD9]  blog.hotdry.top 2026-06-09 "MiMo-V2.5 ultra-speed inference
 *          architecture", sections "Hybrid SWA：用 1/7 计算量捕获长程依赖"
 *          (6:1 interleave, match clipped to the window boundary) and
 *          "PD 分离与长度分桶" (chunked prefill, 64K/256K/1M buckets).
 *   [HD12] blog.hotdry.top 2026-06-12 "MiMo inference optimization / edge
 *          deployment", section "双池分治与三级缓存的工程实现".
 *
 * Semantics. For query position t, query head h, kv head g = h / (Hq/Hkv):
 *   visible keys j: lo(t) <= j <= t, lo = max(0, t-W+1) for SWA layers,
 *   lo = 0 for full layers (W keys including the query itself);
 *   o = softmax_j(scale * q.k_j) v_j, lse = ln sum_j exp(scale * q.k_j).
 *
 * Ownership and threading. The caller owns every buffer (pools, tables, Q/K/V,
 * outputs, workspace). The library allocates no device memory, keeps no state
 * between calls apart from a thread-local error message, and is thread-safe.
 * (Exception: hybrid_attn_decode_noalloc uses one static device array per
 * device that the loader places with the library's code; see there.)
 * Device work is enqueued on the caller's HIP stream (passed as void*, NULL =
 * default stream) and the calls return without synchronising; only
 * window_safe_match runs synchronously on the host.
 *
 * Inputs. K/V values (in the pools and in a prefill chunk) must be finite for
 * the semantics above to hold exactly: prefill contracts V for all rows of a
 * 64-key tile at once, so a NaN/Inf V value of a key that some row masks out
 * still reaches that row (0 * NaN = NaN). Unwritten ring slots and page tails
 * are never read into a product.
 *
 * Errors. Every call returns ha_status. Arguments are validated on the host
 * before any HIP call, so a rejected call never touches the device.
 * ha_last_error() returns a message for the last failure on the calling
 * thread. Ring or page ids out of range (negative, or >= the view's
 * num_blocks) are not reported, and no memory outside the pools is touched:
 *   - a history block whose page-table entry is out of range holds no keys:
 *     decode, verify and prefill alike attend over the remaining positions,
 *     and the appends drop their writes to it;
 *   - a sequence whose ring id is out of range has no history keys (prefill
 *     and verify still see their new tokens; decode then has no key at all
 *     and returns O = 0, LSE = -inf, as for an empty row).
 *
 * Pool layouts (bfloat16, per layer). Both pools are made of blocks of 16
 * tokens x D channels (D = head_dim) of one kv head, 16*D values each:
 *   SWA ring pool, W slots per (ring, kv head), stored as ceil(W/16) blocks
 *   (the last block's slots past W are never written nor read as keys):
 *     K, V  [num_rings][Hkv][ceil(W/16)][16*D]  ring slot s in block s/16, token s%16
 *   Full page pool, page_size/16 blocks per (page, kv head) (PS = page_size,
 *   a power of two >= 16):
 *     K, V  [num_pages][Hkv][PS/16][16*D]  page token r in block r/16, token r%16
 *   Position p of a sequence lives in ring slot p mod W, or in page
 *   page_table[b][p / PS] at page token p mod PS.
 *   Inside a block, values sit in matrix-core operand order: 16-byte units,
 *   unit u = 64a + 16q + c (a < D/32, q < 4, c < 16):
 *     K unit u = K[token c][channels 32a + 8q .. 32a + 8q + 7]
 *     V unit u = V[tokens 4q..4q+3][channel 32a + c],
 *                then V[tokens 4q..4q+3][channel 32a + 16 + c]
 *   i.e. K(t, ch) is value ((ch/32)*64 + ((ch%32)/8)*16 + t)*8 + ch%8 and
 *   V(t, ch) is value ((ch/32)*64 + (t/4)*16 + ch%16)*8 + ((ch%32)/16)*4 + t%4.
 *   A wavefront then loads each operand set with fully contiguous 1 KiB reads.
 *
 * INT8 pools (kv_dtype = HA_KV_INT8; next to the bf16 format, for decode,
 * which is bound by the KV bytes it reads -- [HD12] "KV Cache 量化策略的技术
 * 选型" names low-bit KV storage). Same blocks, one signed byte per value,
 * 16*D bytes per (block, kv head), plus one float32 scale per (block, kv
 * head, token) for K and for V:
 *   code(t, ch) = clamp(rint(x / s), -127, 127), s = max_ch |x| / 127 over
 *   the token's D channels of that kv head (float32 arithmetic; s = 0 for an
 *   all-zero row), value = code * s; x is the bf16 value.
 *   K(t, ch) is byte ((ch/64)*64 + ((ch%32)/8)*16 + t)*16 + ((ch/32)%2)*8 + ch%8,
 *   V(t, ch) is byte ((ch/64)*64 + (t/4)*16 + ch%16)*16 + ((ch/16)%4)*4 + t%4,
 *   so a lane's K chunks of two 32-channel slices and its V values of four
 *   16-channel tiles are each one 16-byte load.
 *   Scales: k_scale / v_scale float32 [num_blocks][Hkv][PS/16][16] for pages
 *   and [rings][Hkv][ceil(W/16)][16] for rings, i.e. the scale of the value at element
 *   offset e of the codes is at e / (16*D) * 16 + token. */
#ifndef HYBRID_ATTN_H
#define HYBRID_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HA_ABI_VERSION 8

typedef enum ha_status {
  HA_OK = 0,
  HA_ERR_NULL = 1,        /* a required pointer is NULL                        */
  HA_ERR_SHAPE = 2,       /* unsupported geometry: Hq % Hkv != 0, group not in
                             {1,2,4,8,16}, head_dim not 64 or 128, window
                             outside [1, 2^24], page_size not a power of
                             two in [16, 2^20], or a non-finite
                             softmax_scale                                    */
  HA_ERR_RANGE = 3,       /* negative or inconsistent sizes, or a page-table
                             row (table_stride x page_size) of more than
                             2^31 tokens                                      */
  HA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required        */
  HA_ERR_UNSUPPORTED = 5, /* dtype or layer kind not supported                 */
  HA_ERR_HIP = 6          /* a HIP launch failed (message has the HIP error)   */
} ha_status;

typedef enum ha_dtype { HA_BF16 = 0, HA_F32 = 1 } ha_dtype;

typedef enum ha_layer_kind { HA_SWA = 0, HA_FULL = 1 } ha_layer_kind;

/* Element format of a pool. */
typedef enum ha_kv_dtype { HA_KV_BF16 = 0, HA_KV_INT8 = 1 } ha_kv_dtype;

/* Head geometry shared by every call of one layer stack, so the window used by
 * the kernels and by window_safe_match cannot drift apart ([HD12] notes that
 * changing W must change the window-safe rule with it).
 *   num_q_heads % num_kv_heads == 0, group = num_q_heads / num_kv_heads in
 *   {1, 2, 4, 8, 16}; head_dim in {64, 128}; 1 <= window <= 2^24;
 *   page_size a power of two in [16, 2^20] (tokens per Full page: pages of
 *   more than 16 tokens hold several 16-token blocks per kv head, which lets
 *   a caller's allocator hand out fewer, larger pages); softmax_scale <= 0
 *   selects 1/sqrt(head_dim). */
typedef struct ha_shape {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t window;
  int32_t page_size;
  float softmax_scale;
} ha_shape;

/* One layer's pool. kind selects the interpretation of table:
 *   HA_SWA : table = ring id per sequence, int32 [batch] (device);
 *            num_blocks = rings in the pool; table_stride ignored.
 *   HA_FULL: table = page table, int32 [batch][table_stride] (device);
 *            num_blocks = pages in the pool. The page table is the
 *            authoritative logical->physical index of the sequence ([YLY]).
 * kv_dtype selects bf16 pools (HA_KV_BF16, scales unused) or INT8 pools
 * (HA_KV_INT8: k_scale / v_scale required, layout above). INT8 pools are
 * written by the two append calls (and by the fused appends of
 * hybrid_attn_decode and hybrid_attn_verify, which quantize the new tokens
 * the same way) and read by hybrid_attn_decode and hybrid_attn_verify;
 * prefill and the pool reads reject them (HA_ERR_UNSUPPORTED). */
typedef struct ha_kv_view {
  int32_t kind;
  void* k;
  void* v;
  int32_t num_blocks;
  const int32_t* table;
  int32_t table_stride;
  int32_t kv_dtype;
  float* k_scale;
  float* v_scale;
} ha_kv_view;

/* ---- a1: SWA ring append ([YLY] KVCache系统重构; [HD12] 双池分治) ----------
 * Writes the new tokens of each sequence into its ring: token i of sequence b
 * (row cu_new[b] + i of k_new/v_new, absolute position pos0[b] + i) goes to
 * slot (pos0[b] + i) mod W of ring ring->table[b]. Only the last min(n_b, W)
 * tokens are written; the result equals appending all of them in order.
 *   ring      HA_SWA view
 *   pos0      int32 [batch] device, >= 0
 *   cu_new    int32 [batch+1] device, non-decreasing, cu_new[0] = 0,
 *             cu_new[batch] = num_tokens
 *   k_new, v_new  [num_tokens][Hkv][D] device, src_dtype (HA_F32 is rounded
 *             to bfloat16 to nearest-even) */
ha_status swa_ring_append(const ha_shape* shape, const ha_kv_view* ring, const int32_t* pos0,
                          const int32_t* cu_new, int32_t batch, int32_t num_tokens,
                          const void* k_new, const void* v_new, int32_t src_dtype, void* stream);

/* ---- a2: Full pool append ([YLY] KVCache系统重构: grows on demand) --------
 * Writes token i of sequence b (position p = pos0[b] + i) to page
 * pages->table[b][p / page_size], page token p mod page_size. The caller
 * allocates the pages (the pool grows by the caller handing out more page
 * ids). Arguments as for swa_ring_append; every page id used must be
 * < pages->num_blocks and p / page_size < table_stride. */
ha_status full_pool_append(const ha_shape* shape, const ha_kv_view* pages, const int32_t* pos0,
                           const int32_t* cu_new, int32_t batch, int32_t num_tokens,
                           const void* k_new, const void* v_new, int32_t src_dtype, void* stream);

/* ---- reading positions back out of a pool (the inverse of the appends) ----
 * Copies position p = pos0[b] + i (i < cu[b+1] - cu[b]) of sequence b from the
 * pool into row cu[b] + i of k_out / v_out, [num_tokens][Hkv][D] bfloat16
 * (device, caller-owned). Used to move a reused prefix's window between
 * requests' rings, to copy a page a new request only partly shares before it
 * writes to it, and to save a layer's K/V to a host-memory tier ([YLY]
 * KVCache系统重构: the prefix tree's SWA map and Full index point into
 * these pools; [HD9] "三层 KVCache 系统": KV moves between HBM and host
 * memory). A ring returns slot p mod W, whatever position it holds now: the
 * caller reads only positions the ring still holds. Page ids and ring ids
 * out of range give rows that are left unwritten. bf16 pools only
 * (HA_ERR_UNSUPPORTED for INT8). Arguments otherwise as for the appends. */
ha_status swa_ring_read(const ha_shape* shape, const ha_kv_view* ring, const int32_t* pos0, const int32_t* cu,
                        int32_t batch, int32_t num_tokens, void* k_out, void* v_out, void* stream);
ha_status full_pool_read(const ha_shape* shape, const ha_kv_view* pages, const int32_t* pos0, const int32_t* cu,
                         int32_t batch, int32_t num_tokens, void* k_out, void* v_out, void* stream);

/* ---- a3: window-safe prefix match ([HTX] 工程三; [YLY] KVCache系统重构;
 *          [HD9] Hybrid SWA 节; [HD12] 双池分治) ------------------------------
 * Host-only, synchronous. m = longest common prefix of the request and the
 * cached tokens; *out_len = the largest L <= m such that every position in
 * [max(0, L - window), L) has swa_valid[pos] != 0. L = 0 is always safe.
 *   req_tokens [req_len], cached_tokens [cached_len], swa_valid [cached_len]
 *   (all host memory); window >= 1. */
ha_status window_safe_match(const int32_t* req_tokens, int64_t req_len, const int32_t* cached_tokens,
                            int64_t cached_len, const uint8_t* swa_valid, int32_t window,
                            int64_t* out_len);

/* ---- a4/a5: prefill attention ([YLY] 为什么选择 Hybrid SWA 架构; [HD9]
 *          PD 分离与长度分桶: chunked prefill) ---------------------------------
 * Causal attention of a chunk of new tokens per sequence. Sequence b already
 * holds positions [0, hist_len[b]) in the pool; its n_b = cu_new[b+1] -
 * cu_new[b] new tokens are at positions [hist_len[b], hist_len[b] + n_b) and
 * their K/V are read from k_new/v_new (not from the pool). Attention is a pure
 * read: append the chunk afterwards (for SWA with n_b > 1 this order is
 * required, as the chunk would overwrite ring slots its first queries read).
 * For SWA layers the ring must hold positions [max(0, hist-W+1), hist).
 *   hist_len  int32 [batch] device;  cu_new int32 [batch+1] device
 *   num_tokens = cu_new[batch] (host);  max_new >= every n_b (host, sizes the grid)
 *   q [num_tokens][Hq][D], k_new/v_new [num_tokens][Hkv][D], in_dtype
 *   out float32 [num_tokens][Hq][D], lse float32 [num_tokens][Hq] (natural log)
 *   workspace: hybrid_attn_workspace_size(shape, kind, 0, batch, num_tokens, 0)
 *   bytes of device memory (the chunk's K/V re-laid as 16-token blocks; for
 *   full layers also the partial rows of work items split by keys, at the
 *   end of large calls and throughout calls of few items, merged into
 *   out/lse by a third kernel);
 *   it is scratch for this call only. */
ha_status hybrid_attn_prefill(const ha_shape* shape, const ha_kv_view* kv, const int32_t* hist_len,
                              const int32_t* cu_new, int32_t batch, int32_t num_tokens, int32_t max_new,
                              const void* q, const void* k_new, const void* v_new, int32_t in_dtype,
                              float* out, float* lse, void* workspace, size_t workspace_bytes,
                              void* stream);

/* ---- a6/a7/a8: decode attention with split-K ([YLY] 为什么选择 Hybrid SWA
 *          架构 and Decode加速与多模态优化: decode cost follows KV bytes read) --
 * One query per sequence at position t = kv_len[b] - 1; it sees its own
 * token. Full layers split the key range over workgroups (split-K) and merge
 * the partial results with lse = ln sum_s exp(lse_s), o = sum_s exp(lse_s -
 * lse) o_s.
 *   kv_len int32 [batch] device (0 = empty row: out = 0, lse = -inf)
 *   max_kv_len >= every kv_len[b] (host; sizes the split grid)
 *   q [batch][Hq][D] in_dtype; out float32 [batch][Hq][D]; lse float32 [batch][Hq]
 *   k_new, v_new: the new token's K/V, [batch][Hkv][D] in_dtype, or both NULL.
 *     Given: the pool holds positions < t and the call also appends position
 *     t (ring slot t mod W, or page t / page_size at page token t mod
 *     page_size) -- the same pool and outputs as swa_ring_append /
 *     full_pool_append followed by this call with NULL, in one launch.
 *     NULL: position t must already be in the pool and the pool is only read.
 *   num_splits: maximum key splits per sequence, 0 = automatic
 *   workspace: hybrid_attn_workspace_size(..., decode = 1) bytes. */
ha_status hybrid_attn_decode(const ha_shape* shape, const ha_kv_view* kv, const int32_t* kv_len,
                             int32_t batch, int32_t max_kv_len, const void* q, const void* k_new,
                             const void* v_new, int32_t in_dtype, float* out, float* lse,
                             int32_t num_splits, void* workspace, size_t workspace_bytes,
                             void* stream);

/* ---- hybrid_attn_decode without a workspace: for callers that cannot
 *          allocate device memory (code under HIP graph capture, tight serving
 *          loops, harnesses that forbid allocation) -----------------------------
 * Same arguments, results and errors as hybrid_attn_decode, minus the
 * workspace: the split-K partials go to a library-owned static device array
 * of HA_DECODE_SCRATCH_BYTES per device, loaded with the library and held
 * until the process ends. The call allocates and frees nothing.
 *   Limit: calls whose partials need more (batch * Hq * splits * (D + 1) * 4
 *   bytes when a full-layer call splits; SWA calls and single-split calls
 *   need none) fail with HA_ERR_WORKSPACE before any HIP call: pass a smaller
 *   num_splits, or use hybrid_attn_decode with a workspace.
 *   The stream must belong to the current device (HA_ERR_RANGE otherwise);
 *   the first call on a device looks up that device's array (one HIP symbol
 *   query, with the device current).
 *   Every call on a device shares its one array, which keeps the last call's
 *   contents: calls that overlap on one device (concurrent streams, several
 *   host threads) race and give undefined results. */
#define HA_DECODE_SCRATCH_BYTES (64u << 20)

ha_status hybrid_attn_decode_noalloc(const ha_shape* shape, const ha_kv_view* kv, const int32_t* kv_len,
                                     int32_t batch, int32_t max_kv_len, const void* q, const void* k_new,
                                     const void* v_new, int32_t in_dtype, float* out, float* lse,
                                     int32_t num_splits, void* stream);

/* Workspace bytes needed by hybrid_attn_decode (decode = 1: max_kv_len and
 * num_splits as passed to the call) or hybrid_attn_prefill (decode = 0: pass
 * num_tokens as max_kv_len; num_splits ignored); 0 on invalid input. */
size_t hybrid_attn_workspace_size(const ha_shape* shape, int32_t kind, int32_t decode, int32_t batch,
                                  int32_t max_kv_len, int32_t num_splits);

/* Key splits per sequence hybrid_attn_decode uses for these sizes (after
 * resolving num_splits = 0), or 0 on invalid input. */
int32_t hybrid_attn_decode_splits(const ha_shape* shape, int32_t kind, int32_t batch, int32_t max_kv_len,
                                  int32_t num_splits);

/* ---- multi-token verify decode ([HTX] 工程六 and [HD9] "MTP 与多模态流水线":
 *          the MTP head's 1 + 3 proposed tokens are verified in one step) --
 * nq new tokens per sequence at positions t0 .. t0 + nq - 1, t0 = kv_len[b] -
 * nq; the pool holds positions < t0 and the tokens' K/V are given. Query
 * token i sees keys [0, t0 + i] (full) or [t0 + i - W + 1, t0 + i] (SWA):
 * causal among the new tokens. The call also appends the nq tokens (ring
 * slots p mod W, or page p / page_size at page token p mod page_size) after
 * reading: pool and outputs equal hybrid_attn_prefill over a chunk of nq
 * tokens followed by the append. INT8 pools: the new tokens are quantized
 * with the appends' arithmetic and attend, like the history, as the codes
 * times the scales they are stored with; the pool afterwards equals the
 * append of the nq tokens.
 * Full layers split the history over workgroups like hybrid_attn_decode.
 *   kv_len int32 [batch] device (kv_len[b] < nq: rows out = 0, lse = -inf,
 *     nothing appended);  max_kv_len >= every kv_len[b] (host)
 *   nq: 1 <= nq <= 16 and nq * (Hq / Hkv) <= 32
 *   q [batch][nq][Hq][D], k_new/v_new [batch][nq][Hkv][D] in_dtype (required)
 *   out float32 [batch][nq][Hq][D]; lse float32 [batch][nq][Hq] (natural log)
 *   num_splits: maximum key splits per sequence, 0 = automatic
 *   workspace: hybrid_attn_verify_workspace_size(...) bytes (0 for SWA or a
 *   single split); scratch for this call only. */
ha_status hybrid_attn_verify(const ha_shape* shape, const ha_kv_view* kv, const int32_t* kv_len,
                             int32_t batch, int32_t max_kv_len, int32_t nq, const void* q,
                             const void* k_new, const void* v_new, int32_t in_dtype, float* out, float* lse,
                             int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes hybrid_attn_verify needs for these arguments; 0 when none
 * is needed or on invalid input. */
size_t hybrid_attn_verify_workspace_size(const ha_shape* shape, int32_t kind, int32_t batch, int32_t max_kv_len,
                                         int32_t nq, int32_t num_splits);

const char* ha_status_str(int32_t status);
const char* ha_last_error(void);
int32_t ha_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HYBRID_ATTN_H */
