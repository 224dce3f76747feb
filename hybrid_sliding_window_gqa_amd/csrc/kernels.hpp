// Launch parameters and host-side launchers of the hybrid attention kernels.
// Validation happens in api.cpp; launchers assume valid arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ha {

// Geometry after validation.
struct Geometry {
  int hq, hkv, d, window, group;  // group = hq / hkv
  int ring;                       // slots per (ring, kv head): window rounded up to 16-slot blocks
  int page_shift;                 // log2(page_size / 16): a page holds 1 << page_shift 16-token blocks
  float scale;                    // softmax scale (natural units)
};

struct AppendArgs {
  Geometry geo;
  bool full;              // false: SWA ring, true: Full pages
  uint16_t* k_pool;
  uint16_t* v_pool;
  int32_t num_blocks;     // rings or pages in the pool
  const int32_t* table;   // ring ids [B] or page table [B][stride]
  int32_t table_stride;
  const int32_t* pos0;
  const int32_t* cu_new;
  int32_t batch;
  int32_t num_tokens;
  const void* k_new;
  const void* v_new;
  bool src_f32;
  bool kv8;               // INT8 pools: codes in k_pool/v_pool (bytes), scales below
  float* k_scale;
  float* v_scale;
};

struct DecodeArgs {
  Geometry geo;
  bool full;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  int32_t num_blocks;
  const int32_t* table;
  int32_t table_stride;
  const int32_t* kv_len;
  int32_t batch;
  const void* q;
  bool q_f32;
  float* out;
  float* lse;
  int32_t splits;         // max splits per sequence (grid x)
  int32_t split_blocks;   // 16-token blocks per split
  float* part_o;          // [batch][hq][splits][d]
  float* part_lse;        // [batch][hq][splits]  (log2 domain)
  const void* k_new;      // [batch][hkv][d] new token's K (NULL: already in the pool)
  const void* v_new;      // [batch][hkv][d]
  uint16_t* k_pool_w;     // writable pool views for the fused append
  uint16_t* v_pool_w;
  bool kv8;               // INT8 pools: codes + per-token scales (written by a fused append)
  float* k_scale;
  float* v_scale;
};

struct PrefillArgs {
  Geometry geo;
  bool full;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  int32_t num_blocks;
  const int32_t* table;
  int32_t table_stride;
  const int32_t* hist_len;
  const int32_t* cu_new;
  int32_t batch;
  int32_t num_tokens;
  int32_t max_new;
  const void* q;
  const void* k_new;
  const void* v_new;
  bool in_f32;
  float* out;
  float* lse;
  uint16_t* stage;        // workspace: chunk K/V re-laid as 16-token blocks
  int64_t stage_blocks;   // blocks the workspace holds
  // Full layers: an XCD's sequence of work items ends in split_n1 items run
  // in split_p1 parts each, then split_n2 items in split_p2 parts (one
  // workgroup per part, over that share of the item's key tiles). A part
  // writes normalised partial rows to its entry of `part` (kPrefillPartEntries
  // entries of kPrefillFullRows rows: O [entry][row][D], then LSE
  // [entry][row] in the log2 domain) and prefill_merge_kernel combines an
  // item's parts into out / lse; parts without a key tile write nothing, and
  // an item with a single tile is written by its one part directly.
  int32_t split_n1, split_p1, split_n2, split_p2;
  float* part;
};

// Multi-token verify decode: nq new tokens per sequence at positions
// kv_len - nq .. kv_len - 1 (their K/V in k_new / v_new [B][nq][Hkv][D]).
struct VerifyArgs {
  Geometry geo;
  bool full;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  uint16_t* k_pool_w;     // writable views: the new tokens are appended
  uint16_t* v_pool_w;
  int32_t num_blocks;
  const int32_t* table;
  int32_t table_stride;
  const int32_t* kv_len;
  int32_t batch;
  int32_t nq;
  const void* q;          // [B][nq][Hq][D]
  const void* k_new;      // [B][nq][Hkv][D]
  const void* v_new;
  bool in_f32;
  bool kv8;               // INT8 pools: codes + per-token scales
  float* k_scale;
  float* v_scale;
  float* out;             // [B][nq][Hq][D]
  float* lse;             // [B][nq][Hq]
  int32_t splits;
  int32_t split_blocks;
  float* part_o;          // [B][nq][Hq][splits][D]
  float* part_lse;        // [B][nq][Hq][splits] (log2 domain)
};

// Workspace of hybrid_attn_prefill: the chunk's K and V in 16-token blocks
// (same layout as a pool page), sequence b's blocks starting at
// ceil(cu_new[b] / 16) + b.
int64_t prefill_stage_blocks(int num_tokens, int batch);

// Full-layer prefill work items: 384 rows (query position x query head of
// one kv head's group). Items of each of the 8 XCDs' sequences may run split
// by keys, in at most kPrefillPartsPerXcd workgroups per XCD (two rounds of
// its 32 CUs).
constexpr int kPrefillFullRows = 384;
constexpr int kPrefillPartsPerXcd = 64;
constexpr int kPrefillPartEntries = 8 * kPrefillPartsPerXcd;
// How a call of `items_per_xcd` work items per XCD splits them: the last n1
// items of each XCD's sequence in p1 parts, then n2 items in p2 parts
// (n1 * p1 + n2 * p2 <= kPrefillPartsPerXcd; all zero: no split).
void prefill_split_policy(int64_t items_per_xcd, int* n1, int* p1, int* n2, int* p2);
// Bytes of the partial rows of the split items (full layers), head dim d.
int64_t prefill_partial_bytes(int d);

hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
// Pool -> token-major rows (k_new / v_new of the args are the outputs).
hipError_t launch_read(const AppendArgs& a, void* k_out, void* v_out, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream);

// Device address of `device`'s copy of the decode kernels' static scratch
// array (HA_DECODE_SCRATCH_BYTES); `device` must be the current device.
hipError_t decode_scratch(int device, void** out);

// Decode split policy shared by the workspace query and the launcher.
int decode_split_blocks(bool full, int window, int max_kv_len, int batch, int hkv, int requested_splits);
int decode_num_splits(bool full, int window, int max_kv_len, int split_blocks);

}  // namespace ha
