// a4 / a5: causal prefill attention over the dual-pool KV cache.
//
// A chunk of new tokens per sequence attends to the sequence's history in the
// pool (the SWA ring's last W-1 positions, or every page of the Full pool)
// and causally to the chunk itself. SWA layers cut the attended range from
// the whole sequence to the window (youleyou.com
// "小米MiMo首次公开模型推理系统全链路优化降价99%", section 1
// "为什么选择 Hybrid SWA 架构"); chunked prefill is what the serving stack runs
// for long requests (blog.hotdry.top 2026-06-09, section "PD 分离与长度分桶").
//
// Two kernels per call, three when a full-layer call splits work items:
//  1. stage_chunk_kernel re-lays the chunk's K/V (bf16 or f32) into 16-token
//     blocks in the workspace, in exactly the pools' block format (matrix-core
//     operand order, common.hpp), zero-padded past the chunk's end. Every key
//     source then looks the same to the attention kernel: a K block and a V
//     block of 16*D bf16 each.
//  2. prefill_kernel. A workgroup holds the rows of one (sequence, kv head);
//     a row is a (query position, query head of the GQA group) pair, so the
//     whole group shares every K/V tile. Full layers: 8 waves of 48 rows
//     (three 16-row MFMA column groups; 384 rows) share each staged tile, one
//     workgroup per CU -- every wave reads the whole tile from LDS, so more
//     rows per wave means fewer LDS bytes per MFMA, and staging per MFMA is a
//     third of what 4 waves of 32 rows would need. SWA layers (three tiles
//     or so per workgroup, bound by the latency of that short chain): 4
//     waves of 32 rows, two workgroups per CU. Keys
//     are consumed in 64-key tiles of four blocks and staged into LDS in
//     stage tiles of 128 keys (full: one block per wave, two compute tiles
//     per barrier) or 64 keys (SWA). The waves stage the next stage tile
//     while the current one is consumed -- K straight from global memory
//     into LDS (buffer loads with the LDS bit), V through registers, one
//     phase per compute tile -- so one barrier per stage tile suffices.
//     LDS operand reads are scheduled ahead of their MFMAs.
//     The K tiles are plain copies of the blocks; since blocks are in
//     operand order, every K operand read is one ds_read_b128 at 16 * lane:
//     consecutive lanes, consecutive 16 bytes, no bank conflicts.
//     Per tile and wave: S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (Q^T held in
//     registers), exp2-domain online softmax per row, P^T cast to bf16 in the
//     accumulator layout, then O^T += V^T P^T, also on
//     v_mfma_f32_16x16x32_bf16 (two key blocks per product; the older
//     16x16x16 form runs at half the rate on gfx950). Full layers keep the
//     softmax's vector work per score at one FMA, one exp2, one add and half
//     a conversion: the exp2 reference is not the row max but any value that
//     keeps every probability <= 2^16 (checked on the lane's partial row
//     sums after the exp2s); only a tile that fails the check, or a row's
//     first keys, takes the row max (a cross-lane reduction), rescales O and
//     l and recomputes. SWA layers (a few tiles per row) take the row max
//     every tile and raise the reference only past a slack. Their chunk
//     tiles start at the block holding the window's first key, and a tile's
//     blocks that hold no key are not computed (a 16-position query block's
//     143 keys take 9 blocks, not 12).
//     Tiles a wave sees completely skip masking; tiles no row of the wave
//     sees are skipped.
//
//  3. prefill_merge_kernel (full layers). Some items ran as several
//     workgroups over parts of their key tiles, and this merges their
//     partial rows (O, LSE) into the output: in calls of more than one round
//     of items per XCD, the last items of each XCD's sequence (two or four
//     parts), so that the final round is not a few whole items on otherwise
//     idle CUs; in calls of at most 21 items per XCD (short chunks of few
//     sequences over long histories), every item, so that all 32 CUs of an
//     XCD have work.
//
// Grid order: workgroup i runs on XCD i % 8 (round-robin dispatch). All query
// blocks of one (sequence, kv head) pair are placed on the same XCD and
// dispatched back to back (heaviest, i.e. latest, first), so the workgroups
// resident on an XCD stream one pair's K/V in near lockstep through its L2.
// When the pairs are not a multiple of 8 (few kv heads, small batches), each
// pair's blocks are dealt into 8 / gcd(pairs, 8) units placed the same way,
// so every XCD gets the same number of units of about equal work.
#include <cmath>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace ha {

namespace {

// Keys are consumed in 64-key tiles of four blocks; they are staged into LDS
// in stage tiles of kStageKeys: 128 keys for full layers (two compute tiles
// per barrier), 64 for SWA layers.
constexpr int kTileKeys = 64;
constexpr int kTileBlocks = kTileKeys / kBlock;   // 4
template <bool kFull>
constexpr int stage_keys() { return kFull ? 128 : 64; }
constexpr int kXcds = 8;
// Full layers: 8 waves (384 rows) share each staged tile, one workgroup per
// CU. SWA layers: 4 waves (128 rows), two workgroups per CU so one's
// prologue/epilogue overlaps the other.
template <bool kFull>
constexpr int waves_per_wg() { return kFull ? 8 : 4; }
template <bool kFull>
constexpr int rows_per_wave() { return kFull ? 48 : 32; }
template <bool kFull>
constexpr int rows_per_wg() { return rows_per_wave<kFull>() * waves_per_wg<kFull>(); }
static_assert(rows_per_wg<true>() == kPrefillFullRows, "partial-row layout of split full-layer items");

// Work units: each (sequence, kv head) pair's query blocks, latest
// (heaviest) first, dealt into 2^rsh units of qb_sub blocks (unit r of a
// pair takes its blocks r, r + 2^rsh, ...), where 2^rsh = 8 / gcd(pairs, 8)
// makes the unit count a multiple of the 8 XCDs (one unit per pair when the
// pairs already are). Dealt rather than cut into ranges, a pair's units
// carry equal work: causal blocks grow with their position. Units on XCD x
// are x, x + 8, ...; item jj of an XCD's sequence is block jj % qb_sub of
// its unit jj / qb_sub, so a unit's blocks run back to back on one XCD.
__device__ __forceinline__ int unit_shift(int npairs) { return 3 - min(__builtin_ctz(static_cast<unsigned>(npairs)), 3); }
__device__ __forceinline__ void work_item(int jj, int xcd, int qb_max, int qb_sub, int rsh, int& pair, int& qblk) {
  const int unit = (jj / qb_sub) * kXcds + xcd;
  pair = unit >> rsh;
  qblk = qb_max - 1 - (((jj % qb_sub) << rsh) + (unit & ((1 << rsh) - 1)));
}

// Split items of full layers (PrefillArgs::split_*): an XCD's sequence ends
// in n1 items of p1 parts, then n2 items of p2 parts. Split item k (counted
// from the first split item) has split_parts(k) parts, whose partial rows
// take consecutive entries from xcd * kPrefillPartsPerXcd + split_entry(k).
__device__ __forceinline__ int split_parts(const PrefillArgs& a, int k) { return k < a.split_n1 ? a.split_p1 : a.split_p2; }
__device__ __forceinline__ int split_entry(const PrefillArgs& a, int k) {
  return k < a.split_n1 ? k * a.split_p1 : a.split_n1 * a.split_p1 + (k - a.split_n1) * a.split_p2;
}
// Stage tiles of a full-layer work item: history tiles (128 keys of the
// pages, up to the page-table row's `row_blocks` 16-token blocks), then chunk
// tiles up to the block's end.
__device__ __forceinline__ int full_item_tiles(int hist, int i_end, int row_blocks, int stage_keys) {
  const int hist_blocks = min((hist + kBlock - 1) / kBlock, row_blocks);
  const int blocks_per_tile = stage_keys / kBlock;
  return (hist_blocks + blocks_per_tile - 1) / blocks_per_tile + (i_end + stage_keys - 1) / stage_keys;
}
// SWA layers write O through LDS with full-row non-temporal stores (see the
// kernel's epilogue): 2% faster SWA layers on the chunked workload; full
// layers, whose epilogue is a small part of a workgroup's time, measured the
// same either way and keep the direct stores.
template <bool kFull>
constexpr bool lds_epilogue() { return !kFull; }

// LDS tiles as 16-byte units (alignment known to the compiler, so stores and
// loads are single ds_write_b128 / ds_read_b128 instructions).
//   k: the four K blocks as they are (operand order).
//   v: the V blocks interleaved by pairs: unit [pair][a][h][lane] holds the
//      8 bytes of half h (dim tile 2a + h) of V unit (a, lane) from block
//      2*pair, then the same 8 bytes from block 2*pair + 1 -- exactly the
//      v_mfma_f32_16x16x32_bf16 A operand of a 32-key product.
template <int D, int kBlocks>
struct Smem {
  static constexpr int kUnits = kBlocks * kBlock * D / 8;   // 16-byte units per stage tile
  u32x4 k[2][kUnits];
  u32x4 v[2][kUnits];
  int4 pos[2][kBlocks * kBlock / 4];
};

// Largest partial row sum (one lane's 16 probabilities of a tile) accepted
// without recomputing the tile against a raised reference (full layers).
constexpr float kAcceptSum = 65536.0f;
// Softmax reference slack (log2 units, SWA layers): the running max used as
// the exp2 reference is only raised when a tile's max exceeds it by more
// than this, so probabilities stay <= 2^8 and the O/l rescale is rare.
constexpr float kRescaleSlack = 8.0f;
// Position staged for an SWA ring slot that holds no key: far enough below
// every query position that the window test's unsigned distance exceeds W.
constexpr int kNoKey = -(1 << 30);

// V unit of lane group q holds tokens 4q..4q+3 (for two channels): zero the
// tokens at index >= nv.
__device__ __forceinline__ u32x4 keep_tokens_v(u32x4 v, int q, int nv) {
  const int first = 4 * q;
  if (first + 4 <= nv) return v;
  const uint32_t m0 = (first + 0 < nv ? 0x0000ffffu : 0u) | (first + 1 < nv ? 0xffff0000u : 0u);
  const uint32_t m1 = (first + 2 < nv ? 0x0000ffffu : 0u) | (first + 3 < nv ? 0xffff0000u : 0u);
  return u32x4{v.x & m0, v.y & m1, v.z & m0, v.w & m1};
}

// Zero token `tok` (0..15) of a V unit of lane group q (tokens 4q..4q+3).
__device__ __forceinline__ u32x4 drop_token_v(u32x4 v, int q, int tok) {
  if ((tok >> 2) != q) return v;
  const uint32_t m = (tok & 1) ? 0x0000ffffu : 0xffff0000u;
  if (tok & 2) return u32x4{v.x, v.y & m, v.z, v.w & m};
  return u32x4{v.x & m, v.y, v.z & m, v.w};
}

}  // namespace

// ---- 1. stage the chunk's K/V as 16-token blocks ----
// Grid (ceil(max_new/16), batch); one workgroup per (sequence, block), all kv heads.
template <int D, bool kF32>
__global__ __launch_bounds__(256) void stage_chunk_kernel(PrefillArgs a) {
  constexpr int CPR = D / 8;                   // 16-byte chunks per row
  __shared__ uint16_t tile[kBlock][D + 2];     // one head's 16 V rows
  const int b = blockIdx.y;
  const int i = blockIdx.x;
  const int tok0 = a.cu_new[b];
  const int n = min(a.cu_new[b + 1], a.num_tokens) - tok0;
  if (tok0 < 0 || kBlock * i >= n) return;
  const int64_t blk = (tok0 + kBlock - 1) / kBlock + b + i;
  if (blk >= a.stage_blocks) return;
  const int hkv = a.geo.hkv;
  const int64_t blk_elems = static_cast<int64_t>(kBlock) * D;
  uint16_t* ws_k = a.stage + blk * hkv * blk_elems;
  uint16_t* ws_v = a.stage + (a.stage_blocks + blk) * hkv * blk_elems;
  const int tid = threadIdx.x;
  for (int g = 0; g < hkv; ++g) {
    // K rows (and V rows into LDS): thread -> (key, chunk)
    for (int e = tid; e < kBlock * CPR; e += blockDim.x) {
      const int key = e / CPR;
      const int col = e - key * CPR;
      const int ci = kBlock * i + key;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (ci < n) {
        const int64_t off = (static_cast<int64_t>(tok0 + ci) * hkv + g) * D + col * 8;
        kv = load8_as_bf16_stream<kF32>(a.k_new, off);
        vv = load8_as_bf16_stream<kF32>(a.v_new, off);
      }
      *reinterpret_cast<u32x4*>(ws_k + g * blk_elems + k_elem(key, col * 8)) = kv;
      const uint32_t w4[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        tile[key][col * 8 + 2 * j] = static_cast<uint16_t>(w4[j] & 0xffffu);
        tile[key][col * 8 + 2 * j + 1] = static_cast<uint16_t>(w4[j] >> 16);
      }
    }
    __syncthreads();
    // V units: thread e -> unit (p, q, c): tokens 4q..4q+3 of channels 32p+c, 32p+16+c
    for (int e = tid; e < 2 * D; e += blockDim.x) {
      const int p = e / 64;
      const int q = (e / 16) & 3;
      const int c = e & 15;
      uint32_t w4[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ch = 32 * p + 16 * h + c;
        w4[2 * h] = static_cast<uint32_t>(tile[4 * q][ch]) | (static_cast<uint32_t>(tile[4 * q + 1][ch]) << 16);
        w4[2 * h + 1] = static_cast<uint32_t>(tile[4 * q + 2][ch]) | (static_cast<uint32_t>(tile[4 * q + 3][ch]) << 16);
      }
      *reinterpret_cast<u32x4*>(ws_v + g * blk_elems + 8 * e) = u32x4{w4[0], w4[1], w4[2], w4[3]};
    }
    __syncthreads();
  }
}

// ---- 2. attention ----
template <int D, bool kFull, bool kF32>
__global__ __launch_bounds__(64 * waves_per_wg<kFull>(), kFull ? 1 : 2) void prefill_kernel(PrefillArgs a) {
  constexpr int kWaves = waves_per_wg<kFull>();
  constexpr int kRowsPerWave = rows_per_wave<kFull>();
  constexpr int kRowGroups = kRowsPerWave / 16;
  constexpr int kRowsPerWg = rows_per_wg<kFull>();
  constexpr int kStageKeys = stage_keys<kFull>();
  constexpr int kStageBlocks = kStageKeys / kBlock;
  constexpr int kSubTiles = kStageKeys / kTileKeys;   // compute tiles per stage tile
  constexpr int kWavesPerBlock = kWaves / kStageBlocks;
  static_assert(kWaves % kStageBlocks == 0, "each block of a stage tile is staged by whole waves");
  constexpr int KS = D / 32;            // QK^T reduction steps
  constexpr int DT = D / 16;            // output dim tiles
  constexpr int CPL = D / 32;           // 16-byte units per lane of one block
  constexpr int kBlk = kBlock * D;      // bf16 per block
  __shared__ Smem<D, kStageBlocks> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4;
  const int c16 = lane & 15;

  const int hkv = a.geo.hkv;
  const int hq = a.geo.hq;
  const int G = a.geo.group;
  // The group is a power of two (1..16, checked at the boundary): row ->
  // (position, head) by shift and mask, not by integer division.
  const int gsh = __builtin_ctz(static_cast<unsigned>(G));
  const int W = a.geo.window;
  const int QB = kRowsPerWg >> gsh;     // query positions per workgroup

  // ---- workgroup -> (sequence, kv head, query block), XCD-aware ----
  const int npairs = a.batch * hkv;
  const int qb_max = (a.max_new + QB - 1) / QB;
  const int rsh = unit_shift(npairs);
  const int qb_sub = (qb_max + (1 << rsh) - 1) >> rsh;
  const int items = qb_sub * ((npairs << rsh) / kXcds);   // work items per XCD
  const int lin = blockIdx.x;
  const int xcd = lin % kXcds;
  int jj = lin / kXcds;
  // Full layers: the split items at the end of the XCD's sequence run in
  // parts (part key_part of key_parts takes that share of the item's key
  // tiles), one workgroup each, which write partial rows to entry
  // `part_entry` for prefill_merge_kernel.
  int key_part = 0, key_parts = 1, part_entry = -1;
  if constexpr (kFull) {
    const int n1 = a.split_n1, p1 = a.split_p1, n2 = a.split_n2, p2 = a.split_p2;
    const int first_split = items - n1 - n2;
    if (n1 + n2 > 0 && jj >= first_split) {
      const int r = jj - first_split;            // workgroup within the XCD's split region
      part_entry = xcd * kPrefillPartsPerXcd + r;
      int k;
      if (r < n1 * p1) {
        k = r / p1;
        key_part = r - k * p1;
        key_parts = p1;
      } else {
        const int r2 = r - n1 * p1;
        k = n1 + r2 / p2;
        key_part = r2 - (k - n1) * p2;
        key_parts = p2;
      }
      jj = first_split + k;
    }
  }
  // Unit-major within an XCD: the workgroups resident on one XCD at a time
  // are query blocks of ONE pair (of one unit of it), so they stream the
  // same K/V tiles at nearly the same time and the XCD's L2 serves most of
  // them.
  int pair, qblk;
  work_item(jj, xcd, qb_max, qb_sub, rsh, pair, qblk);
  if (pair >= npairs || qblk < 0) return;
  const int b = pair / hkv;
  const int g = pair - b * hkv;
  const int tok0 = a.cu_new[b];
  // Rows past num_tokens (an inconsistent cu_new) are dropped, never read.
  const int n = min(a.cu_new[b + 1], a.num_tokens) - tok0;
  const int i0 = qblk * QB;               // first chunk index of this block
  if (tok0 < 0 || i0 >= n) return;
  const int hist = max(a.hist_len[b], 0);
  const int i_end = min(n, i0 + QB);      // one past the last chunk index
  const int t_first = hist + i0;
  const int64_t stage_blk0 = (tok0 + kBlock - 1) / kBlock + b;

  // ---- tile list: history tiles, then chunk tiles ----
  int n_hist_tiles = 0;
  int ring = -1;
  const int32_t* page_row = a.table + static_cast<int64_t>(b) * a.table_stride;
  int hist_blocks = 0;
  if constexpr (kFull) {
    hist_blocks = min((hist + kBlock - 1) / kBlock, a.table_stride << a.geo.page_shift);
    n_hist_tiles = (hist_blocks + kStageBlocks - 1) / kStageBlocks;
  } else {
    ring = a.table[b];
    const bool ring_ok = ring >= 0 && ring < a.num_blocks;
    hist_blocks = a.geo.ring / kBlock;
    if (ring_ok && hist > 0 && t_first - W + 1 < hist) n_hist_tiles = (hist_blocks + kStageBlocks - 1) / kStageBlocks;
  }
  // Chunk tiles start at chunk index c_first: 0 for full layers; for SWA
  // layers the block holding the first key any row of the workgroup sees,
  // so a 16-position query block's window (143 keys) takes 9 blocks -- two
  // full tiles and a 1-block tile -- instead of three 64-aligned tiles.
  int c_first = 0;
  if constexpr (!kFull) c_first = kBlock * (max(0, i0 - W + 1) / kBlock);
  const int n_chunk_tiles = (i_end - c_first + kStageKeys - 1) / kStageKeys;
  // (full layers: the count prefill_merge_kernel recomputes for split items)
  const int n_tiles =
      kFull ? full_item_tiles(hist, i_end, a.table_stride << a.geo.page_shift, kStageKeys) : n_hist_tiles + n_chunk_tiles;
  // Stage tiles this workgroup consumes: all, or its part's share. A part
  // with no tile writes nothing; an item of one tile is written, as if
  // whole, by the one part that has it.
  const int t_begin = key_part * n_tiles / key_parts;
  const int t_end = (key_part + 1) * n_tiles / key_parts;
  if (t_begin == t_end && key_parts > 1) return;
  if (n_tiles <= 1) part_entry = -1;

  // ---- rows of this wave ----
  const int row0 = wave * kRowsPerWave;
  const int wave_i_lo = i0 + (row0 >> gsh);
  const int wave_i_hi = min(i_end - 1, i0 + ((row0 + kRowsPerWave - 1) >> gsh));
  const bool wave_live = wave_i_lo < i_end;
  const int qlo = hist + wave_i_lo;
  const int qhi = hist + wave_i_hi;

  // Q^T operands and per-row query positions.
  u32x4 qop[kRowGroups][KS];
  int qpos[kRowGroups];
#pragma unroll
  for (int rg = 0; rg < kRowGroups; ++rg) {
    const int rho = row0 + 16 * rg + c16;
    const int ci = i0 + (rho >> gsh);
    const int hh = g * G + (rho & (G - 1));
    const bool ok = ci < i_end;
    qpos[rg] = hist + ci;
    const int64_t off = (static_cast<int64_t>(tok0 + (ok ? ci : 0)) * hq + hh) * D + 8 * q4;
#pragma unroll
    for (int m = 0; m < KS; ++m) {
      qop[rg][m] = load8_as_bf16<kF32>(a.q, off + 32 * m);
      if (!ok) qop[rg][m] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  // ---- staging: wave w moves block w of a tile ----
  // Page ids of this wave's history blocks, 64 tiles at a time: lane j holds
  // the page of tile (batch_base + j), batches counted from t_begin. One
  // vector load per 64 tiles; the per-tile id is a readlane (scalar), so the
  // tile loop never waits on it.
  // Wave w stages units [part * kStageUnits, +kStageUnits) of block sb.
  constexpr int kStageUnits = CPL / kWavesPerBlock;
  const int sb = wave / kWavesPerBlock;
  const int part = wave % kWavesPerBlock;
  int pg_vec = -1;
  auto fetch_pages = [&](int batch_base) {
    if constexpr (kFull) {
      const int t = batch_base + lane;
      const int lb = t * kStageBlocks + sb;
      pg_vec = (t < n_hist_tiles && lb < hist_blocks) ? page_row[lb >> a.geo.page_shift] : -1;
    }
  };
  auto page_for = [&](int tile) -> int {
    if constexpr (kFull) return __builtin_amdgcn_readlane(pg_vec, (tile - t_begin) & 63);
    else return -1;
  };
  // Element offset of this wave's block of tile `tile` (-1: nothing to load),
  // plus the number of leading valid keys of that block. `no_page`: a full
  // history block whose page id is out of range; like decode and verify,
  // prefill then treats its 16 positions as missing keys (masked).
  auto block_of = [&](int tile, int pg, int& valid, bool& no_page) -> int64_t {
    no_page = false;
    if (tile < n_hist_tiles) {
      const int lb = tile * kStageBlocks + sb;
      if (lb >= hist_blocks) { valid = 0; return -1; }
      if constexpr (kFull) {
        valid = min(kBlock, hist - lb * kBlock);
        if (pg < 0 || pg >= a.num_blocks) { valid = 0; no_page = true; return -1; }
        return page_block_offset(pg, g, hkv, lb & ((1 << a.geo.page_shift) - 1), a.geo.page_shift, kBlock * D);
      } else {
        // leading slots holding a position: min(hist, W) of the ring's slots
        valid = min(kBlock, max(0, min(hist, W) - lb * kBlock));
        return ((static_cast<int64_t>(ring) * hkv + g) * a.geo.ring + kBlock * lb) * D;
      }
    } else {
      const int cb = c_first / kBlock + (tile - n_hist_tiles) * kStageBlocks + sb;  // chunk block
      if (kBlock * cb >= i_end) { valid = 0; return -1; }
      valid = min(kBlock, i_end - kBlock * cb);
      return ((stage_blk0 + cb) * hkv + g) * kBlock * D;  // K part; V part is offset by stage_blocks
    }
  };

  // Ring slot of the newest history position (hist - 1) mod W, in [0, W).
  const int last_slot = kFull ? 0 : ((hist - 1) % W + W) % W;
  auto key_position = [&](int tile, int kk) -> int {   // kk = key within the tile
    if (tile < n_hist_tiles) {
      if constexpr (kFull) {
        const int p = tile * kStageKeys + kk;
        return p < hist ? p : -1;
      } else {
        const int s = tile * kStageKeys + kk;             // ring slot
        if (s >= W) return kNoKey;
        int d = last_slot - s;                            // slots back from the newest
        if (d < 0) d += W;
        const int p = hist - 1 - d;
        return p >= 0 ? p : kNoKey;
      }
    } else {
      const int ci = c_first + (tile - n_hist_tiles) * kStageKeys + kk;
      return (ci < i_end) ? hist + ci : kNoKey;
    }
  };

  // V is staged in kSubTiles phases (one per compute tile of the stage
  // tile), so only kVUnits 16-byte units per lane are held in registers at
  // a time.
  constexpr int kVUnits = kStageUnits / kSubTiles;
  static_assert(kStageUnits % kSubTiles == 0, "V phases split the wave's units evenly");
  u32x4 stv[kVUnits];
  int st_pos = -1;
  __amdgpu_buffer_rsrc_t st_rv;   // V source of the block being staged
  int st_valid = kBlock;          // leading valid tokens of that block
  bool st_partial = false;        // partial history block: zero its unwritten V
  int st_drop = -1;               // ring slot of position hist - W in this block (zeroed), or -1
  bool st_no_page = false;        // full history block without a valid page (its keys are masked)
  // K goes global -> LDS directly (buffer_load ... lds: lane l's 16 bytes land
  // at the wave's LDS base + 16 l); V goes through registers (partial history
  // blocks get their unwritten tokens zeroed on the way).
  auto load_tile = [&](int tile, int pg, int buf) {
    int valid;
    const int64_t base = block_of(tile, pg, valid, st_no_page);
    const int64_t b0 = base >= 0 ? base : 0;
    const uint32_t bytes = base >= 0 ? kBlock * D * 2 : 0;   // 0: loads return zeros, no traffic
    const bool hist_tile = tile < n_hist_tiles;
    const uint16_t* kp = hist_tile ? a.k_pool + b0 : a.stage + b0;
    const uint16_t* vp = hist_tile ? a.v_pool + b0 : a.stage + a.stage_blocks * hkv * kBlock * D + b0;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kp, bytes);
    st_rv = make_rsrc(vp, bytes);
    st_valid = valid;
    st_partial = hist_tile && valid < kBlock;
    // SWA: the slot of position hist - W is outside every query's window and
    // need not hold it (the ring only has to keep [hist - W + 1, hist)); its
    // V is zeroed so that whatever it holds cannot reach O through P = 0.
    st_drop = -1;
    if constexpr (!kFull) {
      if (hist_tile && hist >= W && (hist % W) / kBlock == tile * kStageBlocks + sb) st_drop = (hist % W) % kBlock;
    }
#pragma unroll
    for (int j = 0; j < kStageUnits; ++j) {
      const int e = lane + 64 * (part * kStageUnits + j);      // 16-byte chunk of the block
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, (__attribute__((address_space(3))) void*)(&sm.k[buf][sb * (kBlk / 8) + e - lane]), 16, 16 * e, 0, 0, 0);
    }
    // Full-layer key positions are contiguous per tile (computed in the
    // mask); only the SWA ring's positions are staged.
    if constexpr (!kFull)
      if (part == 0 && lane < kBlock) st_pos = key_position(tile, sb * kBlock + lane);
  };
  auto load_v = [&](int phase) {
#pragma unroll
    for (int j = 0; j < kVUnits; ++j) {
      const int e = lane + 64 * (part * kStageUnits + phase * kVUnits + j);
      stv[j] = buf_load16(st_rv, 16 * e);
    }
    if (st_partial) {
#pragma unroll
      for (int j = 0; j < kVUnits; ++j) stv[j] = keep_tokens_v(stv[j], lane >> 4, st_valid);
    }
    if constexpr (!kFull) {
      if (st_drop >= 0) {
#pragma unroll
        for (int j = 0; j < kVUnits; ++j) stv[j] = drop_token_v(stv[j], lane >> 4, st_drop);
      }
    }
  };
  auto store_v = [&](int buf, int phase) {
    u32x2* vpair = reinterpret_cast<u32x2*>(sm.v[buf]);
    const int pair = sb >> 1;
    const int slot = sb & 1;
#pragma unroll
    for (int j = 0; j < kVUnits; ++j) {
      const int u = part * kStageUnits + phase * kVUnits + j;
      // V unit (a = u, lane): half 0 -> dim tile 2u, half 1 -> dim tile 2u + 1
      const int base = ((pair * CPL + u) * 2) * 64 + lane;        // [pair][a][h=0][lane]
      vpair[2 * base + slot] = u32x2{stv[j].x, stv[j].y};
      vpair[2 * (base + 64) + slot] = u32x2{stv[j].z, stv[j].w};
    }
  };
  auto store_pos = [&](int buf) {
    if constexpr (!kFull) {
      if (part == 0 && lane < kBlock) reinterpret_cast<int32_t*>(sm.pos[buf])[sb * kBlock + lane] = st_pos;
    } else {
      // one flag per block of the stage tile: 1 = no valid page
      if (part == 0 && lane == 0) reinterpret_cast<int32_t*>(sm.pos[buf])[sb] = st_no_page ? 1 : 0;
    }
  };

  // Key-position bounds of compute tile `sub` of stage tile `tile` (uniform):
  // [kmin, kmax] (empty when kmax < kmin); exact = every key valid.
  auto tile_bounds = [&](int tile, int sub, int& kmin, int& kmax, bool& exact) {
    if (tile < n_hist_tiles) {
      if constexpr (kFull) {
        kmin = tile * kStageKeys + kTileKeys * sub;
        kmax = min(kmin + kTileKeys, hist) - 1;
        exact = kmin + kTileKeys <= hist;
      } else {
        kmin = max(0, hist - W);
        kmax = hist - 1;
        exact = false;
      }
    } else {
      const int c0 = c_first + (tile - n_hist_tiles) * kStageKeys + kTileKeys * sub;
      kmin = hist + c0;
      kmax = hist + min(c0 + kTileKeys, i_end) - 1;
      exact = c0 + kTileKeys <= i_end;
    }
  };

  // ---- main loop ----
  bool have_ref = false;   // SWA: the wave has computed a tile (O and l may be nonzero)
  const float sl2 = a.geo.scale * kLog2e;
  float m_run[kRowGroups], l_run[kRowGroups];
  f32x4 o[kRowGroups][DT];
#pragma unroll
  for (int rg = 0; rg < kRowGroups; ++rg) {
    m_run[rg] = -INFINITY;
    l_run[rg] = 0.0f;
#pragma unroll
    for (int d = 0; d < DT; ++d) o[rg][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  fetch_pages(t_begin);
  if (t_end > t_begin) {
    load_tile(t_begin, page_for(t_begin), 0);
#pragma unroll
    for (int ph = 0; ph < kSubTiles; ++ph) {
      load_v(ph);
      store_v(0, ph);
    }
    store_pos(0);
  }
  // Full layers: does any history block of this workgroup's tiles lack a
  // valid page (a hole in the page table, which the tiles then mask)? Only
  // then do the tiles read the per-block flags from LDS; skipping that read
  // made the chunked workload's full-layer call 1.5-4.8% faster (three
  // rounds on one box). Each wave checks a share of the page ids and
  // publishes the result before the barrier below.
  __shared__ int sm_bad[kWaves];
  if constexpr (kFull) {
    bool bad = false;
    const int hb0 = min(t_begin * kStageBlocks, hist_blocks);
    const int hb1 = min(min(t_end, n_hist_tiles) * kStageBlocks, hist_blocks);
    if (hb1 > hb0) {
      const int p1 = ((hb1 - 1) >> a.geo.page_shift) + 1;
      for (int p = (hb0 >> a.geo.page_shift) + tid; p < p1; p += 64 * kWaves) {
        const int pg = page_row[p];
        bad = bad || pg < 0 || pg >= a.num_blocks;
      }
    }
    const bool wave_bad = __any(bad);
    if (lane == 0) sm_bad[wave] = wave_bad ? 1 : 0;
  }
  // Everything loaded so far (Q, first tile) is complete before the loop, so
  // the loop's only outstanding global loads are the next tile's staging.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  bool any_bad = false;
  if constexpr (kFull) {
    int acc = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) acc |= sm_bad[w];
    any_bad = __builtin_amdgcn_readfirstlane(acc) != 0;
  }

  for (int tile = t_begin; tile < t_end; ++tile) {
    const int buf = (tile - t_begin) & 1;
    const bool has_next = tile + 1 < t_end;
    if (((tile + 1 - t_begin) & 63) == 0 && tile + 1 < n_hist_tiles) fetch_pages(tile + 1);
    if (has_next) {
      load_tile(tile + 1, page_for(tile + 1), buf ^ 1);
      load_v(0);
    }

#pragma unroll
    for (int sub = 0; sub < kSubTiles; ++sub) {
    int kmin, kmax;
    bool exact;
    tile_bounds(tile, sub, kmin, kmax, exact);
    bool visible_any = wave_live && kmin <= qhi && kmin <= kmax;
    if constexpr (!kFull) visible_any = visible_any && kmax >= qlo - W + 1;
    bool need_mask = !(exact && kmax <= qlo);
    if constexpr (!kFull) need_mask = need_mask || kmin < qhi - W + 1;
    // Full history tiles: bit kb set = block kb of this compute tile has no valid page.
    int no_page_bits = 0;
    if constexpr (kFull) {
      if (any_bad && tile < n_hist_tiles) {
        const int4 f = reinterpret_cast<const int4*>(sm.pos[buf])[sub];
        no_page_bits = __builtin_amdgcn_readfirstlane((f.x & 1) | ((f.y & 1) << 1) | ((f.z & 1) << 2) |
                                                      ((f.w & 1) << 3));
        need_mask = need_mask || no_page_bits != 0;
      }
    }

    // One compute tile whose keys sit in its first NB blocks (NB < 4 only
    // for the last chunk tile of an SWA window; the other blocks hold
    // zeros and are not computed).
    auto compute_tile = [&](auto nb_const) __attribute__((always_inline)) {
      constexpr int NB = decltype(nb_const)::value;
      constexpr int kPairs = (NB + 1) / 2;
      const u32x4* sk = sm.k[buf] + sub * kTileBlocks * (kBlk / 8);
      const u32x4* sv = sm.v[buf] + sub * (kTileBlocks / 2) * (DT / 2) * 2 * 64;
      f32x4 s[NB][kRowGroups];
      // S^T = K Q^T for the tile (then masked where needed).
      auto scores = [&]() __attribute__((always_inline)) {
        // Compiler-only fence: the recomputation must read K again rather
        // than keep the first reads' registers alive across the softmax.
        asm volatile("" ::: "memory");
        // K operands stream through a short register window: operand j
        // (block j / KS, reduction step j % KS) feeds one MFMA per row group.
        constexpr int kKOps = NB * KS;
        constexpr int kAhead = (kFull ? 5 : 8) < kKOps ? (kFull ? 5 : 8) : kKOps;   // K operands in flight
        u32x4 kr[kKOps];
#pragma unroll
        for (int j = 0; j < kKOps; ++j) kr[j] = sk[(j / KS) * (kBlk / 8) + 64 * (j % KS) + lane];
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
          for (int rg = 0; rg < kRowGroups; ++rg) s[kb][rg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kKOps; ++j) {
#pragma unroll
          for (int rg = 0; rg < kRowGroups; ++rg) s[j / KS][rg] = mfma_16x16x32(kr[j], qop[rg][j % KS], s[j / KS][rg]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
        for (int j = 0; j < kKOps - kAhead; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, kRowGroups, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kAhead * kRowGroups, 0);

        if (need_mask) {
          // A block that every row of the wave sees in full keeps its scores
          // (ring tiles: positions are not contiguous, always masked).
          auto block_all_visible = [&](int kb) -> bool {
            const int klo = kmin + kBlock * kb;
            const int khi = klo + kBlock - 1;
            if constexpr (kFull) return khi <= kmax && khi <= qlo && !((no_page_bits >> kb) & 1);
            else return tile >= n_hist_tiles && khi <= kmax && khi <= qlo && klo > qhi - W;
          };
#pragma unroll
          for (int kb = 0; kb < NB; ++kb) {
            if (block_all_visible(kb)) continue;
            int kps[4];
            if constexpr (kFull) {
              // key kk of the tile sits at position kmin + kk, valid up to kmax
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int kpos = kmin + kBlock * kb + 4 * q4 + r;
                kps[r] = (kpos <= kmax && !((no_page_bits >> kb) & 1)) ? kpos : -1;
              }
            } else if (tile < n_hist_tiles) {
              // ring slots: their staged positions (kNoKey where a slot holds none)
              const int4 kp = sm.pos[buf][(sub * kTileBlocks + kb) * 4 + q4];
              kps[0] = kp.x; kps[1] = kp.y; kps[2] = kp.z; kps[3] = kp.w;
            } else {
              // chunk keys: contiguous from kmin, present up to kmax
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int kpos = kmin + kBlock * kb + 4 * q4 + r;
                kps[r] = kpos <= kmax ? kpos : kNoKey;
              }
            }
#pragma unroll
            for (int rg = 0; rg < kRowGroups; ++rg) {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                bool ok;
                if constexpr (kFull) {
                  ok = kps[r] >= 0 && kps[r] <= qpos[rg];
                } else {
                  // in the window: 0 <= qpos - kpos < W, one unsigned compare
                  // (a key after the query wraps to a large distance; kNoKey too)
                  ok = static_cast<uint32_t>(qpos[rg]) - static_cast<uint32_t>(kps[r]) < static_cast<uint32_t>(W);
                }
                s[kb][rg][r] = ok ? s[kb][rg][r] : -INFINITY;
              }
            }
          }
        }
      };
      scores();

      // Probabilities against the current reference m_run, in bf16 for the
      // matrix cores and summed in fp32 for l.
      u32x4 pb[kPairs][kRowGroups];   // P^T for block pairs: B operands of P.V
      float lsum[kRowGroups];
      auto probabilities = [&]() __attribute__((always_inline)) {
        float m_use[kRowGroups];
#pragma unroll
        for (int rg = 0; rg < kRowGroups; ++rg) {
          m_use[rg] = (m_run[rg] == -INFINITY) ? 0.0f : m_run[rg];
          lsum[rg] = 0.0f;
        }
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
          for (int rg = 0; rg < kRowGroups; ++rg) {
            float p[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) p[r] = fast_exp2(s[kb][rg][r] * sl2 - m_use[rg]);
            lsum[rg] += (p[0] + p[1]) + (p[2] + p[3]);
            const uint32_t lo = pack_bf16x2(p[0], p[1]), hi = pack_bf16x2(p[2], p[3]);
            if (kb & 1) {
              pb[kb / 2][rg].z = lo;
              pb[kb / 2][rg].w = hi;
            } else {
              pb[kb / 2][rg].x = lo;
              pb[kb / 2][rg].y = hi;
            }
          }
        }
        if constexpr (NB & 1) {   // the last pair's second block has no keys: P = 0
#pragma unroll
          for (int rg = 0; rg < kRowGroups; ++rg) {
            pb[NB / 2][rg].z = 0u;
            pb[NB / 2][rg].w = 0u;
          }
        }
      };
      // Raise each row's reference to the max of its scores in this tile
      // (a cross-lane reduction) where that is higher, rescaling O and l.
      auto raise_to_row_max = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int rg = 0; rg < kRowGroups; ++rg) {
          float mx = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < NB; ++kb)
            mx = max_prop(mx, max_prop(max_prop(s[kb][rg][0], s[kb][rg][1]), max_prop(s[kb][rg][2], s[kb][rg][3])));
          const float m_new = max_prop(m_run[rg], group4_max(mx) * sl2);
          const float alpha = (m_new == -INFINITY || m_run[rg] == -INFINITY) ? 1.0f : fast_exp2(m_run[rg] - m_new);
          l_run[rg] *= alpha;
#pragma unroll
          for (int d = 0; d < DT; ++d) o[rg][d] *= alpha;
          m_run[rg] = m_new;
        }
      };
      if constexpr (kFull) {
        // The reference only has to keep every probability finite and l
        // away from underflow, not equal the row max. Try the tile against
        // the current reference: while a lane's partial row sum stays at
        // most 2^16, so does every probability of the tile, and the tile is
        // accepted. Otherwise -- and while a row has not seen a key yet, so
        // that its reference is a real score and l >= 1 -- raise the
        // reference to the row max, rescale, and recompute the tile.
        probabilities();
        bool redo = false;
#pragma unroll
        for (int rg = 0; rg < kRowGroups; ++rg) redo = redo || m_run[rg] == -INFINITY || !(lsum[rg] <= kAcceptSum);
        if (__any(redo)) {
          // Rare: the scores are not kept across the first attempt (their
          // registers are reused for the probabilities); recompute them.
          scores();
          raise_to_row_max();
          probabilities();
        }
      } else {
        // A window's few tiles: the row max every tile. The reference is
        // raised (O and l rescaled) only when a row's tile max exceeds it by
        // more than the slack, so probabilities stay at most 2^slack.
        float tmax[kRowGroups];
        bool grow = false;
#pragma unroll
        for (int rg = 0; rg < kRowGroups; ++rg) {
          float mx = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < NB; ++kb)
            mx = max_prop(mx, max_prop(max_prop(s[kb][rg][0], s[kb][rg][1]), max_prop(s[kb][rg][2], s[kb][rg][3])));
          tmax[rg] = group4_max(mx) * sl2;
          grow = grow || (tmax[rg] > m_run[rg] + kRescaleSlack);
        }
        if (!have_ref) {
          // the wave's first tile: O and l are still zero, nothing to rescale
#pragma unroll
          for (int rg = 0; rg < kRowGroups; ++rg) m_run[rg] = max_prop(m_run[rg], tmax[rg]);
          have_ref = true;
        } else if (__any(grow)) {
#pragma unroll
          for (int rg = 0; rg < kRowGroups; ++rg) {
            const float m_new = max_prop(m_run[rg], tmax[rg]);
            const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_run[rg] - m_new);
            l_run[rg] *= alpha;
#pragma unroll
            for (int d = 0; d < DT; ++d) o[rg][d] *= alpha;
            m_run[rg] = m_new;
          }
        }
        probabilities();
      }
#pragma unroll
      for (int rg = 0; rg < kRowGroups; ++rg) l_run[rg] += lsum[rg];

      // P.V on v_mfma_f32_16x16x32_bf16, two 16-key blocks per product: the
      // reduction slots 8q..8q+3 of a lane are keys 4q..4q+3 of block kb,
      // slots 8q+4..8q+7 the same keys of block kb+1, in both operands.
#pragma unroll
      for (int pair = 0; pair < kPairs; ++pair) {
#pragma unroll
        for (int p = 0; p < DT / 2; ++p) {
          const u32x4 v0 = sv[((pair * (DT / 2) + p) * 2 + 0) * 64 + lane];   // dim tile 2p
          const u32x4 v1 = sv[((pair * (DT / 2) + p) * 2 + 1) * 64 + lane];   // dim tile 2p+1
#pragma unroll
          for (int rg = 0; rg < kRowGroups; ++rg) {
            o[rg][2 * p] = mfma_16x16x32(v0, pb[pair][rg], o[rg][2 * p]);
            o[rg][2 * p + 1] = mfma_16x16x32(v1, pb[pair][rg], o[rg][2 * p + 1]);
          }
        }
      }
      // V operand reads run two (dim tile, block pair) steps ahead of their
      // MFMAs: on one MI355X, 3.9% faster full layers than one step ahead,
      // with K operands five reads ahead instead of three.
      constexpr int kVAhead = 2;
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kVAhead, 1);
#pragma unroll
      for (int i = 0; i < (DT / 2) * kPairs - kVAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * kRowGroups, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * kRowGroups * kVAhead, 1);
    };
    if (visible_any) {
      if constexpr (kFull) {
        compute_tile(std::integral_constant<int, kTileBlocks>{});
      } else {
        // ring tiles use all four blocks; a chunk tile only those its keys reach
        const int nb = tile < n_hist_tiles ? kTileBlocks : (kmax - kmin) / kBlock + 1;
        if (nb >= 4) compute_tile(std::integral_constant<int, 4>{});
        else if (nb == 3) compute_tile(std::integral_constant<int, 3>{});
        else if (nb == 2) compute_tile(std::integral_constant<int, 2>{});
        else compute_tile(std::integral_constant<int, 1>{});
      }
    }
    if (sub + 1 < kSubTiles && has_next) {
      // next V phase: this one's loads (and the K loads before them) are done
      __builtin_amdgcn_s_waitcnt(0x0F70);
      store_v(buf ^ 1, sub);
      load_v(sub + 1);
    }
    }   // compute tiles of the stage tile

    if (has_next) {
      store_v(buf ^ 1, kSubTiles - 1);
      store_pos(buf ^ 1);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's direct K loads have landed
    __syncthreads();
  }

  // ---- epilogue: normalise and write rows ----
  if constexpr (lds_epilogue<kFull>()) {
    // Each 16-row group goes through the wave's own LDS slab (the K/V tiles
    // are no longer read: every wave passed the last tile's barrier), so
    // that a store instruction writes two whole rows (2 x D floats,
    // contiguous: consecutive heads of one position) instead of 16 rows x
    // 64 bytes. O is written once and never read here: non-temporal stores.
    constexpr int kPitch = D + 4;                                  // floats per LDS row
    static_assert(kWaves * 16 * kPitch * 4 <= sizeof(sm), "O slabs fit in the tile buffers");
    float* slab = reinterpret_cast<float*>(&sm) + wave * 16 * kPitch;
    // Row rho of the workgroup is O row (tok0 + i0 + (rho >> gsh)) * hq + g * G + (rho & (G - 1)):
    // one 64-bit base per workgroup, a small offset per row.
    float* out_wg = a.out + (static_cast<int64_t>(tok0 + i0) * hq + g * G) * D;
    float* lse_wg = a.lse + static_cast<int64_t>(tok0 + i0) * hq + g * G;
    constexpr int kLanesPerRow = D / 4;                           // 16-byte pieces per row
    constexpr int kRowsPerStore = 64 / kLanesPerRow;              // rows one instruction covers
#pragma unroll
    for (int rg = 0; rg < kRowGroups; ++rg) {
      const float l = group4_sum(l_run[rg]);
      const float inv = __builtin_amdgcn_rcpf(l);
#pragma unroll
      for (int d = 0; d < DT; ++d)
        *reinterpret_cast<f32x4*>(&slab[c16 * kPitch + 16 * d + 4 * q4]) = o[rg][d] * inv;
      {
        const int rho = row0 + 16 * rg + c16;
        const int ci = i0 + (rho >> gsh);
        if (q4 == 0 && ci < i_end) {
          const float mu = (m_run[rg] == -INFINITY) ? 0.0f : m_run[rg];
          lse_wg[(rho >> gsh) * hq + (rho & (G - 1))] = (mu + fast_log2(l)) * kLn2;
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);                          // lgkmcnt(0): the slab is written
#pragma unroll
      for (int j = 0; j < 16 / kRowsPerStore; ++j) {
        const int r = j * kRowsPerStore + lane / kLanesPerRow;     // row of the slab
        const int col = 4 * (lane % kLanesPerRow);
        const f32x4 val = *reinterpret_cast<const f32x4*>(&slab[r * kPitch + col]);
        const int rho = row0 + 16 * rg + r;
        const int ci = i0 + (rho >> gsh);
        if (ci < i_end) {
          const int rel = (rho >> gsh) * hq + (rho & (G - 1));
          __builtin_nontemporal_store(val, reinterpret_cast<f32x4*>(out_wg + static_cast<int64_t>(rel) * D + col));
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);                          // reads done before the slab is rewritten
    }
  } else if (part_entry >= 0) {
    // A split item's partial rows: O normalised by this part's l, and the
    // part's LSE (log2 domain); a row that saw no key here writes O = 0 and
    // LSE = -inf, which the merge weighs as nothing.
    float* po = a.part + static_cast<int64_t>(part_entry) * kRowsPerWg * D;
    float* pl = a.part + static_cast<int64_t>(kPrefillPartEntries) * kRowsPerWg * D +
                static_cast<int64_t>(part_entry) * kRowsPerWg;
#pragma unroll
    for (int rg = 0; rg < kRowGroups; ++rg) {
      const float l = group4_sum(l_run[rg]);
      const int rho = row0 + 16 * rg + c16;
      if (i0 + (rho >> gsh) >= i_end) continue;
      const float inv = l > 0.0f ? __builtin_amdgcn_rcpf(l) : 0.0f;
#pragma unroll
      for (int d = 0; d < DT; ++d)
        *reinterpret_cast<f32x4*>(&po[rho * D + 16 * d + 4 * q4]) = o[rg][d] * inv;
      if (q4 == 0) {
        const float mu = (m_run[rg] == -INFINITY) ? 0.0f : m_run[rg];
        pl[rho] = l > 0.0f ? mu + fast_log2(l) : -INFINITY;
      }
    }
  } else {
#pragma unroll
  for (int rg = 0; rg < kRowGroups; ++rg) {
    const float l = group4_sum(l_run[rg]);
    const int rho = row0 + 16 * rg + c16;
    const int ci = i0 + (rho >> gsh);
    if (ci >= i_end) continue;
    const int hh = g * G + (rho & (G - 1));
    const int64_t row = static_cast<int64_t>(tok0 + ci) * hq + hh;
    const float inv = __builtin_amdgcn_rcpf(l);
#pragma unroll
    for (int d = 0; d < DT; ++d)
      *reinterpret_cast<f32x4*>(&a.out[row * D + 16 * d + 4 * q4]) = o[rg][d] * inv;
    if (q4 == 0) {
      const float mu = (m_run[rg] == -INFINITY) ? 0.0f : m_run[rg];
      a.lse[row] = (mu + fast_log2(l)) * kLn2;
    }
  }
  }
}

// ---- 3. merge of split full-layer items ----
// Workgroup (split item, row group): rows of one split item, one thread per
// 4 channels. With each part's partial O_p (normalised by its own l_p) and
// LSE_p = log2 of its weight, the item's row is O = sum_p 2^(LSE_p - LSE) O_p
// with LSE = log2 sum_p 2^LSE_p, over the parts that hold a key tile (the
// others wrote nothing). Items of one tile were written by their one part.
template <int D>
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefillArgs a) {
  constexpr int kRows = kPrefillFullRows;
  constexpr int kLanesPerRow = D / 4;
  constexpr int kRowsPerBlock = 256 / kLanesPerRow;
  const int n_split = a.split_n1 + a.split_n2;
  const int xcd = blockIdx.x / n_split;
  const int k = blockIdx.x - xcd * n_split;     // split item of the XCD
  const int G = a.geo.group;
  const int hq = a.geo.hq;
  const int gsh = __builtin_ctz(static_cast<unsigned>(G));
  const int QB = kRows >> gsh;
  const int npairs = a.batch * a.geo.hkv;
  const int qb_max = (a.max_new + QB - 1) / QB;
  const int rsh = unit_shift(npairs);
  const int qb_sub = (qb_max + (1 << rsh) - 1) >> rsh;
  const int items = qb_sub * ((npairs << rsh) / kXcds);
  int pair, qblk;
  work_item(items - n_split + k, xcd, qb_max, qb_sub, rsh, pair, qblk);
  if (pair >= npairs || qblk < 0) return;
  const int b = pair / a.geo.hkv;
  const int g = pair - b * a.geo.hkv;
  const int tok0 = a.cu_new[b];
  const int n = min(a.cu_new[b + 1], a.num_tokens) - tok0;
  const int i0 = qblk * QB;
  if (tok0 < 0 || i0 >= n) return;
  const int i_end = min(n, i0 + QB);
  const int n_tiles =
      full_item_tiles(max(a.hist_len[b], 0), i_end, a.table_stride << a.geo.page_shift, stage_keys<true>());
  if (n_tiles <= 1) return;
  const int rho = blockIdx.y * kRowsPerBlock + static_cast<int>(threadIdx.x) / kLanesPerRow;
  const int col = 4 * (static_cast<int>(threadIdx.x) % kLanesPerRow);
  const int ci = i0 + (rho >> gsh);
  if (rho >= kRows || ci >= i_end) return;
  const int parts = split_parts(a, k);
  const int e0 = xcd * kPrefillPartsPerXcd + split_entry(a, k);
  const float* pl = a.part + static_cast<int64_t>(kPrefillPartEntries) * kRows * D;
  auto has_tile = [&](int p) { return p * n_tiles / parts < (p + 1) * n_tiles / parts; };
  float mx = -INFINITY;
  for (int p = 0; p < parts; ++p)
    if (has_tile(p)) mx = fmaxf(mx, pl[(e0 + p) * kRows + rho]);
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  float lse = -INFINITY;
  if (mx != -INFINITY) {
    float wsum = 0.0f;
    for (int p = 0; p < parts; ++p) {
      if (!has_tile(p)) continue;
      const float w = fast_exp2(pl[(e0 + p) * kRows + rho] - mx);
      wsum += w;
      o += *reinterpret_cast<const f32x4*>(a.part + (static_cast<int64_t>(e0 + p) * kRows + rho) * D + col) * w;
    }
    o *= __builtin_amdgcn_rcpf(wsum);
    lse = (mx + fast_log2(wsum)) * kLn2;
  }
  const int64_t row = static_cast<int64_t>(tok0 + ci) * hq + g * G + (rho & (G - 1));
  *reinterpret_cast<f32x4*>(a.out + row * D + col) = o;
  if (col == 0) a.lse[row] = lse;
}

template <int D>
static void launch_prefill_d(const PrefillArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 sgrid((a.max_new + kBlock - 1) / kBlock, a.batch);
  const dim3 bfull(64 * waves_per_wg<true>()), bswa(64 * waves_per_wg<false>());
  if (a.in_f32) {
    hipLaunchKernelGGL((stage_chunk_kernel<D, true>), sgrid, dim3(256), 0, stream, a);
    if (a.full) hipLaunchKernelGGL((prefill_kernel<D, true, true>), grid, bfull, 0, stream, a);
    else hipLaunchKernelGGL((prefill_kernel<D, false, true>), grid, bswa, 0, stream, a);
  } else {
    hipLaunchKernelGGL((stage_chunk_kernel<D, false>), sgrid, dim3(256), 0, stream, a);
    if (a.full) hipLaunchKernelGGL((prefill_kernel<D, true, false>), grid, bfull, 0, stream, a);
    else hipLaunchKernelGGL((prefill_kernel<D, false, false>), grid, bswa, 0, stream, a);
  }
  if (a.full && a.split_n1 + a.split_n2 > 0) {
    const dim3 mgrid(kXcds * (a.split_n1 + a.split_n2), (kPrefillFullRows * (D / 4) + 255) / 256);
    hipLaunchKernelGGL((prefill_merge_kernel<D>), mgrid, dim3(256), 0, stream, a);
  }
}

hipError_t launch_prefill(const PrefillArgs& args, hipStream_t stream) {
  if (args.batch == 0 || args.max_new == 0) return hipSuccess;
  PrefillArgs a = args;
  const int qb = (a.full ? rows_per_wg<true>() : rows_per_wg<false>()) / a.geo.group;
  const int64_t qb_max = (a.max_new + qb - 1) / qb;
  const int64_t npairs = static_cast<int64_t>(a.batch) * a.geo.hkv;
  // Work units as in the kernel: each pair dealt into 8 / gcd(pairs, 8) units.
  int rsh = 3;
  for (int64_t p = npairs; rsh > 0 && (p & 1) == 0; p >>= 1) --rsh;
  const int64_t qb_sub = (qb_max + (int64_t{1} << rsh) - 1) >> rsh;
  const int64_t items = qb_sub * ((npairs << rsh) / kXcds);   // work items per XCD
  a.split_n1 = a.split_p1 = a.split_n2 = a.split_p2 = 0;
  if (a.full && a.part != nullptr) prefill_split_policy(items, &a.split_n1, &a.split_p1, &a.split_n2, &a.split_p2);
  // a split item adds one workgroup per part beyond the first
  const int64_t blocks =
      (items + a.split_n1 * (a.split_p1 - 1) + a.split_n2 * (a.split_p2 - 1)) * kXcds;
  if (blocks > 0x7fffffff || a.batch > 65535) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks));
  if (a.geo.d == 64) launch_prefill_d<64>(a, grid, stream);
  else launch_prefill_d<128>(a, grid, stream);
  return hipGetLastError();
}

}  // namespace ha
