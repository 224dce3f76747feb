// a4 / a5: causal prefill attention over the dual-pool KV cache.
//
// A chunk of new tokens per sequence attends to the sequence's history in the
// pool (the SWA ring's last W-1 positions, or every page of the Full pool)
// and causally to the chunk itself, read from k_new / v_new. SWA layers cut
// the attended range from the whole sequence to the window (youleyou.com
// "小米MiMo首次公开模型推理系统全链路优化降价99%", section 1
// "为什么选择 Hybrid SWA 架构"); chunked prefill is what the serving stack runs
// for long requests (blog.hotdry.top 2026-06-09, section "PD 分离与长度分桶").
//
// Workgroup = 4 wavefronts = 128 rows of one (sequence, kv head), where a row
// is a (query position, query head of the GQA group) pair: the whole group
// shares every K/V tile, so K/V are read once per group instead of once per
// query head. Each wave owns 32 rows (two 16-row MFMA column groups).
// Keys stream in 64-key tiles (four 16-token blocks) staged in LDS with two
// buffers: the next tile's global loads are in flight while the current tile
// is consumed.
//   K tile   [64 keys][D]   padded rows -> conflict-free 16-byte A-operand reads
//   V^T tile [4][D][16]     dim-major blocks, rows padded to 40 bytes ->
//                           conflict-free 8-byte A-operand reads
// Per tile and wave: S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (Q^T held in
// registers), exp2-domain online softmax per row (in-lane over 16 scores plus
// two cross-lane steps), P^T cast to bf16 in the accumulator layout, then
// O^T += V^T P^T with v_mfma_f32_16x16x16_bf16. Tiles that every row of a
// wave sees completely skip the masking; tiles no row of the wave sees are
// skipped.
//
// Grid order: workgroup i runs on XCD i % 8 (round-robin dispatch). All query
// blocks of one (sequence, kv head) pair are placed on the same XCD, so the
// pair's K/V stream is shared through that XCD's L2, and the heaviest
// (latest) query blocks are dispatched first.
#include <cmath>

#include "common.hpp"
#include "kernels.hpp"

namespace ha {

namespace {

constexpr int kRowsPerWave = 32;
constexpr int kRowGroups = kRowsPerWave / 16;
constexpr int kWaves = 4;
constexpr int kRowsPerWg = kRowsPerWave * kWaves;  // 128
constexpr int kTileKeys = 64;
constexpr int kTileBlocks = kTileKeys / kBlock;   // 4
constexpr int kVRow = 20;                          // bf16 per padded V^T row (40 bytes)
constexpr int kXcds = 8;

template <int D>
struct Smem {
  static constexpr int kKRow = D + 8;  // bf16 per padded K row
  uint16_t k[2][kTileKeys * kKRow];
  uint16_t v[2][kTileBlocks * D * kVRow];
  int32_t pos[2][kTileKeys];
};

// Per-thread staging registers for one tile: D/32 16-byte chunks of K and of V.
template <int D>
struct Stage {
  u32x4 k[D / 32];
  u32x4 v[D / 32];
};

// Zero all but the first `nv` of the 8 bfloat16 values in `v` (nv may be <0 or >8).
__device__ __forceinline__ u32x4 keep_first_bf16(u32x4 v, int nv) {
  if (nv >= 8) return v;
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = (2 * j < nv) ? 0x0000ffffu : 0u;
    const uint32_t hi = (2 * j + 1 < nv) ? 0xffff0000u : 0u;
    w[j] &= lo | hi;
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

}  // namespace

template <int D, bool kFull, bool kF32>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
  constexpr int KS = D / 32;            // QK^T reduction steps
  constexpr int DT = D / 16;            // output dim tiles
  constexpr int CPR = D / 8;            // 16-byte chunks per key row
  constexpr int CPT = D / 32;           // chunks per thread per tile (K and V each)
  constexpr int KROW = Smem<D>::kKRow;
  __shared__ Smem<D> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4;
  const int c16 = lane & 15;

  const int hkv = a.geo.hkv;
  const int hq = a.geo.hq;
  const int G = a.geo.group;
  const int W = a.geo.window;
  const int QB = kRowsPerWg / G;        // query positions per workgroup

  // ---- workgroup -> (sequence, kv head, query block), XCD-aware ----
  const int npairs = a.batch * hkv;
  const int ppx = (npairs + kXcds - 1) / kXcds;   // pairs per XCD
  const int qb_max = (a.max_new + QB - 1) / QB;
  const int lin = blockIdx.x;
  const int xcd = lin % kXcds;
  const int j = lin / kXcds;
  const int pair = (j % ppx) * kXcds + xcd;
  const int qblk = qb_max - 1 - j / ppx;
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

  // ---- tile list: history tiles, then chunk tiles ----
  int n_hist_tiles = 0;
  int ring = -1;
  const int32_t* page_row = a.table + static_cast<int64_t>(b) * a.table_stride;
  if constexpr (kFull) {
    const int nblk = (hist + kBlock - 1) / kBlock;
    n_hist_tiles = (nblk + kTileBlocks - 1) / kTileBlocks;
    // loads below also require the logical block to lie inside the page-table row
  } else {
    ring = a.table[b];
    const bool ring_ok = ring >= 0 && ring < a.num_blocks;
    if (ring_ok && hist > 0 && t_first - W + 1 < hist) n_hist_tiles = (W + kTileKeys - 1) / kTileKeys;
  }
  int c_lo = 0;
  if constexpr (!kFull) c_lo = max(0, i0 - W + 1);
  const int first_ctile = c_lo / kTileKeys;
  const int n_chunk_tiles = (i_end + kTileKeys - 1) / kTileKeys - first_ctile;
  const int n_tiles = n_hist_tiles + n_chunk_tiles;

  // ---- rows of this wave ----
  const int row0 = wave * kRowsPerWave;
  const int wave_i_lo = i0 + row0 / G;
  const int wave_i_hi = min(i_end - 1, i0 + (row0 + kRowsPerWave - 1) / G);
  const bool wave_live = wave_i_lo < i_end;
  const int qlo = hist + wave_i_lo;
  const int qhi = hist + wave_i_hi;

  // Q^T operands and per-row query positions.
  u32x4 qop[kRowGroups][KS];
  int qpos[kRowGroups];
#pragma unroll
  for (int rg = 0; rg < kRowGroups; ++rg) {
    const int rho = row0 + 16 * rg + c16;
    const int ci = i0 + rho / G;
    const int hh = g * G + rho % G;
    const bool ok = ci < i_end;
    qpos[rg] = hist + ci;
    const int64_t off = (static_cast<int64_t>(tok0 + (ok ? ci : 0)) * hq + hh) * D + 8 * q4;
#pragma unroll
    for (int m = 0; m < KS; ++m) {
      qop[rg][m] = ok ? load8_as_bf16<kF32>(a.q, off + 32 * m) : u32x4{0u, 0u, 0u, 0u};
    }
  }

  // ---- tile loading ----
  // Global -> registers for tile `tile`, and the key positions (threads < 64).
  auto key_position = [&](int tile, int kk) -> int {
    if (tile < n_hist_tiles) {
      if constexpr (kFull) {
        const int p = tile * kTileKeys + kk;
        return p < hist ? p : -1;
      } else {
        const int s = tile * kTileKeys + kk;              // ring slot
        if (s >= W) return -1;
        const int last = hist - 1;
        int d = (last - s) % W;
        if (d < 0) d += W;
        const int p = last - d;
        return p >= 0 ? p : -1;
      }
    } else {
      const int ci = (first_ctile + tile - n_hist_tiles) * kTileKeys + kk;
      return (ci < i_end) ? hist + ci : -1;
    }
  };

  auto load_tile = [&](int tile, Stage<D>& st, int& mypos) {
    if (tile < n_hist_tiles) {
      // K: chunk e -> key e / CPR, column e % CPR; V^T: chunk e -> block, dim row, half.
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const int e = tid + 256 * u;
        {
          const int key = e / CPR;
          const int col = e - key * CPR;
          const int blk = key >> 4;
          const int kin = key & 15;
          int64_t base = -1;
          if constexpr (kFull) {
            const int lb = tile * kTileBlocks + blk;
            if (lb * kBlock + kin < hist && lb < a.table_stride) {
              const int pg = page_row[lb];
              if (pg >= 0 && pg < a.num_blocks) base = (static_cast<int64_t>(pg) * hkv + g) * kBlock * D;
            }
          } else {
            const int rb = tile * kTileBlocks + blk;
            if (rb * kBlock < W) base = ((static_cast<int64_t>(ring) * hkv + g) * W + kBlock * rb) * D;
          }
          st.k[u] = base >= 0 ? *reinterpret_cast<const u32x4*>(a.k_pool + base + kin * D + col * 8)
                              : u32x4{0u, 0u, 0u, 0u};
        }
        {
          const int blk = e / (2 * D);
          const int rem = e - blk * 2 * D;
          const int row = rem >> 1;
          const int half = rem & 1;
          int64_t base = -1;
          int first_key, limit;  // the chunk's 8 keys are valid while first_key + j < limit
          if constexpr (kFull) {
            const int lb = tile * kTileBlocks + blk;
            first_key = lb * kBlock + half * 8;
            limit = hist;
            if (lb * kBlock < hist && lb < a.table_stride) {
              const int pg = page_row[lb];
              if (pg >= 0 && pg < a.num_blocks) base = (static_cast<int64_t>(pg) * hkv + g) * kBlock * D;
            }
          } else {
            const int rb = tile * kTileBlocks + blk;
            first_key = rb * kBlock + half * 8;          // ring slot; slots >= hist unwritten while hist < W
            limit = hist >= W ? W : hist;
            if (rb * kBlock < W) base = ((static_cast<int64_t>(ring) * hkv + g) * W + kBlock * rb) * D;
          }
          st.v[u] = base >= 0 ? *reinterpret_cast<const u32x4*>(a.v_pool + base + row * kBlock + half * 8)
                              : u32x4{0u, 0u, 0u, 0u};
          st.v[u] = keep_first_bf16(st.v[u], limit - first_key);
        }
      }
    } else {
      const int cbase = (first_ctile + tile - n_hist_tiles) * kTileKeys;
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const int e = tid + 256 * u;
        const int key = e / CPR;
        const int col = e - key * CPR;
        const int ci = cbase + key;
        if (ci < i_end) {
          const int64_t off = (static_cast<int64_t>(tok0 + ci) * hkv + g) * D + col * 8;
          st.k[u] = load8_as_bf16<kF32>(a.k_new, off);
          st.v[u] = load8_as_bf16<kF32>(a.v_new, off);
        } else {
          st.k[u] = u32x4{0u, 0u, 0u, 0u};
          st.v[u] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
    if (tid < kTileKeys) mypos = key_position(tile, tid);
  };

  // Registers -> LDS buffer `buf`. History V is already dim-major; chunk V is
  // transposed here. Keys with an invalid position hold zeros in K and V, so
  // masked probabilities never multiply stale data.
  auto store_tile = [&](int tile, const Stage<D>& st, int mypos, int buf) {
    const bool hist_tile = tile < n_hist_tiles;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int e = tid + 256 * u;
      const int key = e / CPR;
      const int col = e - key * CPR;
      *reinterpret_cast<u32x4*>(&sm.k[buf][key * KROW + col * 8]) = st.k[u];
      if (hist_tile) {
        const int blk = e / (2 * D);
        const int rem = e - blk * 2 * D;
        const int row = rem >> 1;
        const int half = rem & 1;
        uint16_t* dst = &sm.v[buf][(blk * D + row) * kVRow + half * 8];
        reinterpret_cast<u32x2*>(dst)[0] = u32x2{st.v[u].x, st.v[u].y};
        reinterpret_cast<u32x2*>(dst)[1] = u32x2{st.v[u].z, st.v[u].w};
      } else {
        const int blk = key >> 4;
        const int kin = key & 15;
        uint16_t* dst = &sm.v[buf][(blk * D + col * 8) * kVRow + kin];
        const uint32_t w4[4] = {st.v[u].x, st.v[u].y, st.v[u].z, st.v[u].w};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          dst[(2 * jj) * kVRow] = static_cast<uint16_t>(w4[jj] & 0xffffu);
          dst[(2 * jj + 1) * kVRow] = static_cast<uint16_t>(w4[jj] >> 16);
        }
      }
    }
    if (tid < kTileKeys) sm.pos[buf][tid] = mypos;
  };

  // Key-position bounds of a tile (uniform): [kmin, kmax], all_valid.
  auto tile_bounds = [&](int tile, int& kmin, int& kmax, bool& all_valid, bool& contiguous) {
    if (tile < n_hist_tiles) {
      if constexpr (kFull) {
        kmin = tile * kTileKeys;
        kmax = min(kmin + kTileKeys, hist) - 1;
        all_valid = kmin + kTileKeys <= hist;
        contiguous = true;
      } else {
        kmin = max(0, hist - W);
        kmax = hist - 1;
        all_valid = false;
        contiguous = false;
      }
    } else {
      const int c0 = (first_ctile + tile - n_hist_tiles) * kTileKeys;
      kmin = hist + c0;
      kmax = hist + min(c0 + kTileKeys, i_end) - 1;
      all_valid = c0 + kTileKeys <= i_end;
      contiguous = true;
    }
  };

  // ---- main loop ----
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

  Stage<D> stage;
  int mypos = -1;
  if (n_tiles > 0) {
    load_tile(0, stage, mypos);
    store_tile(0, stage, mypos, 0);
  }
  __syncthreads();

  for (int tile = 0; tile < n_tiles; ++tile) {
    const int buf = tile & 1;
    const bool has_next = tile + 1 < n_tiles;
    if (has_next) load_tile(tile + 1, stage, mypos);

    int kmin, kmax;
    bool all_valid, contiguous;
    tile_bounds(tile, kmin, kmax, all_valid, contiguous);
    bool visible_any = wave_live && kmin <= qhi;
    if constexpr (!kFull) visible_any = visible_any && kmax >= qlo - W + 1;
    bool need_mask = !(all_valid && contiguous && kmax <= qlo);
    if constexpr (!kFull) need_mask = need_mask || kmin < qhi - W + 1;

    if (visible_any) {
      const uint16_t* sk = sm.k[buf];
      const uint16_t* sv = sm.v[buf];
      f32x4 s[kTileBlocks][kRowGroups];
#pragma unroll
      for (int kb = 0; kb < kTileBlocks; ++kb) {
#pragma unroll
        for (int rg = 0; rg < kRowGroups; ++rg) s[kb][rg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < KS; ++m) {
          const u32x4 kop = *reinterpret_cast<const u32x4*>(&sk[(16 * kb + c16) * KROW + 32 * m + 8 * q4]);
#pragma unroll
          for (int rg = 0; rg < kRowGroups; ++rg) s[kb][rg] = mfma_16x16x32(kop, qop[rg][m], s[kb][rg]);
        }
      }

      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < kTileBlocks; ++kb) {
          const int4 kp = *reinterpret_cast<const int4*>(&sm.pos[buf][16 * kb + 4 * q4]);
          const int kps[4] = {kp.x, kp.y, kp.z, kp.w};
#pragma unroll
          for (int rg = 0; rg < kRowGroups; ++rg) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              bool ok = kps[r] >= 0 && kps[r] <= qpos[rg];
              if constexpr (!kFull) ok = ok && kps[r] > qpos[rg] - W;
              if (!ok) s[kb][rg][r] = -INFINITY;
            }
          }
        }
      }

      u32x2 pb[kTileBlocks][kRowGroups];
#pragma unroll
      for (int rg = 0; rg < kRowGroups; ++rg) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < kTileBlocks; ++kb)
          mx = fmaxf(mx, fmaxf(fmaxf(s[kb][rg][0], s[kb][rg][1]), fmaxf(s[kb][rg][2], s[kb][rg][3])));
        const float tmax = group4_max(mx) * sl2;
        const float m_new = fmaxf(m_run[rg], tmax);
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        const float alpha = fast_exp2(m_run[rg] - m_use);
        float lsum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < kTileBlocks; ++kb) {
          float p[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) p[r] = fast_exp2(s[kb][rg][r] * sl2 - m_use);
          lsum += (p[0] + p[1]) + (p[2] + p[3]);
          pb[kb][rg] = u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
        }
        l_run[rg] = l_run[rg] * alpha + lsum;
        m_run[rg] = m_new;
#pragma unroll
        for (int d = 0; d < DT; ++d) o[rg][d] *= alpha;
      }

#pragma unroll
      for (int d = 0; d < DT; ++d) {
#pragma unroll
        for (int kb = 0; kb < kTileBlocks; ++kb) {
          const u32x2 vop = *reinterpret_cast<const u32x2*>(&sv[(kb * D + 16 * d + c16) * kVRow + 4 * q4]);
#pragma unroll
          for (int rg = 0; rg < kRowGroups; ++rg) o[rg][d] = mfma_16x16x16(vop, pb[kb][rg], o[rg][d]);
        }
      }
    }

    if (has_next) store_tile(tile + 1, stage, mypos, buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise and write rows ----
#pragma unroll
  for (int rg = 0; rg < kRowGroups; ++rg) {
    const float l = group4_sum(l_run[rg]);
    const int rho = row0 + 16 * rg + c16;
    const int ci = i0 + rho / G;
    if (ci >= i_end) continue;
    const int hh = g * G + rho % G;
    const int64_t row = static_cast<int64_t>(tok0 + ci) * hq + hh;
    const float inv = 1.0f / l;
#pragma unroll
    for (int d = 0; d < DT; ++d)
      *reinterpret_cast<f32x4*>(&a.out[row * D + 16 * d + 4 * q4]) = o[rg][d] * inv;
    if (q4 == 0) {
      const float mu = (m_run[rg] == -INFINITY) ? 0.0f : m_run[rg];
      a.lse[row] = (mu + fast_log2(l)) * kLn2;
    }
  }
}

template <int D, bool kFull>
static void launch_prefill_dk(const PrefillArgs& a, dim3 grid, hipStream_t stream) {
  if (a.in_f32)
    hipLaunchKernelGGL((prefill_kernel<D, kFull, true>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<D, kFull, false>), grid, dim3(256), 0, stream, a);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.batch == 0 || a.max_new == 0) return hipSuccess;
  const int qb = kRowsPerWg / a.geo.group;
  const int64_t qb_max = (a.max_new + qb - 1) / qb;
  const int64_t npairs = static_cast<int64_t>(a.batch) * a.geo.hkv;
  const int64_t ppx = (npairs + kXcds - 1) / kXcds;
  const int64_t blocks = qb_max * ppx * kXcds;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks));
  if (a.geo.d == 64) {
    if (a.full) launch_prefill_dk<64, true>(a, grid, stream);
    else launch_prefill_dk<64, false>(a, grid, stream);
  } else {
    if (a.full) launch_prefill_dk<128, true>(a, grid, stream);
    else launch_prefill_dk<128, false>(a, grid, stream);
  }
  return hipGetLastError();
}

}  // namespace ha
