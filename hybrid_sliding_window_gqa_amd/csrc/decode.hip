// a6 / a7 / a8: decode attention over the dual-pool KV cache, with split-K.
//
// Decode reads every visible K/V byte once, so its cost follows the KV bytes
// read (youleyou.com "小米MiMo首次公开模型推理系统全链路优化降价99%",
// section 1 "为什么选择 Hybrid SWA 架构"). SWA layers read only the W-slot
// ring; full layers read all pages of the sequence, split over workgroups
// (split-K) when sequences are long, then merged by decode_reduce_kernel.
//
// Workgroup = 4 wavefronts = one (split, kv head, sequence). Each wave takes
// every fourth 16-token block of the split; for each block it
//   * loads K (16 keys x D, token-major) straight into v_mfma_f32_16x16x32_bf16
//     A operands: lane (q, c) reads key c, channels 32m + 8q .. +7 -- 64
//     contiguous bytes per key row per instruction;
//   * computes S^T = K Q^T (16 keys x 16 query heads of the GQA group; heads
//     beyond the group are zero padding);
//   * runs an exp2-domain online softmax per head: the 4 keys a lane holds
//     plus two cross-lane steps;
//   * loads V^T (dim-major block) straight into v_mfma_f32_16x16x16_bf16 A
//     operands (8 contiguous bytes per lane) and accumulates O^T += V^T P^T,
//     where P^T is the softmax tile in exactly the accumulator layout.
// The next block's operands are loaded before the current one is consumed.
// The four waves merge through LDS; a workgroup writes either the final
// row (one split) or a partial (o, lse) for the reduce kernel.
#include <cmath>

#include "common.hpp"
#include "kernels.hpp"

namespace ha {

namespace {

constexpr int kWaves = 4;

template <int D>
struct BlockOps {
  u32x4 k[D / 32];
  u32x2 v[D / 16];
};

template <int D>
__device__ __forceinline__ void load_block(BlockOps<D>& ops, const uint16_t* kp, const uint16_t* vp,
                                           int64_t base, int q4, int c16) {
#pragma unroll
  for (int m = 0; m < D / 32; ++m)
    ops.k[m] = *reinterpret_cast<const u32x4*>(kp + base + c16 * D + 32 * m + 8 * q4);
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
    ops.v[t] = *reinterpret_cast<const u32x2*>(vp + base + (16 * t + c16) * kBlock + 4 * q4);
}

}  // namespace

template <int D, bool kFull, bool kQF32>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int kPad = 4;
  __shared__ float sm_o[kWaves][16][D + kPad];
  __shared__ float sm_m[kWaves][16];
  __shared__ float sm_l[kWaves][16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q4 = lane >> 4;
  const int c16 = lane & 15;
  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int G = a.geo.group;
  const int hq = a.geo.hq;
  const int hkv = a.geo.hkv;
  const int W = a.geo.window;

  const int len = a.kv_len[b];
  if (len <= 0) {
    if (split == 0) {
      for (int e = threadIdx.x; e < G * D; e += blockDim.x)
        a.out[(static_cast<int64_t>(b) * hq + g * G) * D + e] = 0.0f;
      if (threadIdx.x < G) a.lse[static_cast<int64_t>(b) * hq + g * G + threadIdx.x] = -INFINITY;
    }
    return;
  }
  const int t = len - 1;  // query position

  int first, last, nsplit;
  if constexpr (kFull) {
    // Blocks past the page-table row or past the split grid (kv_len larger
    // than the caller's bounds) are dropped rather than read out of range.
    const int nblk = min((len + kBlock - 1) / kBlock, a.table_stride);
    nsplit = min((nblk + a.split_blocks - 1) / a.split_blocks, a.splits);
    first = split * a.split_blocks;
    last = min(nblk, first + a.split_blocks);
  } else {
    // Ring blocks holding at least one written slot: all of them once t >= W-1.
    const int nrb = (t >= W - 1) ? W / kBlock : (t + kBlock) / kBlock;
    nsplit = 1;
    first = 0;
    last = nrb;
  }
  if (split >= nsplit) return;

  int ring = 0;
  if constexpr (!kFull) {
    ring = a.table[b];
    if (ring < 0 || ring >= a.num_blocks) last = first;  // invalid ring id: no keys
  }
  const int32_t* page_row = a.table + static_cast<int64_t>(b) * a.table_stride;

  auto block_base = [&](int i) -> int64_t {
    if constexpr (kFull) {
      const int pg = page_row[i];
      if (pg < 0 || pg >= a.num_blocks) return -1;
      return (static_cast<int64_t>(pg) * hkv + g) * kBlock * D;
    } else {
      return ((static_cast<int64_t>(ring) * hkv + g) * W + kBlock * i) * D;
    }
  };

  // Q^T as the B operand: column c16 = query head g*G + c16 (zero past the group).
  u32x4 qop[KS];
  {
    const bool head_ok = c16 < G;
    const int64_t qoff = (static_cast<int64_t>(b) * hq + g * G + (head_ok ? c16 : 0)) * D + 8 * q4;
#pragma unroll
    for (int m = 0; m < KS; ++m) {
      qop[m] = load8_as_bf16<kQF32>(a.q, qoff + 32 * m);
      if (!head_ok) qop[m] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  const float sl2 = a.geo.scale * kLog2e;
  float m_run = -INFINITY;  // running max of this head (log2 domain), same in all lane groups
  float l_run = 0.0f;       // partial sum over this lane's keys
  f32x4 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  int i = first + wave;
  int64_t base_cur = (i < last) ? block_base(i) : -1;
  int64_t base_nxt = (i + kWaves < last) ? block_base(i + kWaves) : -1;
  BlockOps<D> cur, nxt;
  if (base_cur >= 0) load_block<D>(cur, a.k_pool, a.v_pool, base_cur, q4, c16);

  for (; i < last; i += kWaves) {
    if (base_nxt >= 0) load_block<D>(nxt, a.k_pool, a.v_pool, base_nxt, q4, c16);
    const int64_t base_nn = (i + 2 * kWaves < last) ? block_base(i + 2 * kWaves) : -1;

    if (base_cur >= 0) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < KS; ++m) s = mfma_16x16x32(cur.k[m], qop[m], s);

      // Keys this lane holds: 4*q4 + r of block i.
      bool partial;
      if constexpr (kFull) partial = (kBlock * i + kBlock - 1 > t);
      else partial = (t < W - 1) && (kBlock * i + kBlock - 1 > t);
      if (partial) {
        uint32_t keep[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kBlock * i + 4 * q4 + r;  // position (full) or slot (ring, t < W-1)
          const bool ok = key <= t;
          keep[r] = ok ? 0xffffu : 0u;
          if (!ok) s[r] = -INFINITY;
        }
        const uint32_t mlo = keep[0] | (keep[1] << 16);
        const uint32_t mhi = keep[2] | (keep[3] << 16);
#pragma unroll
        for (int d = 0; d < DT; ++d) {
          cur.v[d].x &= mlo;
          cur.v[d].y &= mhi;
        }
      }

      const float tmax = group4_max(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]))) * sl2;
      const float m_new = fmaxf(m_run, tmax);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = fast_exp2(s[r] * sl2 - m_use);
      l_run = l_run * alpha + (p[0] + p[1]) + (p[2] + p[3]);
      m_run = m_new;
#pragma unroll
      for (int d = 0; d < DT; ++d) o[d] *= alpha;
      const u32x2 pb = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
#pragma unroll
      for (int d = 0; d < DT; ++d) o[d] = mfma_16x16x16(cur.v[d], pb, o[d]);
    }
    cur = nxt;
    base_cur = base_nxt;
    base_nxt = base_nn;
  }

  // Merge the four waves.
  l_run = group4_sum(l_run);
#pragma unroll
  for (int d = 0; d < DT; ++d)
    *reinterpret_cast<f32x4*>(&sm_o[wave][c16][16 * d + 4 * q4]) = o[d];
  if (q4 == 0) {
    sm_m[wave][c16] = m_run;
    sm_l[wave][c16] = l_run;
  }
  __syncthreads();

  const bool final_row = (nsplit == 1);
  for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
    const int h = e / D;
    const int dd = e - h * D;
    float mx = sm_m[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, sm_m[w][h]);
    const float mu = (mx == -INFINITY) ? 0.0f : mx;
    float l = 0.0f, acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(sm_m[w][h] - mu);
      l += sm_l[w][h] * f;
      acc += sm_o[w][h][dd] * f;
    }
    const int64_t row = static_cast<int64_t>(b) * hq + g * G + h;
    const float lse2 = mu + fast_log2(l);
    if (final_row) {
      a.out[row * D + dd] = acc / l;
      if (dd == 0) a.lse[row] = lse2 * kLn2;
    } else {
      a.part_o[(row * a.splits + split) * D + dd] = acc / l;
      if (dd == 0) a.part_lse[row * a.splits + split] = lse2;
    }
  }
}

// a8: lse = log2 sum_s 2^lse_s; o = sum_s 2^(lse_s - lse) o_s (log2 domain),
// written back in natural-log units. One workgroup per (query head, sequence).
template <int D>
__global__ __launch_bounds__(64) void decode_reduce_kernel(DecodeArgs a) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int len = a.kv_len[b];
  if (len <= 0) return;
  const int nblk = min((len + kBlock - 1) / kBlock, a.table_stride);
  const int nsplit = min((nblk + a.split_blocks - 1) / a.split_blocks, a.splits);
  if (nsplit <= 1) return;
  const int64_t row = static_cast<int64_t>(b) * a.geo.hq + h;
  const float* pl = a.part_lse + row * a.splits;
  float mx = -INFINITY;
  for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, pl[s]);
  const float mu = (mx == -INFINITY) ? 0.0f : mx;
  float l = 0.0f;
  for (int s = 0; s < nsplit; ++s) l += fast_exp2(pl[s] - mu);
  const float inv = 1.0f / l;
  const float* po = a.part_o + row * a.splits * D;
  for (int dd = threadIdx.x; dd < D; dd += 64) {
    float acc = 0.0f;
    for (int s = 0; s < nsplit; ++s) acc += fast_exp2(pl[s] - mu) * po[static_cast<int64_t>(s) * D + dd];
    a.out[row * D + dd] = acc * inv;
  }
  if (threadIdx.x == 0) a.lse[row] = (mu + fast_log2(l)) * kLn2;
}

int decode_split_blocks(bool full, int window, int max_kv_len, int batch, int hkv, int requested_splits) {
  if (!full) return window / kBlock;
  const int nblk = (max(max_kv_len, 1) + kBlock - 1) / kBlock;
  if (requested_splits > 0) return max(1, (nblk + requested_splits - 1) / requested_splits);
  // Aim for a few thousand workgroups overall, 4..16 blocks per wave.
  const int64_t total = static_cast<int64_t>(nblk) * max(batch, 1) * max(hkv, 1);
  int64_t sb = (total + 4095) / 4096;
  sb = sb < 16 ? 16 : (sb > 64 ? 64 : sb);
  return static_cast<int>(sb);
}

int decode_num_splits(bool full, int window, int max_kv_len, int split_blocks) {
  if (!full) return 1;
  const int nblk = (max(max_kv_len, 1) + kBlock - 1) / kBlock;
  return (nblk + split_blocks - 1) / split_blocks;
}

template <int D>
static hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.full ? a.splits : 1, a.geo.hkv, a.batch);
  const dim3 block(256);
  if (a.full) {
    if (a.q_f32) hipLaunchKernelGGL((decode_kernel<D, true, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((decode_kernel<D, true, false>), grid, block, 0, stream, a);
  } else {
    if (a.q_f32) hipLaunchKernelGGL((decode_kernel<D, false, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((decode_kernel<D, false, false>), grid, block, 0, stream, a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (a.full && a.splits > 1) {
    hipLaunchKernelGGL(decode_reduce_kernel<D>, dim3(a.geo.hq, a.batch), dim3(64), 0, stream, a);
    err = hipGetLastError();
  }
  return err;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  return a.geo.d == 64 ? launch_decode_d<64>(a, stream) : launch_decode_d<128>(a, stream);
}

}  // namespace ha
