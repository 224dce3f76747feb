// a6 / a7 / a8: decode attention over the dual-pool KV cache, with split-K.
//
// Decode reads every visible K/V byte once, so its cost follows the KV bytes
// read (youleyou.com "小米MiMo首次公开模型推理系统全链路优化降价99%",
// section 1 "为什么选择 Hybrid SWA 架构"). SWA layers read only the W-slot
// ring; full layers read all pages of the sequence, split over workgroups
// (split-K) when sequences are long, then merged by decode_reduce_kernel.
//
// Workgroup = one (split, kv head, sequence): 4 wavefronts for full layers,
// 8 for SWA layers (one ring block per wave, so a W = 128 ring is fetched in
// a single round trip; one operand buffer per wave keeps the SWA kernel at
// 128 VGPRs, so two workgroups share a CU and a whole decode batch runs as a
// single round of workgroups). Wave w takes blocks w, w+NW, w+2NW, ... of the split
// and keeps two of them in flight in ping-pong register buffers (no register
// copies, so a block's loads are only waited for right before it is
// consumed). For each 16-token block it
//   * loads K straight into v_mfma_f32_16x16x32_bf16 A operands (lane (q, c):
//     key c, channels 32m + 8q .. +7); the pools keep blocks in operand
//     order, so each load instruction reads 1 KiB contiguous;
//   * computes S^T = K Q^T (16 keys x 16 query heads of the GQA group; heads
//     beyond the group are zero padding);
//   * runs an exp2-domain online softmax per head: the 4 keys a lane holds
//     plus two cross-lane steps;
//   * loads V^T straight into v_mfma_f32_16x16x16_bf16 A operands (16 bytes
//     per lane = two dim tiles, again 1 KiB contiguous per instruction) and
//     accumulates O^T += V^T P^T, where P^T is the softmax tile in exactly the
//     accumulator layout.
// INT8 pools (include/hybrid_attn.h) take half the bytes per block: the
// raw codes and the block's scales are what the ping-pong buffers hold. In
// full layers the K codes go to the int8 matrix cores as loaded, against Q
// split into three int8 parts per head; V codes (and the K codes of SWA
// layers) are widened to the same bf16 operands the bf16 path loads right
// before the block is consumed (codes are exact in bf16). The K scale
// multiplies the scores and the V scale is folded into the probabilities. A fused append quantizes the token in
// the owning wave with append8_kernel's arithmetic (absmax butterflies over
// the lanes that hold the K row and the V row) and patches codes and scales
// into the raw operands.
// Page ids are scalar loads issued two blocks ahead of their use. The waves
// merge through LDS; a workgroup writes either the final row (one split) or a
// partial (o, lse) for the reduce kernel.
//
// Fused append. When the caller passes the new token's K/V (k_new/v_new), the
// pool does not hold position t yet: the wave that consumes the block of
// position t patches the token's K row and V column into its operand
// registers after the block's load, and after consuming the block writes the
// token into the pool (ring slot t mod W, or the page of t at its token). No
// other workgroup reads that slot in this launch, so the result equals
// append-then-decode with one launch instead of two.
#include <climits>
#include <cmath>
#include <mutex>

#include "../../include/hybrid_attn.h"
#include "common.hpp"
#include "kernels.hpp"

namespace ha {

namespace {

template <bool kFull>
constexpr int waves_per_wg() { return kFull ? 4 : 8; }

template <int D>
struct BlockOps {
  u32x4 k[D / 32];
  u32x2 v[D / 16];
};

// Loads one block's K and V^T operands; base < 0 loads zeros without traffic.
template <int D>
__device__ __forceinline__ void load_block(BlockOps<D>& ops, const uint16_t* kp, const uint16_t* vp,
                                           int64_t base, int q4, int c16) {
  const bool ok = base >= 0;
  const int64_t b0 = ok ? base : 0;
  const uint32_t bytes = ok ? kBlock * D * 2 : 0;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kp + b0, bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vp + b0, bytes);
  const int lane = 16 * q4 + c16;
#pragma unroll
  for (int m = 0; m < D / 32; ++m) ops.k[m] = buf_load16_stream(rk, 16 * (64 * m + lane));
#pragma unroll
  for (int p = 0; p < D / 32; ++p) {
    const u32x4 w = buf_load16_stream(rv, 16 * (64 * p + lane));
    ops.v[2 * p] = u32x2{w.x, w.y};
    ops.v[2 * p + 1] = u32x2{w.z, w.w};
  }
}

// One 16-token block: scores, masking of keys past index `t` (the last
// position or ring slot that holds a key; when `partial`), online-softmax
// update and the P.V accumulation.
template <int D>
__device__ __forceinline__ void consume_block(BlockOps<D>& ops, const u32x4* qop, int first_key, int t,
                                              bool partial, float sl2, float& m_run, float& l_run, f32x4* o,
                                              int q4) {
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < KS; ++m) s = mfma_16x16x32(ops.k[m], qop[m], s);
  if (partial) {
    uint32_t keep[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = first_key + 4 * q4 + r <= t;
      keep[r] = ok ? 0xffffu : 0u;
      s[r] = ok ? s[r] : -INFINITY;
    }
    const uint32_t mlo = keep[0] | (keep[1] << 16);
    const uint32_t mhi = keep[2] | (keep[3] << 16);
#pragma unroll
    for (int d = 0; d < DT; ++d) {
      ops.v[d].x &= mlo;
      ops.v[d].y &= mhi;
    }
  }
  const float tmax = group4_max(max_prop(max_prop(s[0], s[1]), max_prop(s[2], s[3]))) * sl2;
  const float m_new = max_prop(m_run, tmax);
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
  for (int d = 0; d < DT; ++d) o[d] = mfma_16x16x16(ops.v[d], pb, o[d]);
}

// Slack of the INT8 path's exp2 reference (log2 units); see consume_block8.
constexpr float kDecodeSlack = 8.0f;

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 mfma_i8_16x16x64(const u32x4& a, const u32x4& b, const i32x4& c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0,
                                               0);
}

// INT8 pools: Q^T as operands of the int8 matrix cores, so the K codes are
// multiplied as they are loaded, with no widening. Each head's query row
// (the bf16 values the bf16 path uses) is split into kQParts int8 parts
// against a per-head step sq = amax / 127: q = sq * (c0 + c1 / 254 +
// c2 / 254^2) up to sq / (2 * 254^2), about amax * 6e-8. The integer
// products are exact. Two parts (about amax * 1.5e-5) are not enough: the
// error of a score grows with |k|, and keys 40 times the typical size then
// moved LSE by 2.5e-3. In lane (q4, c16), the operand of 64-channel group j
// holds the channels of bf16 operands 2j (bytes 0-7) and 2j + 1 (bytes 8-15),
// the byte order of the pool's K units; part p goes to q8[p * D/64 + j].
// Returns sq (1 for a zero row, such as the heads past the group; NaN for a
// NaN row, which then reaches the row's output).
constexpr int kQParts = 3;
template <int D>
__device__ __forceinline__ float split_q8(const u32x4* qop, u32x4* q8) {
  constexpr int KS = D / 32;
  float x[KS][8];
  float amax = 0.0f;
#pragma unroll
  for (int m = 0; m < KS; ++m) {
    const uint32_t w4[4] = {qop[m].x, qop[m].y, qop[m].z, qop[m].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[m][2 * j] = __uint_as_float(w4[j] << 16);
      x[m][2 * j + 1] = __uint_as_float(w4[j] & 0xffff0000u);
      amax = max_prop(amax, max_prop(fabsf(x[m][2 * j]), fabsf(x[m][2 * j + 1])));
    }
  }
  amax = max_prop(amax, __shfl_xor(amax, 16));   // the 4 lanes of column c16
  amax = max_prop(amax, __shfl_xor(amax, 32));
  const float sq = (amax == 0.0f) ? 1.0f : amax / 127.0f;
  const float inv = 1.0f / sq;
#pragma unroll
  for (int j = 0; j < D / 64; ++j) {
    uint32_t c[kQParts][4] = {};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float r = x[2 * j + (e >> 3)][e & 7];
      float step = sq, inv_step = inv;
#pragma unroll
      for (int p = 0; p < kQParts; ++p) {
        const float cv = fminf(fmaxf(rintf(r * inv_step), -127.0f), 127.0f);
        r = fmaf(-cv, step, r);
        step *= 1.0f / 254.0f;
        inv_step *= 254.0f;
        c[p][e >> 2] |= (static_cast<uint32_t>(static_cast<int>(cv)) & 0xffu) << (8 * (e & 3));
      }
    }
#pragma unroll
    for (int p = 0; p < kQParts; ++p) q8[p * (D / 64) + j] = u32x4{c[p][0], c[p][1], c[p][2], c[p][3]};
  }
  return sq;
}

// consume_block for INT8 pools: score = k_scale * (q . code) -- with kI8, the
// dot product on the int8 matrix cores as sq * sum_p (c_p . code) / 254^p
// (split_q8; qop then holds the split operands and sl2 already carries sq),
// otherwise on the bf16 ones with the codes widened --, and the V scale of
// each key multiplies its probability (P'V = P (scale * code)); l keeps the
// unscaled probabilities. Masked keys get a zero V scale so an unwritten
// slot's scale cannot reach O. P' goes to the matrix cores in two bf16 parts
// (pv8); the 32-deep product takes the cycles of the 16-deep one.
template <int D, bool kI8>
__device__ __forceinline__ void consume_block8(const RawBlock8<D>& raw, const u32x4* qop, int first_key, int t,
                                               bool partial, float sl2, float& m_run, float& l_run, f32x4* o,
                                               int q4) {
  constexpr int DT = D / 16;
  BlockOps<D> ops;
  widen_v8<D>(raw, ops.v);
  f32x4 s;
  if constexpr (kI8) {
    i32x4 sp[kQParts];
#pragma unroll
    for (int p = 0; p < kQParts; ++p) {
      sp[p] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < D / 64; ++j) sp[p] = mfma_i8_16x16x64(raw.k[j], qop[p * (D / 64) + j], sp[p]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float acc = static_cast<float>(sp[kQParts - 1][r]);
#pragma unroll
      for (int p = kQParts - 2; p >= 0; --p) acc = fmaf(acc, 1.0f / 254.0f, static_cast<float>(sp[p][r]));
      s[r] = acc * raw.ks[r];
    }
  } else {
    widen_k8<D>(raw, ops.k);
    s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < D / 32; ++m) s = mfma_16x16x32(ops.k[m], qop[m], s);
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] *= raw.ks[r];
  }
  float vs[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) vs[r] = raw.vs[r];
  if (partial) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = first_key + 4 * q4 + r <= t;
      s[r] = ok ? s[r] : -INFINITY;
      vs[r] = ok ? vs[r] : 0.0f;
    }
  }
  // The exp2 reference m_run is raised only when a column's block max exceeds
  // it by more than kDecodeSlack (log2 units), so probabilities stay at most
  // 2^kDecodeSlack and O and l are rescaled only on those blocks, not on
  // every block: the widening already makes this path the vector-heavier one.
  const float tmax = group4_max(max_prop(max_prop(s[0], s[1]), max_prop(s[2], s[3]))) * sl2;
  if (__any(tmax > m_run + kDecodeSlack)) {
    const float m_new = (tmax > m_run + kDecodeSlack) ? tmax : m_run;
    const float alpha = (m_new == m_run) ? 1.0f : (m_run == -INFINITY ? 0.0f : fast_exp2(m_run - m_new));
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < DT; ++d) o[d] *= alpha;
    m_run = m_new;
  }
  const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
  float p[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) p[r] = fast_exp2(s[r] * sl2 - m_use);
  l_run += (p[0] + p[1]) + (p[2] + p[3]);
  float pv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) pv[r] = p[r] * vs[r];
  pv8<D>(ops.v, pv, o);
}

// One block's operands in the pool's format.
template <int D, bool kKv8>
struct BlockBuf;
template <int D>
struct BlockBuf<D, false> {
  BlockOps<D> ops;
};
template <int D>
struct BlockBuf<D, true> {
  RawBlock8<D> raw;
};

template <int D, bool kKv8>
__device__ __forceinline__ void load_buf(BlockBuf<D, kKv8>& b, const DecodeArgs& a, int64_t base, int q4, int c16) {
  if constexpr (kKv8) load_block8<D>(b.raw, a.k_pool, a.v_pool, a.k_scale, a.v_scale, base, 16 * q4 + c16);
  else load_block<D>(b.ops, a.k_pool, a.v_pool, base, q4, c16);
}

template <int D, bool kKv8, bool kI8>
__device__ __forceinline__ void consume_buf(BlockBuf<D, kKv8>& b, const u32x4* qop, int first_key, int t,
                                            bool partial, float sl2, float& m_run, float& l_run, f32x4* o, int q4) {
  if constexpr (kKv8) consume_block8<D, kI8>(b.raw, qop, first_key, t, partial, sl2, m_run, l_run, o, q4);
  else consume_block<D>(b.ops, qop, first_key, t, partial, sl2, m_run, l_run, o, q4);
}

// Replace 16-bit element r (0..3) of a u32x2 holding four bf16 values.
__device__ __forceinline__ void set_bf16(u32x2& w, int r, uint32_t bits) {
  const uint32_t shift = (r & 1) * 16;
  const uint32_t keep = ~(0xffffu << shift);
  if (r < 2) w.x = (w.x & keep) | (bits << shift);
  else w.y = (w.y & keep) | (bits << shift);
}

template <bool kF32>
__device__ __forceinline__ uint32_t load_bf16_bits(const void* src, int64_t elem) {
  if constexpr (kF32) return f32_to_bf16_bits(static_cast<const float*>(src)[elem]);
  else return static_cast<const uint16_t*>(src)[elem];
}

// INT8 pools: the new token's codes in the raw operand format (K: the units
// of lanes c16 == row; V: byte dt%4 of word dt/4 holds dim tile dt's code of
// this lane's channel) and its two scales.
template <int D>
struct NewToken8 {
  u32x4 k[D / 64];
  uint32_t v[D / 64];
  float ks;
  float vs;
};


// The new token's operand pieces for the wave that owns its block: K chunk
// (m, q4) of the token row (used by lanes c16 == row) and the V values of
// channels 32p + c16 and 32p + 16 + c16 (used by lanes q4 == row / 4).
template <int D>
struct NewToken {
  u32x4 k[D / 32];
  uint32_t v[D / 16];
};

}  // namespace

template <int D, bool kFull, bool kQF32, bool kKv8>
__global__ __launch_bounds__(64 * waves_per_wg<kFull>(), kFull ? 3 : 4) void decode_kernel(DecodeArgs a) {
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int kPad = 4;
  constexpr int kWaves = waves_per_wg<kFull>();
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
  // The SWA ring id is read beside the length, so the two scalar loads share
  // one memory round trip before the first K/V load can be addressed.
  const int ring_id = kFull ? 0 : a.table[b];
  // Compiler-only: keeps the ring-id load, and the argument loads of the
  // pointers the first Q and K/V loads need, above the branch below, where
  // the compiler would otherwise sink them (and their waits) past the length
  // check, one dependent round trip each.
  if constexpr (!kFull) asm volatile("" ::"s"(ring_id), "s"(a.q), "s"(a.k_pool), "s"(a.v_pool));
  if (len <= 0) {
    if (split == 0) {
      for (int e = threadIdx.x; e < G * D; e += blockDim.x)
        a.out[(static_cast<int64_t>(b) * hq + g * G) * D + e] = 0.0f;
      if (threadIdx.x < G) a.lse[static_cast<int64_t>(b) * hq + g * G + threadIdx.x] = -INFINITY;
    }
    return;
  }
  const int t = len - 1;  // query position
  // Last pool index holding a key: position t (full), or ring slot
  // min(t, W - 1) (slots past W - 1 of the last ring block hold none).
  const int key_last = kFull ? t : min(t, W - 1);

  int first, last, nsplit;
  if constexpr (kFull) {
    // Blocks past the page-table row or past the split grid (kv_len larger
    // than the caller's bounds) are dropped rather than read out of range.
    const int nblk = min((len + kBlock - 1) / kBlock, a.table_stride << a.geo.page_shift);
    nsplit = min((nblk + a.split_blocks - 1) / a.split_blocks, a.splits);
    first = split * a.split_blocks;
    last = min(nblk, first + a.split_blocks);
  } else {
    // Ring blocks holding at least one written slot: all of them once
    // t >= W-1 (the last one partly, when W is not a multiple of 16).
    const int nrb = (t >= W - 1) ? a.geo.ring / kBlock : (t + kBlock) / kBlock;
    nsplit = 1;
    first = 0;
    last = nrb;
  }
  if (split >= nsplit) return;

  const int ring = ring_id;
  if constexpr (!kFull) {
    if (ring < 0 || ring >= a.num_blocks) last = first;  // invalid ring id: no keys
  }
  const int32_t* page_row = a.table + static_cast<int64_t>(b) * a.table_stride;

  // Page id of block `i` and element offset of its K/V (-1: nothing to read).
  const int psh = a.geo.page_shift;
  auto page_of = [&](int i) -> int { return (i < last) ? page_row[i >> psh] : -1; };
  auto base_of = [&](int i, int pg) -> int64_t {
    if constexpr (kFull) {
      if (i >= last || pg < 0 || pg >= a.num_blocks) return -1;
      return page_block_offset(pg, g, hkv, i & ((1 << psh) - 1), psh, kBlock * D);
    } else {
      if (i >= last) return -1;
      return ((static_cast<int64_t>(ring) * hkv + g) * a.geo.ring + kBlock * i) * D;
    }
  };
  auto is_partial = [&](int i) -> bool {
    if constexpr (kFull) return kBlock * i + kBlock - 1 > t;
    else return kBlock * i + kBlock - 1 > key_last;
  };

  // Q^T as the B operand: column c16 = query head g*G + c16 (zero past the group).
  u32x4 qop[KS];
  if constexpr (kQF32) {
    const bool head_ok = c16 < G;
    const int64_t qoff = (static_cast<int64_t>(b) * hq + g * G + (head_ok ? c16 : 0)) * D + 8 * q4;
#pragma unroll
    for (int m = 0; m < KS; ++m) {
      qop[m] = load8_as_bf16<kQF32>(a.q, qoff + 32 * m);
      if (!head_ok) qop[m] = u32x4{0u, 0u, 0u, 0u};
    }
  } else {
    load_q_rows<D>(qop, a.q, static_cast<int64_t>(b) * hq + g * G, G, q4, c16);
  }

  // Fused append: block of position t, its row in the block, and whether
  // this wave consumes that block.
  const bool fuse = a.k_new != nullptr;
  const int new_slot = kFull ? t : t % W;
  const int new_blk = new_slot >> 4;
  const int new_row = new_slot & (kBlock - 1);
  const bool new_mine = fuse && new_blk >= first && new_blk < last && (new_blk - first) % kWaves == wave;
  NewToken<D> nt;
  NewToken8<D> n8;
  if constexpr (kKv8) {
    // Quantize the token as append8_kernel does: the 4 lanes of a c16
    // column hold the K row (channels 32m + 8*q4 + j), the 16 lanes of a q4
    // row hold the V row (channel 16*dt + c16 for dim tile dt).
    if (new_mine) {
      const int64_t src = (static_cast<int64_t>(b) * hkv + g) * D;
      float kx[KS][8];
      float ka = 0.0f;
#pragma unroll
      for (int m = 0; m < KS; ++m) {
        const u32x4 w = load8_as_bf16<kQF32>(a.k_new, src + 32 * m + 8 * q4);
        const uint32_t w4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kx[m][2 * j] = __uint_as_float(w4[j] << 16);
          kx[m][2 * j + 1] = __uint_as_float(w4[j] & 0xffff0000u);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) ka = max_prop(ka, fabsf(kx[m][j]));
      }
      ka = max_prop(ka, __shfl_xor(ka, 16));
      ka = max_prop(ka, __shfl_xor(ka, 32));
      float vx[DT];
      float va = 0.0f;
#pragma unroll
      for (int p = 0; p < D / 32; ++p) {
        vx[2 * p] = __uint_as_float(load_bf16_bits<kQF32>(a.v_new, src + 32 * p + c16) << 16);
        vx[2 * p + 1] = __uint_as_float(load_bf16_bits<kQF32>(a.v_new, src + 32 * p + 16 + c16) << 16);
        va = max_prop(va, max_prop(fabsf(vx[2 * p]), fabsf(vx[2 * p + 1])));
      }
#pragma unroll
      for (int mask = 1; mask < 16; mask <<= 1) va = max_prop(va, __shfl_xor(va, mask));
      n8.ks = ka / 127.0f;
      n8.vs = va / 127.0f;
#pragma unroll
      for (int j = 0; j < D / 64; ++j) {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 16; ++e) w[e >> 2] |= code8(kx[2 * j + (e >> 3)][e & 7], n8.ks) << (8 * (e & 3));
        n8.k[j] = u32x4{w[0], w[1], w[2], w[3]};
        n8.v[j] = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) n8.v[j] |= code8(vx[4 * j + e], n8.vs) << (8 * e);
      }
    }
  } else if (new_mine) {
    const int64_t src = (static_cast<int64_t>(b) * hkv + g) * D;
#pragma unroll
    for (int m = 0; m < KS; ++m) nt.k[m] = load8_as_bf16<kQF32>(a.k_new, src + 32 * m + 8 * q4);
#pragma unroll
    for (int p = 0; p < D / 32; ++p) {
      nt.v[2 * p] = load_bf16_bits<kQF32>(a.v_new, src + 32 * p + c16);
      nt.v[2 * p + 1] = load_bf16_bits<kQF32>(a.v_new, src + 32 * p + 16 + c16);
    }
  }
  auto patch_new = [&](BlockBuf<D, kKv8>& buf, int i) {
    if (!new_mine || i != new_blk) return;
    if constexpr (kKv8) {
      RawBlock8<D>& raw = buf.raw;
      if (c16 == new_row) {
#pragma unroll
        for (int j = 0; j < D / 64; ++j) raw.k[j] = n8.k[j];
      }
      if (q4 == (new_row >> 2)) {
        const uint32_t sh = 8 * (new_row & 3);
        const uint32_t keep = ~(0xffu << sh);
#pragma unroll
        for (int j = 0; j < D / 64; ++j) {
          raw.v[j].x = (raw.v[j].x & keep) | ((n8.v[j] & 0xffu) << sh);
          raw.v[j].y = (raw.v[j].y & keep) | (((n8.v[j] >> 8) & 0xffu) << sh);
          raw.v[j].z = (raw.v[j].z & keep) | (((n8.v[j] >> 16) & 0xffu) << sh);
          raw.v[j].w = (raw.v[j].w & keep) | ((n8.v[j] >> 24) << sh);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (r == (new_row & 3)) {
            raw.ks[r] = n8.ks;
            raw.vs[r] = n8.vs;
          }
        }
      }
    } else {
    BlockOps<D>& ops = buf.ops;
    if (c16 == new_row) {
#pragma unroll
      for (int m = 0; m < KS; ++m) ops.k[m] = nt.k[m];
    }
    if (q4 == (new_row >> 2)) {
#pragma unroll
      for (int d = 0; d < DT; ++d) set_bf16(ops.v[d], new_row & 3, nt.v[d]);
    }
    }
  };

  const float sl2 = a.geo.scale * kLog2e;
  // INT8 full layers: Q split for the int8 matrix cores (split_q8), its step
  // folded into the scale of this lane's head; done once the first blocks'
  // loads are in flight. An SWA wave consumes one block, too few to repay
  // the split: it widens its K codes instead.
  constexpr bool kI8 = kKv8 && kFull;
  u32x4 q8[kQParts * (D / 64)];
  float sl2k = sl2;
  const u32x4* qk = kI8 ? q8 : qop;
  float m_run = -INFINITY;  // running max of this head (log2 domain), same in all lane groups
  float l_run = 0.0f;       // partial sum over this lane's keys
  f32x4 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Fused append: the owner wave writes the token into the pool, after its
  // block has been read and consumed. (Issued right after the patch instead,
  // the stores made the SWA call about 1 us slower.)
  auto store_new = [&]() {
    if (kKv8 && new_mine) {
      const int64_t nb = base_of(new_blk, kFull ? page_row[new_blk >> psh] : 0);
      if (nb >= 0) {
        uint8_t* kb = reinterpret_cast<uint8_t*>(a.k_pool_w) + nb;
        uint8_t* vb = reinterpret_cast<uint8_t*>(a.v_pool_w) + nb;
        if (c16 == new_row) {
#pragma unroll
          for (int j = 0; j < D / 64; ++j) *reinterpret_cast<u32x4*>(kb + 16 * (64 * j + lane)) = n8.k[j];
        }
        if (q4 == (new_row >> 2)) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            vb[v8_elem(new_row, 16 * dt + c16)] = static_cast<uint8_t>((n8.v[dt >> 2] >> (8 * (dt & 3))) & 0xffu);
        }
        if (lane == 0) {
          a.k_scale[nb / D + new_row] = n8.ks;
          a.v_scale[nb / D + new_row] = n8.vs;
        }
      }
    } else if (new_mine) {
      const int64_t nb = base_of(new_blk, kFull ? page_row[new_blk >> psh] : 0);
      if (nb >= 0) {
        if (c16 == new_row) {
#pragma unroll
          for (int m = 0; m < KS; ++m)
            *reinterpret_cast<u32x4*>(a.k_pool_w + nb + 8 * (64 * m + lane)) = nt.k[m];
        }
        if (q4 == (new_row >> 2)) {
          uint16_t* vb = a.v_pool_w + nb;
#pragma unroll
          for (int p = 0; p < D / 32; ++p) {
            vb[v_elem(new_row, 32 * p + c16)] = static_cast<uint16_t>(nt.v[2 * p]);
            vb[v_elem(new_row, 32 * p + 16 + c16)] = static_cast<uint16_t>(nt.v[2 * p + 1]);
          }
        }
      }
    }
  };

  if constexpr (!kFull) {
    // SWA: with W <= 16 * waves (W = 128: one ring block per wave) every
    // wave has at most one block; a larger ring is walked a block at a
    // time. A single operand buffer keeps the kernel at 128 VGPRs, so two
    // 8-wave workgroups fit on a CU and the whole grid runs in one round.
    BlockBuf<D, kKv8> A;
    if (last - first <= kWaves) {
      const int i = first + wave;
      if (i < last) {
        load_buf<D, kKv8>(A, a, base_of(i, 0), q4, c16);
        patch_new(A, i);
        consume_buf<D, kKv8, kI8>(A, qk, kBlock * i, key_last, is_partial(i), sl2k, m_run, l_run, o, q4);
      }
    } else {
      for (int i = first + wave; i < last; i += kWaves) {
        load_buf<D, kKv8>(A, a, base_of(i, 0), q4, c16);
        patch_new(A, i);
        consume_buf<D, kKv8, kI8>(A, qk, kBlock * i, key_last, is_partial(i), sl2k, m_run, l_run, o, q4);
      }
    }
  } else {
    // Full: blocks of this wave are first + wave + 4k. Buffer A holds even k,
    // B odd k.
    constexpr int kStep = kWaves;
    int ia = first + wave;
    int ib = ia + kStep;
    int pg_a = page_of(ia), pg_b = page_of(ib);
    int64_t base_a = base_of(ia, pg_a);
    int64_t base_b = base_of(ib, pg_b);
    BlockBuf<D, kKv8> A, B;
    load_buf<D, kKv8>(A, a, base_a, q4, c16);
    load_buf<D, kKv8>(B, a, base_b, q4, c16);
    if constexpr (kI8) sl2k = sl2 * split_q8<D>(qop, q8);
    int pg_a2 = page_of(ia + 2 * kStep), pg_b2 = page_of(ib + 2 * kStep);
    // Pairs (A, B) in a loop with a fixed trip count and no early exit, so the
    // loads in flight at the loop head are the same on every path; an odd last
    // block is consumed from A after the loop. Loads past `last` read nothing.
    const int nmine = (last > ia) ? (last - ia + kStep - 1) / kStep : 0;
    for (int k = 0; k + 1 < nmine; k += 2) {
      patch_new(A, ia);
      if (base_a >= 0) consume_buf<D, kKv8, kI8>(A, qk, kBlock * ia, t, is_partial(ia), sl2k, m_run, l_run, o, q4);
      ia += 2 * kStep;
      base_a = base_of(ia, pg_a2);
      load_buf<D, kKv8>(A, a, base_a, q4, c16);
      pg_a2 = page_of(ia + 2 * kStep);
      patch_new(B, ib);
      if (base_b >= 0) consume_buf<D, kKv8, kI8>(B, qk, kBlock * ib, t, is_partial(ib), sl2k, m_run, l_run, o, q4);
      ib += 2 * kStep;
      base_b = base_of(ib, pg_b2);
      load_buf<D, kKv8>(B, a, base_b, q4, c16);
      pg_b2 = page_of(ib + 2 * kStep);
    }
    if (nmine & 1) {
      patch_new(A, ia);
      if (base_a >= 0) consume_buf<D, kKv8, kI8>(A, qk, kBlock * ia, t, is_partial(ia), sl2k, m_run, l_run, o, q4);
    }
  }

  store_new();

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
  // Each thread folds channels of one head, so that head's wave factors and
  // l are computed once per thread, not once per channel. G and the thread
  // count are powers of two, so the threads split evenly over the heads.
  const int tph_shift = __builtin_ctz(static_cast<unsigned>(64 * kWaves)) - __builtin_ctz(static_cast<unsigned>(G));
  const int h = static_cast<int>(threadIdx.x) >> tph_shift;
  const int t_in_head = static_cast<int>(threadIdx.x) - (h << tph_shift);
  float mx = sm_m[0][h];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) mx = max_prop(mx, sm_m[w][h]);
  const float mu = (mx == -INFINITY) ? 0.0f : mx;
  float f[kWaves];
  float l = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    f[w] = fast_exp2(sm_m[w][h] - mu);
    l += sm_l[w][h] * f[w];
  }
  const int64_t row = static_cast<int64_t>(b) * hq + g * G + h;
  const float lse2 = mu + fast_log2(l);
  for (int dd = t_in_head; dd < D; dd += 1 << tph_shift) {
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) acc += sm_o[w][h][dd] * f[w];
    if (final_row) {
      // l = 0: no valid key (an invalid ring id, or no valid page): O = 0, LSE = -inf
      a.out[row * D + dd] = l > 0.0f ? acc / l : 0.0f;
      if (dd == 0) a.lse[row] = lse2 * kLn2;
    } else {
      a.part_o[(row * a.splits + split) * D + dd] = acc / l;
      if (dd == 0) a.part_lse[row * a.splits + split] = lse2;
    }
  }
}

// a8: lse = log2 sum_s 2^lse_s; o = sum_s 2^(lse_s - lse) o_s (log2 domain),
// written back in natural-log units. One thread per output element (row,
// channel); the splits are folded with a running max so every split's lse
// and o load is issued up front (one memory round trip for typical counts).
// A split that saw no key (lse_s = -inf) contributes nothing.
template <int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs a) {
  const int b = blockIdx.y;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;  // element of the sequence's Hq*D outputs
  if (e >= a.geo.hq * D) return;
  const int len = a.kv_len[b];
  if (len <= 0) return;
  const int nblk = min((len + kBlock - 1) / kBlock, a.table_stride << a.geo.page_shift);
  const int nsplit = min((nblk + a.split_blocks - 1) / a.split_blocks, a.splits);
  if (nsplit <= 1) return;
  const int h = e / D;
  const int dd = e - h * D;
  const int64_t row = static_cast<int64_t>(b) * a.geo.hq + h;
  const float* pl = a.part_lse + row * a.splits;
  const float* po = a.part_o + row * a.splits * D + dd;
  float m = -INFINITY, l = 0.0f, acc = 0.0f;
#pragma unroll 4
  for (int s = 0; s < nsplit; ++s) {
    const float ls = pl[s];
    const float os = po[static_cast<int64_t>(s) * D];
    const float mn = max_prop(m, ls);
    const float mu = (mn == -INFINITY) ? 0.0f : mn;
    const float f = fast_exp2(m - mu);
    const float w = fast_exp2(ls - mu);
    l = l * f + w;
    acc = acc * f + (w > 0.0f ? w * os : 0.0f);
    m = mn;
  }
  a.out[row * D + dd] = l > 0.0f ? acc / l : 0.0f;
  if (dd == 0) a.lse[row] = ((m == -INFINITY ? 0.0f : m) + fast_log2(l)) * kLn2;
}

template <int D>
static hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.full ? a.splits : 1, a.geo.hkv, a.batch);
  if (a.full) {
    const dim3 block(64 * waves_per_wg<true>());
    if (a.kv8) {
      if (a.q_f32) hipLaunchKernelGGL((decode_kernel<D, true, true, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((decode_kernel<D, true, false, true>), grid, block, 0, stream, a);
    } else if (a.q_f32) {
      hipLaunchKernelGGL((decode_kernel<D, true, true, false>), grid, block, 0, stream, a);
    } else {
      hipLaunchKernelGGL((decode_kernel<D, true, false, false>), grid, block, 0, stream, a);
    }
  } else {
    const dim3 block(64 * waves_per_wg<false>());
    if (a.kv8) {
      if (a.q_f32) hipLaunchKernelGGL((decode_kernel<D, false, true, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((decode_kernel<D, false, false, true>), grid, block, 0, stream, a);
    } else if (a.q_f32) {
      hipLaunchKernelGGL((decode_kernel<D, false, true, false>), grid, block, 0, stream, a);
    } else {
      hipLaunchKernelGGL((decode_kernel<D, false, false, false>), grid, block, 0, stream, a);
    }
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (a.full && a.splits > 1) {
    const unsigned per_seq = static_cast<unsigned>((a.geo.hq * D + 255) / 256);
    hipLaunchKernelGGL(decode_reduce_kernel<D>, dim3(per_seq, a.batch), dim3(256), 0, stream, a);
    err = hipGetLastError();
  }
  return err;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  return a.geo.d == 64 ? launch_decode_d<64>(a, stream) : launch_decode_d<128>(a, stream);
}

// Split-K partials of hybrid_attn_decode_noalloc: one library-owned array per
// device, loaded with the code object and kept until the process ends. Every
// call on a device shares it, so calls that overlap on one device race.
// Nothing in it has to start at zero: every split a merge reads is written
// by its workgroup in the same call.
static __device__ __align__(256) unsigned char scratch[HA_DECODE_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device (with that device current) and
// only that address is handed to kernels.
hipError_t decode_scratch(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace ha

