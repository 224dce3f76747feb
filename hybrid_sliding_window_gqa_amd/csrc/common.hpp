// Device-side helpers shared by the hybrid attention kernels (gfx950 / CDNA4).
//
// Matrix-core conventions used throughout (64-lane wavefront, lane l,
// q = l / 16 "lane group", c = l % 16):
//   v_mfma_f32_16x16x32_bf16  A[16 x 32]: lane holds A[c][8q .. 8q+7]
//                             B[32 x 16]: lane holds B[8q .. 8q+7][c]
//   v_mfma_f32_16x16x16_bf16  A[16 x 16]: lane holds A[c][4q .. 4q+3]
//                             B[16 x 16]: lane holds B[4q .. 4q+3][c]
//   accumulator C[16 x 16]:   lane holds C[4q + r][c], r = 0..3
// Any relabelling of the reduction index applied to A and B alike leaves the
// product unchanged, which the kernels use to load operands with long
// contiguous runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ha {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 16;         // tokens per page / ring block

// In-block layout of the pools (and of the prefill staging blocks): a block
// of 16 tokens x D channels of one kv head is 16*D bfloat16 stored as 16-byte
// units in matrix-core operand order, so a wavefront loads an operand set
// with one fully contiguous 1 KiB read per instruction.
//   K unit (m, q, c) = m*64 + q*16 + c  holds K[token c][32m + 8q .. +7]
//   V unit (p, q, c) = p*64 + q*16 + c  holds V[tokens 4q..4q+3][32p + c]
//                                         then V[tokens 4q..4q+3][32p + 16 + c]
// Lane l = 16q + c of a wave reads unit (., q, c): for K that is the
// v_mfma_f32_16x16x32_bf16 A operand of S^T = K Q^T, for V the two
// v_mfma_f32_16x16x16_bf16 A operands (dim tiles 2p, 2p+1) of O^T = V^T P^T.
__host__ __device__ constexpr int64_t k_elem(int token, int dim) {
  return (static_cast<int64_t>(dim / 32) * 64 + ((dim % 32) / 8) * 16 + token) * 8 + dim % 8;
}
__host__ __device__ constexpr int64_t v_elem(int token, int dim) {
  return (static_cast<int64_t>(dim / 32) * 64 + (token / 4) * 16 + dim % 16) * 8 + ((dim % 32) / 16) * 4 + token % 4;
}
// INT8 pools: one byte per value, 16-byte units. A K unit holds a lane's
// 8-channel chunks of two consecutive 32-channel slices (MFMA A operands m and
// m+1); a V unit holds a lane's 4 tokens of four 16-channel dim tiles.
__host__ __device__ constexpr int64_t k8_elem(int token, int dim) {
  return (static_cast<int64_t>(dim / 64) * 64 + ((dim % 32) / 8) * 16 + token) * 16 + ((dim / 32) % 2) * 8 + dim % 8;
}
__host__ __device__ constexpr int64_t v8_elem(int token, int dim) {
  return (static_cast<int64_t>(dim / 64) * 64 + (token / 4) * 16 + dim % 16) * 16 + ((dim / 16) % 4) * 4 + token % 4;
}

// Four signed 8-bit codes (one word) -> four bfloat16 values (two words, code
// 0 in bits 0..15 of the first). |code| <= 127 fits bf16's 8-bit significand,
// so dropping the low half of the float32 is exact.
__device__ __forceinline__ u32x2 i8x4_to_bf16x4(uint32_t w) {
  const float f0 = static_cast<float>(static_cast<int8_t>(w & 0xffu));
  const float f1 = static_cast<float>(static_cast<int8_t>((w >> 8) & 0xffu));
  const float f2 = static_cast<float>(static_cast<int8_t>((w >> 16) & 0xffu));
  const float f3 = static_cast<float>(static_cast<int8_t>(w >> 24));
  return u32x2{__builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u),
               __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u)};
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x4 mfma_16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_16x16x16(const u32x2& a, const u32x2& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// Element offset of 16-token block `sub` of page `pg`, kv head g, in a Full
// pool whose pages hold 1 << page_shift blocks per kv head
// ([pages][Hkv][1 << page_shift][block_elems]).
__device__ __forceinline__ int64_t page_block_offset(int pg, int g, int hkv, int sub, int page_shift,
                                                     int block_elems) {
  return ((((static_cast<int64_t>(pg) * hkv + g) << page_shift) + sub) * block_elems);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even float -> bfloat16 (hardware conversion on gfx950).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b));
}

// Two floats -> two round-to-nearest-even bfloat16 in one word (lo in bits
// 0..15): a single two-operand v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  const f32x2v f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v));
}

// 16 bytes holding 8 bfloat16 values loaded from `src` (bf16 or f32 storage).
template <bool kF32>
__device__ __forceinline__ u32x4 load8_as_bf16(const void* src, int64_t elem_off) {
  if constexpr (kF32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(src) + elem_off);
    float4 a = p[0], b = p[1];
    u32x4 r;
    r.x = pack_bf16x2(a.x, a.y);
    r.y = pack_bf16x2(a.z, a.w);
    r.z = pack_bf16x2(b.x, b.y);
    r.w = pack_bf16x2(b.z, b.w);
    return r;
  } else {
    return *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + elem_off);
  }
}

// The same for rows read once per launch (a chunk's new K/V when it is
// staged or appended): bf16 sources use non-temporal loads, which on one
// MI355X cut the chunk staging kernel from 55 to 44 us per 8192-token chunk.
template <bool kF32>
__device__ __forceinline__ u32x4 load8_as_bf16_stream(const void* src, int64_t elem_off) {
  if constexpr (kF32) return load8_as_bf16<true>(src, elem_off);
  else return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + elem_off));
}

// Raw buffer access (gfx9 descriptor word 3 = 0x00020000). A descriptor with
// num_records = 0 makes every lane out of range: the load returns zeros and
// issues no memory traffic, so invalid blocks need no branch around the load
// and the count of outstanding loads stays the same on every path.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
// Streaming variant for bytes read once per launch (decode's K/V): the
// cache-policy operand sets the non-temporal bit (bit 1 on gfx950), so the
// lines are not kept in the caches at the expense of reused data. On one
// MI355X a read of decode's pattern (4 KiB K and V chunks at page-table
// positions) moves 6.7 TB/s this way against 6.0 TB/s with the default
// policy.
__device__ __forceinline__ u32x4 buf_load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 2));
}
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0));
}

// Query rows [row0, row0 + nrows) of a bf16 [rows][D] array as matrix-core
// B operands: lane (q4, c16) gets row row0 + c16, channels 32m + 8 q4 .. +7.
// Lanes with c16 >= nrows read past the buffer's end and get zeros from the
// range check, so no select on the loaded value has to wait for the load
// before the loads that follow it are issued.
template <int D>
__device__ __forceinline__ void load_q_rows(u32x4 (&qop)[D / 32], const void* q, int64_t row0, int nrows,
                                            int q4, int c16) {
  const __amdgpu_buffer_rsrc_t r =
      make_rsrc(static_cast<const uint16_t*>(q) + row0 * D, static_cast<uint32_t>(nrows) * D * 2);
  const uint32_t off = c16 < nrows ? 2u * static_cast<uint32_t>(c16 * D + 8 * q4) : 0x40000000u;
#pragma unroll
  for (int m = 0; m < D / 32; ++m) qop[m] = buf_load16(r, off + 64 * m);
}

// Float maximum that propagates NaN (the IEEE 754-2019 maximum): gfx950 has
// it natively (v_maximum3_f32, three operands), and unlike fmaxf it needs no
// NaN-quieting copy of each operand when NaNs are honoured. A NaN score, e.g.
// from a stray read of poisoned memory, reaches the row's maximum and so its
// output.
__device__ __forceinline__ float max_prop(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// gfx950 lane swaps, one VALU instruction each:
//   permlane32_swap: lanes 32..63 of a <-> lanes 0..31 of b;
//   permlane16_swap: the odd 16-lane rows of a <-> the even rows of b.
// Called with a == b, they leave a = the low half (rows 0, 2) duplicated
// and b = the high half (rows 1, 3) duplicated, so op(a, b) combines lanes
// l and l^32 (resp. l^16) in every lane. Written as inline asm on two
// registers: the compiler's builtin folds the two results into one when
// both operands are the same value, which is wrong for this instruction.
// The leading s_nop covers the VALU-write -> permlane-read hazard.
__device__ __forceinline__ void permlane32_swap(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void permlane16_swap(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// Max / sum over the four lane groups (lanes c, c+16, c+32, c+48), the same
// value in all of them.
__device__ __forceinline__ float group4_max(float v) {
  float a = v, b = v;
  permlane32_swap(a, b);
  v = max_prop(a, b);
  a = v;
  b = v;
  permlane16_swap(a, b);
  return max_prop(a, b);
}
__device__ __forceinline__ float group4_sum(float v) {
  float a = v, b = v;
  permlane32_swap(a, b);
  v = a + b;
  a = v;
  b = v;
  permlane16_swap(a, b);
  return a + b;
}

// ---- INT8 pool blocks (decode and verify) ----
// The raw 16-byte units of one block as a lane (q4, c16) loads them (K: D/64
// units holding two 32-channel slices each; V: D/64 units holding four
// 16-channel tiles each) and the 4 K and 4 V scales of the lane's keys
// 4*q4 .. 4*q4+3.
template <int D>
struct RawBlock8 {
  u32x4 k[D / 64];
  u32x4 v[D / 64];
  f32x4 ks;
  f32x4 vs;
};

// Loads one INT8 block at element offset `base` of the code pools (the
// scales of its 16 tokens at base / D); base < 0 loads zeros without traffic.
template <int D>
__device__ __forceinline__ void load_block8(RawBlock8<D>& raw, const void* k_pool, const void* v_pool,
                                            const float* k_scale, const float* v_scale, int64_t base, int lane) {
  const bool ok = base >= 0;
  const int64_t b0 = ok ? base : 0;
  const uint32_t bytes = ok ? kBlock * D : 0;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<const uint8_t*>(k_pool) + b0, bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(static_cast<const uint8_t*>(v_pool) + b0, bytes);
#pragma unroll
  for (int j = 0; j < D / 64; ++j) {
    raw.k[j] = buf_load16_stream(rk, 16 * (64 * j + lane));
    raw.v[j] = buf_load16_stream(rv, 16 * (64 * j + lane));
  }
  const uint32_t sbytes = ok ? kBlock * 4 : 0;
  const __amdgpu_buffer_rsrc_t rks = make_rsrc(k_scale + b0 / D, sbytes);
  const __amdgpu_buffer_rsrc_t rvs = make_rsrc(v_scale + b0 / D, sbytes);
  raw.ks = __builtin_bit_cast(f32x4, buf_load16_stream(rks, 16 * (lane >> 4)));
  raw.vs = __builtin_bit_cast(f32x4, buf_load16_stream(rvs, 16 * (lane >> 4)));
}

// K codes -> the bf16 K operands of the bf16 pools (codes are exact in bf16).
template <int D>
__device__ __forceinline__ void widen_k8(const RawBlock8<D>& raw, u32x4* k) {
#pragma unroll
  for (int j = 0; j < D / 64; ++j) {
    const u32x2 k0 = i8x4_to_bf16x4(raw.k[j].x), k1 = i8x4_to_bf16x4(raw.k[j].y);
    const u32x2 k2 = i8x4_to_bf16x4(raw.k[j].z), k3 = i8x4_to_bf16x4(raw.k[j].w);
    k[2 * j] = u32x4{k0.x, k0.y, k1.x, k1.y};
    k[2 * j + 1] = u32x4{k2.x, k2.y, k3.x, k3.y};
  }
}

// V codes -> the bf16 V^T operands of the bf16 pools.
template <int D>
__device__ __forceinline__ void widen_v8(const RawBlock8<D>& raw, u32x2* v) {
#pragma unroll
  for (int j = 0; j < D / 64; ++j) {
    v[4 * j] = i8x4_to_bf16x4(raw.v[j].x);
    v[4 * j + 1] = i8x4_to_bf16x4(raw.v[j].y);
    v[4 * j + 2] = i8x4_to_bf16x4(raw.v[j].z);
    v[4 * j + 3] = i8x4_to_bf16x4(raw.v[j].w);
  }
}

// The INT8 code of x against its row's scale, with append8_kernel's float32
// operations (a zero scale, an all-zero row, gives code 0).
__device__ __forceinline__ uint32_t code8(float x, float scale) {
  return scale > 0.0f ? static_cast<uint32_t>(static_cast<int>(fminf(fmaxf(rintf(x / scale), -127.0f), 127.0f))) & 0xffu
                      : 0u;
}

// P'^T V^T for one block of INT8 V codes (v: the widened codes): P' = P times
// each key's V scale goes to the matrix cores as two bf16 parts, hi =
// bf16(P') and lo = bf16(P' - hi), in one v_mfma_f32_16x16x32_bf16 per dim
// tile whose A operand holds the codes twice (exact in bf16). A single bf16
// P' would carry a 2^-9 relative error on every term, also on a row's
// dominant key, whose probability times an arbitrary scale is not 1.
template <int D>
__device__ __forceinline__ void pv8(const u32x2* v, const float (&pv)[4], f32x4* o) {
  const uint32_t h01 = pack_bf16x2(pv[0], pv[1]), h23 = pack_bf16x2(pv[2], pv[3]);
  const uint32_t l01 = pack_bf16x2(pv[0] - bf16_bits_to_f32(h01 & 0xffffu), pv[1] - bf16_bits_to_f32(h01 >> 16));
  const uint32_t l23 = pack_bf16x2(pv[2] - bf16_bits_to_f32(h23 & 0xffffu), pv[3] - bf16_bits_to_f32(h23 >> 16));
  const u32x4 pb = {h01, h23, l01, l23};
#pragma unroll
  for (int d = 0; d < D / 16; ++d) o[d] = mfma_16x16x32(u32x4{v[d].x, v[d].y, v[d].x, v[d].y}, pb, o[d]);
}

}  // namespace ha
