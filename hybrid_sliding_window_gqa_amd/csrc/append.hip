// a1 / a2: scatter new K/V rows into the SWA ring pool or the Full page pool.
//
// The SWA pool is a per-sequence ring of W slots whose storage never grows
// beyond the window, and the Full pool is a paged store that grows as the
// caller hands out pages; both are physically separate (youleyou.com
// "小米MiMo首次公开模型推理系统全链路优化降价99%", section
// "KVCache系统重构：让缓存真正省下来"; blog.hotdry.top 2026-06-12,
// section "双池分治与三级缓存的工程实现").
//
// One thread moves 8 channels (16 bytes of bfloat16) of one token row of one
// kv head into its 16-token block, in the blocks' matrix-core operand order
// (common.hpp): the K channels form one 16-byte unit (one store), the V
// channels land in 8 different units (8 two-byte stores).
// Appends are a few KiB per decode step and a few hundred MiB per prefill
// chunk, far below the attention traffic, so they favour simplicity. INT8
// pools (include/hybrid_attn.h) are written by append8_kernel, which
// quantizes each (token, kv head) row with its own scale.
#include "common.hpp"
#include "kernels.hpp"

namespace ha {

template <bool kF32>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int d = a.geo.d;
  const int hkv = a.geo.hkv;
  const int chunks = d >> 3;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(a.num_tokens) * hkv * chunks;
  if (gid >= total) return;
  const int c = static_cast<int>(gid % chunks);
  const int64_t rest = gid / chunks;
  const int g = static_cast<int>(rest % hkv);
  const int tok = static_cast<int>(rest / hkv);

  // Sequence owning this row: the largest b with cu_new[b] <= tok.
  int lo = 0, hi = a.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.cu_new[mid] <= tok) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int i = tok - a.cu_new[b];
  const int n = a.cu_new[b + 1] - a.cu_new[b];
  if (i < 0 || i >= n) return;
  const int64_t p = static_cast<int64_t>(a.pos0[b]) + i;
  if (p < 0) return;

  int64_t block_base;  // element offset of the token's 16-token block for head g
  int in_blk;
  if (!a.full) {
    const int w = a.geo.window;
    if (i < n - w) return;  // overwritten later in this same call
    const int r = a.table[b];
    if (r < 0 || r >= a.num_blocks) return;
    const int s = static_cast<int>(p % w);
    block_base = ((static_cast<int64_t>(r) * hkv + g) * a.geo.ring + (s & ~(kBlock - 1))) * d;
    in_blk = s & (kBlock - 1);
  } else {
    const int64_t lb = p >> 4;                    // 16-token block of the sequence
    const int64_t lp = lb >> a.geo.page_shift;    // its page in the table row
    if (lp >= a.table_stride) return;
    const int pg = a.table[static_cast<int64_t>(b) * a.table_stride + lp];
    if (pg < 0 || pg >= a.num_blocks) return;
    block_base = page_block_offset(pg, g, hkv, static_cast<int>(lb & ((1 << a.geo.page_shift) - 1)),
                                   a.geo.page_shift, kBlock * d);
    in_blk = static_cast<int>(p & (kBlock - 1));
  }

  const int64_t src = (static_cast<int64_t>(tok) * hkv + g) * d + c * 8;
  const u32x4 kv = load8_as_bf16<kF32>(a.k_new, src);
  *reinterpret_cast<u32x4*>(a.k_pool + block_base + k_elem(in_blk, c * 8)) = kv;

  const u32x4 vv = load8_as_bf16<kF32>(a.v_new, src);
  uint16_t* vblk = a.v_pool + block_base;
  const uint32_t w4[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    vblk[v_elem(in_blk, c * 8 + 2 * j)] = static_cast<uint16_t>(w4[j] & 0xffffu);
    vblk[v_elem(in_blk, c * 8 + 2 * j + 1)] = static_cast<uint16_t>(w4[j] >> 16);
  }
}

// Full pools, prefill-sized appends: one workgroup per (16-token page block
// of a sequence's appended range, all kv heads). Each K row chunk is one
// 16-byte store; V goes through LDS so that a 16-byte V unit (4 tokens x 2
// channels) whose four slots are all appended in this call is written with
// one store, where append_kernel needs eight 2-byte stores. Units with a slot
// outside the appended range (at its first and last block) keep that slot
// and get 2-byte stores for the others. The slots written, and their values,
// are exactly append_kernel's.
template <bool kF32>
__global__ __launch_bounds__(256) void append_pages_kernel(AppendArgs a) {
  __shared__ uint16_t tile[kBlock][128 + 2];   // one head's V rows (D <= 128)
  const int d = a.geo.d;
  const int hkv = a.geo.hkv;
  const int cpr = d >> 3;                       // 16-byte chunks per row
  const int b = blockIdx.y;
  const int tok_b = a.cu_new[b];
  const int n = min(a.cu_new[b + 1], a.num_tokens) - tok_b;   // rows past num_tokens are never read
  const int64_t p0 = a.pos0[b];
  const int64_t start = p0 > 0 ? p0 : 0;       // positions below 0 are dropped
  const int64_t end = p0 + n;
  if (tok_b < 0 || start >= end) return;
  const int64_t jb = (start >> 4) + blockIdx.x; // 16-token block of the sequence
  const int64_t lo = max(start, jb * kBlock), hi = min(end, jb * kBlock + kBlock);
  const int64_t jp = jb >> a.geo.page_shift;    // its page in the table row
  if (lo >= hi || jp >= a.table_stride) return;
  const int pg = a.table[static_cast<int64_t>(b) * a.table_stride + jp];
  if (pg < 0 || pg >= a.num_blocks) return;
  const int sub = static_cast<int>(jb & ((1 << a.geo.page_shift) - 1));
  const int first = static_cast<int>(lo - jb * kBlock);   // slots [first, last) are appended
  const int last = static_cast<int>(hi - jb * kBlock);
  const int64_t tok_slot0 = tok_b + (jb * kBlock - p0);   // token index of slot 0
  const int tid = threadIdx.x;
  for (int g = 0; g < hkv; ++g) {
    const int64_t blk = page_block_offset(pg, g, hkv, sub, a.geo.page_shift, kBlock * d);
    for (int e = tid; e < kBlock * cpr; e += blockDim.x) {
      const int key = e / cpr;
      const int col = e - key * cpr;
      if (key < first || key >= last) continue;
      const int64_t src = ((tok_slot0 + key) * hkv + g) * d + col * 8;
      *reinterpret_cast<u32x4*>(a.k_pool + blk + k_elem(key, col * 8)) = load8_as_bf16_stream<kF32>(a.k_new, src);
      const u32x4 vv = load8_as_bf16_stream<kF32>(a.v_new, src);
      const uint32_t w4[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        tile[key][col * 8 + 2 * j] = static_cast<uint16_t>(w4[j] & 0xffffu);
        tile[key][col * 8 + 2 * j + 1] = static_cast<uint16_t>(w4[j] >> 16);
      }
    }
    __syncthreads();
    // V unit e = (p, q, c): tokens 4q..4q+3 of channels 32p + c and 32p + 16 + c
    for (int e = tid; e < 2 * d; e += blockDim.x) {
      const int p = e / 64;
      const int q = (e / 16) & 3;
      const int c = e & 15;
      if (4 * q + 3 < first || 4 * q >= last) continue;
      if (4 * q >= first && 4 * q + 3 < last) {
        uint32_t w4[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int ch = 32 * p + 16 * h + c;
          w4[2 * h] = static_cast<uint32_t>(tile[4 * q][ch]) | (static_cast<uint32_t>(tile[4 * q + 1][ch]) << 16);
          w4[2 * h + 1] = static_cast<uint32_t>(tile[4 * q + 2][ch]) | (static_cast<uint32_t>(tile[4 * q + 3][ch]) << 16);
        }
        *reinterpret_cast<u32x4*>(a.v_pool + blk + 8 * e) = u32x4{w4[0], w4[1], w4[2], w4[3]};
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = 4 * q + r;
          if (key < first || key >= last) continue;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int ch = 32 * p + 16 * h + c;
            a.v_pool[blk + v_elem(key, ch)] = tile[key][ch];
          }
        }
      }
    }
    __syncthreads();
  }
}

// INT8 pools: the same thread mapping; the chunks/lanes of one (token, kv
// head) row are consecutive lanes of a wave, so the row's absmax is a
// butterfly over them. scale = amax / 127 and code = rint(x / scale), both
// in IEEE float32 (x = the bf16 value), so the codes are exactly those of
// the definition; lane 0 of the row writes the two scales.
template <bool kF32>
__global__ __launch_bounds__(256) void append8_kernel(AppendArgs a) {
  const int d = a.geo.d;
  const int hkv = a.geo.hkv;
  const int chunks = d >> 3;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(a.num_tokens) * hkv * chunks;
  if (gid >= total) return;   // whole rows: total and the block size are multiples of chunks
  const int c = static_cast<int>(gid % chunks);
  const int64_t rest = gid / chunks;
  const int g = static_cast<int>(rest % hkv);
  const int tok = static_cast<int>(rest / hkv);

  int lo = 0, hi = a.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.cu_new[mid] <= tok) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int i = tok - a.cu_new[b];
  const int n = a.cu_new[b + 1] - a.cu_new[b];
  if (i < 0 || i >= n) return;
  const int64_t p = static_cast<int64_t>(a.pos0[b]) + i;
  if (p < 0) return;

  int64_t block_base;  // byte offset of the token's 16-token block for head g
  int in_blk;
  if (!a.full) {
    const int w = a.geo.window;
    if (i < n - w) return;
    const int r = a.table[b];
    if (r < 0 || r >= a.num_blocks) return;
    const int s = static_cast<int>(p % w);
    block_base = ((static_cast<int64_t>(r) * hkv + g) * a.geo.ring + (s & ~(kBlock - 1))) * d;
    in_blk = s & (kBlock - 1);
  } else {
    const int64_t lb = p >> 4;                    // 16-token block of the sequence
    const int64_t lp = lb >> a.geo.page_shift;    // its page in the table row
    if (lp >= a.table_stride) return;
    const int pg = a.table[static_cast<int64_t>(b) * a.table_stride + lp];
    if (pg < 0 || pg >= a.num_blocks) return;
    block_base = page_block_offset(pg, g, hkv, static_cast<int>(lb & ((1 << a.geo.page_shift) - 1)),
                                   a.geo.page_shift, kBlock * d);
    in_blk = static_cast<int>(p & (kBlock - 1));
  }
  // Every early return above is uniform over the lanes of one row, so the
  // whole row takes part in the butterflies below.

  const int64_t src = (static_cast<int64_t>(tok) * hkv + g) * d + c * 8;
  const u32x4 kraw = load8_as_bf16<kF32>(a.k_new, src);
  const u32x4 vraw = load8_as_bf16<kF32>(a.v_new, src);
  float kx[8], vx[8];
  const uint32_t kw[4] = {kraw.x, kraw.y, kraw.z, kraw.w};
  const uint32_t vw[4] = {vraw.x, vraw.y, vraw.z, vraw.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    kx[2 * j] = __uint_as_float(kw[j] << 16);
    kx[2 * j + 1] = __uint_as_float(kw[j] & 0xffff0000u);
    vx[2 * j] = __uint_as_float(vw[j] << 16);
    vx[2 * j + 1] = __uint_as_float(vw[j] & 0xffff0000u);
  }
  float ka = 0.0f, va = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ka = max_prop(ka, fabsf(kx[j]));
    va = max_prop(va, fabsf(vx[j]));
  }
  for (int m = chunks >> 1; m >= 1; m >>= 1) {
    ka = max_prop(ka, __shfl_xor(ka, m));
    va = max_prop(va, __shfl_xor(va, m));
  }
  const float ks = ka / 127.0f;
  const float vs = va / 127.0f;
  uint32_t kq[2] = {0u, 0u};
  uint8_t* vblk = reinterpret_cast<uint8_t*>(a.v_pool) + block_base;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int kc = ks > 0.0f ? static_cast<int>(fminf(fmaxf(rintf(kx[j] / ks), -127.0f), 127.0f)) : 0;
    const int vc = vs > 0.0f ? static_cast<int>(fminf(fmaxf(rintf(vx[j] / vs), -127.0f), 127.0f)) : 0;
    kq[j >> 2] |= (static_cast<uint32_t>(kc) & 0xffu) << (8 * (j & 3));
    vblk[v8_elem(in_blk, c * 8 + j)] = static_cast<uint8_t>(vc & 0xff);
  }
  *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(a.k_pool) + block_base + k8_elem(in_blk, c * 8)) =
      u32x2{kq[0], kq[1]};
  if (c == 0) {
    const int64_t si = block_base / d + in_blk;
    a.k_scale[si] = ks;
    a.v_scale[si] = vs;
  }
}

// Inverse of append_kernel: one thread per (token, kv head, 8 channels)
// gathers the K unit and the 8 V values from the block and writes them as
// token-major rows. Every position is read (no ring overwrite skipping).
__global__ __launch_bounds__(256) void read_kernel(AppendArgs a, uint16_t* k_out, uint16_t* v_out) {
  const int d = a.geo.d;
  const int hkv = a.geo.hkv;
  const int chunks = d >> 3;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(a.num_tokens) * hkv * chunks;
  if (gid >= total) return;
  const int c = static_cast<int>(gid % chunks);
  const int64_t rest = gid / chunks;
  const int g = static_cast<int>(rest % hkv);
  const int tok = static_cast<int>(rest / hkv);
  int lo = 0, hi = a.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.cu_new[mid] <= tok) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int i = tok - a.cu_new[b];
  if (i < 0 || i >= a.cu_new[b + 1] - a.cu_new[b]) return;
  const int64_t p = static_cast<int64_t>(a.pos0[b]) + i;
  if (p < 0) return;
  int64_t block_base;
  int in_blk;
  if (!a.full) {
    const int w = a.geo.window;
    const int r = a.table[b];
    if (r < 0 || r >= a.num_blocks) return;
    const int s = static_cast<int>(p % w);
    block_base = ((static_cast<int64_t>(r) * hkv + g) * a.geo.ring + (s & ~(kBlock - 1))) * d;
    in_blk = s & (kBlock - 1);
  } else {
    const int64_t lb = p >> 4;                    // 16-token block of the sequence
    const int64_t lp = lb >> a.geo.page_shift;    // its page in the table row
    if (lp >= a.table_stride) return;
    const int pg = a.table[static_cast<int64_t>(b) * a.table_stride + lp];
    if (pg < 0 || pg >= a.num_blocks) return;
    block_base = page_block_offset(pg, g, hkv, static_cast<int>(lb & ((1 << a.geo.page_shift) - 1)),
                                   a.geo.page_shift, kBlock * d);
    in_blk = static_cast<int>(p & (kBlock - 1));
  }
  const int64_t dst = (static_cast<int64_t>(tok) * hkv + g) * d + c * 8;
  *reinterpret_cast<u32x4*>(k_out + dst) =
      *reinterpret_cast<const u32x4*>(a.k_pool + block_base + k_elem(in_blk, c * 8));
  const uint16_t* vblk = a.v_pool + block_base;
  uint32_t w4[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    w4[j] = static_cast<uint32_t>(vblk[v_elem(in_blk, c * 8 + 2 * j)]) |
            (static_cast<uint32_t>(vblk[v_elem(in_blk, c * 8 + 2 * j + 1)]) << 16);
  *reinterpret_cast<u32x4*>(v_out + dst) = u32x4{w4[0], w4[1], w4[2], w4[3]};
}

hipError_t launch_read(const AppendArgs& a, void* k_out, void* v_out, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(a.num_tokens) * a.geo.hkv * (a.geo.d >> 3);
  if (total == 0 || a.batch == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(read_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a,
                     static_cast<uint16_t*>(k_out), static_cast<uint16_t*>(v_out));
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(a.num_tokens) * a.geo.hkv * (a.geo.d >> 3);
  if (total == 0 || a.batch == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks));
  // Full pools with at least 16 new tokens per sequence on average: one
  // workgroup per page block (grid.x bounds the blocks any one sequence's
  // range can touch; workgroups past a sequence's range exit at once).
  const bool by_pages = a.full && !a.kv8 && a.geo.d <= 128 &&
                        static_cast<int64_t>(a.num_tokens) >= static_cast<int64_t>(kBlock) * a.batch;
  if (by_pages) {
    const int64_t gx = (static_cast<int64_t>(a.num_tokens) + kBlock - 1) / kBlock + 1;
    if (gx > 0x7fffffff || a.batch > 65535) return hipErrorInvalidValue;
    const dim3 pgrid(static_cast<unsigned>(gx), a.batch);
    if (a.src_f32) hipLaunchKernelGGL(append_pages_kernel<true>, pgrid, dim3(threads), 0, stream, a);
    else hipLaunchKernelGGL(append_pages_kernel<false>, pgrid, dim3(threads), 0, stream, a);
  } else if (a.kv8) {
    if (a.src_f32) hipLaunchKernelGGL(append8_kernel<true>, grid, dim3(threads), 0, stream, a);
    else hipLaunchKernelGGL(append8_kernel<false>, grid, dim3(threads), 0, stream, a);
  } else if (a.src_f32) {
    hipLaunchKernelGGL(append_kernel<true>, grid, dim3(threads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(append_kernel<false>, grid, dim3(threads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace ha
