// Measurement probes (include/ha_probe.h): the read ceiling of decode's
// access pattern over the real page pools, and the matrix-core rate alone.
// They share the pool layout with the attention kernels but none of their
// arithmetic.
#include <hip/hip_runtime.h>

#include <cmath>

#include "../../include/ha_probe.h"
#include "common.hpp"
#include "status.hpp"

namespace ha {
namespace {

// Workgroup = (kv head, sequence), 4 waves; wave w reads blocks w, w+4, ...
// of [0, ceil(len / 16)) with two blocks in flight (buffers A and B), each
// block's K and V as D/32 + D/32 loads of 1 KiB per wave. Out-of-range page
// ids read nothing (zero-size descriptor), like the decode kernel.
template <int D, bool kNT>
__global__ __launch_bounds__(256) void paged_read_kernel(const uint16_t* kp, const uint16_t* vp, int num_blocks,
                                                         const int32_t* table, int stride, const int32_t* kv_len,
                                                         int hkv, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = blockIdx.x;
  const int b = blockIdx.y;
  const int len = kv_len[b];
  const int nblk = min((max(len, 0) + kBlock - 1) / kBlock, stride);
  const int32_t* row = table + static_cast<int64_t>(b) * stride;
  uint32_t acc = 0;
  u32x4 ka[D / 32], va[D / 32], kb[D / 32], vb[D / 32];
  auto load = [&](u32x4* kk, u32x4* vv, int i) {
    const int pg = i < nblk ? row[i] : -1;
    const bool ok = pg >= 0 && pg < num_blocks;
    const int64_t base = ok ? (static_cast<int64_t>(pg) * hkv + g) * kBlock * D : 0;
    const uint32_t bytes = ok ? kBlock * D * 2 : 0;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kp + base, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vp + base, bytes);
#pragma unroll
    for (int m = 0; m < D / 32; ++m) {
      kk[m] = kNT ? buf_load16_stream(rk, 16 * (64 * m + lane)) : buf_load16(rk, 16 * (64 * m + lane));
      vv[m] = kNT ? buf_load16_stream(rv, 16 * (64 * m + lane)) : buf_load16(rv, 16 * (64 * m + lane));
    }
  };
  auto fold = [&](const u32x4* kk, const u32x4* vv) {
#pragma unroll
    for (int m = 0; m < D / 32; ++m) acc ^= kk[m].x ^ kk[m].w ^ vv[m].y ^ vv[m].z;
  };
  int i = wave;
  load(ka, va, i);
  load(kb, vb, i + 4);
  const int nmine = nblk > wave ? (nblk - wave + 3) / 4 : 0;
  for (int k = 0; k + 1 < nmine; k += 2) {
    fold(ka, va);
    load(ka, va, i + 8);
    fold(kb, vb);
    load(kb, vb, i + 12);
    i += 8;
  }
  if (nmine & 1) fold(ka, va);
  sink[(static_cast<int64_t>(b) * hkv + g) * 256 + threadIdx.x] = acc;
}

// 8 independent accumulator chains per wave, operands in registers. The
// operands depend on the thread index so the products cannot be folded.
__global__ __launch_bounds__(256) void mfma_kernel(int iterations, float* sink) {
  const uint32_t t = threadIdx.x;
  const u32x4 a = {0x3f803f80u ^ t, 0x3f003f00u, 0x3e803e80u, 0x3f803f00u};
  const u32x4 b = {0x3f003f80u, 0x3f803f80u ^ (t << 1), 0x3e803f00u, 0x3f003f00u};
  f32x4 c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iterations; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = mfma_16x16x32(a, b, c[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  sink[static_cast<int64_t>(blockIdx.x) * 256 + t] = s;
}


// Matrix cores next to vector ALU work, 8 wavefronts (two per SIMD). A
// matrix block is 12 x 8 products on register operands (8 chains); a vector
// block is 6 x 16 dependent (FMA, exp2) pairs (16 chains), no memory.
//   0: every wave matrix blocks only      1: waves 0-3 matrix, 4-7 vector
//   2: every wave a matrix then a vector block, a barrier after each (in phase)
//   3: waves 0-3 matrix then vector, 4-7 vector then matrix, same barriers
//   4: every wave vector blocks only
template <int kMode>
__global__ __launch_bounds__(512, 1) void coissue_kernel(int iterations, float* sink) {
  const uint32_t t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(t >> 6));
  const u32x4 a = {0x3f803f80u ^ (t & 7u), 0x3f003f00u, 0x3e803e80u, 0x3f803f00u};
  const u32x4 b = {0x3f003f80u, 0x3f803f80u, 0x3e803f00u ^ (t & 3u), 0x3f003f00u};
  f32x4 c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float x[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] = 1e-3f * static_cast<float>(t + j);
  const float sc = 0.5f + 1e-7f * static_cast<float>(t);
  auto matrix = [&]() {
#pragma unroll
    for (int i = 0; i < 12; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = mfma_16x16x32(a, b, c[j]);
  };
  auto vector = [&]() {
#pragma unroll
    for (int i = 0; i < 6; ++i)
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] = fast_exp2(x[j] * sc - 1.0f);
  };
  for (int it = 0; it < iterations; ++it) {
    if constexpr (kMode == 0) {
      matrix();
    } else if constexpr (kMode == 1) {
      if (wave < 4) matrix();
      else vector();
    } else if constexpr (kMode == 2) {
      matrix();
      __syncthreads();
      vector();
      __syncthreads();
    } else if constexpr (kMode == 3) {
      if (wave < 4) matrix();
      else vector();
      __syncthreads();
      if (wave < 4) vector();
      else matrix();
      __syncthreads();
    } else {
      vector();
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
#pragma unroll
  for (int j = 0; j < 16; ++j) s += x[j];
  sink[static_cast<int64_t>(blockIdx.x) * 512 + t] = s;
}

}  // namespace
}  // namespace ha

extern "C" {

ha_status ha_probe_paged_read(const ha_shape* shape, const ha_kv_view* pages, const int32_t* kv_len, int32_t batch,
                              uint32_t* sink, int32_t nontemporal, void* stream) {
  if (!shape || !pages) return ha::set_error(HA_ERR_NULL, "shape or view is NULL");
  if (shape->head_dim != 64 && shape->head_dim != 128)
    return ha::set_error(HA_ERR_SHAPE, "head_dim must be 64 or 128 (got %d)", shape->head_dim);
  if (shape->num_kv_heads <= 0 || shape->num_kv_heads > 65535)
    return ha::set_error(HA_ERR_SHAPE, "num_kv_heads out of range (%d)", shape->num_kv_heads);
  if (shape->page_size != 16)
    return ha::set_error(HA_ERR_SHAPE, "the paged read probe walks 16-token pages (page_size %d)", shape->page_size);
  if (pages->kind != HA_FULL || pages->kv_dtype != HA_KV_BF16)
    return ha::set_error(HA_ERR_UNSUPPORTED, "the paged read probe takes a bf16 HA_FULL view");
  if (batch < 0 || batch > 65535) return ha::set_error(HA_ERR_RANGE, "batch out of range (%d)", batch);
  if (batch == 0) return ha::clear_error();
  if (!pages->k || !pages->v || !pages->table || !kv_len || !sink)
    return ha::set_error(HA_ERR_NULL, "pool, page table, kv_len or sink is NULL");
  if (pages->table_stride <= 0 || pages->num_blocks < 0)
    return ha::set_error(HA_ERR_RANGE, "page table stride must be positive");
  const dim3 grid(shape->num_kv_heads, batch);
  const auto* kp = static_cast<const uint16_t*>(pages->k);
  const auto* vp = static_cast<const uint16_t*>(pages->v);
  hipStream_t s = static_cast<hipStream_t>(stream);
#define HA_PROBE_LAUNCH(D, NT)                                                                                 \
  hipLaunchKernelGGL((ha::paged_read_kernel<D, NT>), grid, dim3(256), 0, s, kp, vp, pages->num_blocks,      \
                     pages->table, pages->table_stride, kv_len, shape->num_kv_heads, sink)
  if (shape->head_dim == 128) {
    if (nontemporal) HA_PROBE_LAUNCH(128, true);
    else HA_PROBE_LAUNCH(128, false);
  } else {
    if (nontemporal) HA_PROBE_LAUNCH(64, true);
    else HA_PROBE_LAUNCH(64, false);
  }
#undef HA_PROBE_LAUNCH
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return ha::set_error(HA_ERR_HIP, "probe launch: %s", hipGetErrorString(e));
  return ha::clear_error();
}

ha_status ha_probe_mfma_bf16(int32_t workgroups, int32_t iterations, float* sink, void* stream) {
  if (workgroups < 1 || iterations < 1)
    return ha::set_error(HA_ERR_RANGE, "workgroups and iterations must be >= 1 (got %d, %d)", workgroups,
                         iterations);
  if (!sink) return ha::set_error(HA_ERR_NULL, "sink is NULL");
  hipLaunchKernelGGL(ha::mfma_kernel, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream), iterations,
                     sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return ha::set_error(HA_ERR_HIP, "probe launch: %s", hipGetErrorString(e));
  return ha::clear_error();
}

ha_status ha_probe_coissue(int32_t mode, int32_t workgroups, int32_t iterations, float* sink, void* stream) {
  if (mode < 0 || mode > 4) return ha::set_error(HA_ERR_RANGE, "mode must be 0..4 (got %d)", mode);
  if (workgroups < 1 || iterations < 1)
    return ha::set_error(HA_ERR_RANGE, "workgroups and iterations must be >= 1 (got %d, %d)", workgroups,
                         iterations);
  if (!sink) return ha::set_error(HA_ERR_NULL, "sink is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(workgroups), block(512);
  switch (mode) {
    case 0: hipLaunchKernelGGL(ha::coissue_kernel<0>, grid, block, 0, s, iterations, sink); break;
    case 1: hipLaunchKernelGGL(ha::coissue_kernel<1>, grid, block, 0, s, iterations, sink); break;
    case 2: hipLaunchKernelGGL(ha::coissue_kernel<2>, grid, block, 0, s, iterations, sink); break;
    case 3: hipLaunchKernelGGL(ha::coissue_kernel<3>, grid, block, 0, s, iterations, sink); break;
    default: hipLaunchKernelGGL(ha::coissue_kernel<4>, grid, block, 0, s, iterations, sink); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return ha::set_error(HA_ERR_HIP, "probe launch: %s", hipGetErrorString(e));
  return ha::clear_error();
}

}  // extern "C"
