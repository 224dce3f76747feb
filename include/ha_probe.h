/*
 * ha_probe.h -- measurement probes: the achievable ceilings the attention
 * kernels of hybrid_attn.h are held against on this chip, next to the
 * published peaks (HBM 8 TB/s, dense bf16 matrix 2.5 PFLOP/s).
 *
 * Decode is bound by the KV bytes it reads (youleyou.com
 * "小米MiMo首次公开模型推理系统全链路优化降价99%", section 1 "为什么选择
 * Hybrid SWA 架构"; blog.hotdry.top 2026-06-12, section "架构层面的 KV Cache
 * 压缩"), so its ceiling is a read of the same bytes in the same pattern with
 * no arithmetic. Full-layer prefill is bound by the matrix cores, so its
 * ceiling is the matrix-core rate alone.
 *
 * The probes compute nothing of the method; their outputs are checksums that
 * only keep the loads and products alive. Ownership, streams and errors as in
 * hybrid_attn.h: caller-owned buffers, enqueue on the caller's stream,
 * validation on the host before any HIP call.
 */
#ifndef HA_PROBE_H
#define HA_PROBE_H

#include <stdint.h>

#include "hybrid_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads every K and V block of positions [0, kv_len[b]) of each sequence of a
 * bf16 Full page pool, exactly as the full-layer decode kernel walks them:
 * workgroup = (kv head, sequence), 4 wavefronts, wave w takes blocks w, w+4,
 * ..., two blocks in flight, 1 KiB contiguous per load instruction, page ids
 * through the page table. No arithmetic beyond an XOR per loaded word.
 *   pages      HA_FULL view, kv_dtype HA_KV_BF16, shape->page_size 16
 *   kv_len     int32 [batch] device
 *   sink       uint32 [batch * Hkv * 256] device (written; content meaningless)
 *   nontemporal != 0: the loads carry the non-temporal bit, as decode's do.
 * Bytes read = sum_b ceil(kv_len[b] / 16) * Hkv * 16 * D * 2 * 2. */
ha_status ha_probe_paged_read(const ha_shape* shape, const ha_kv_view* pages, const int32_t* kv_len,
                              int32_t batch, uint32_t* sink, int32_t nontemporal, void* stream);

/* Matrix cores alone: `workgroups` workgroups of 4 wavefronts, each wave
 * issuing `iterations` x 8 v_mfma_f32_16x16x32_bf16 on operands held in
 * registers (8 independent accumulators per wave). 16*16*32*2 flops per
 * instruction, so flops = workgroups * 4 * iterations * 8 * 16384.
 *   workgroups >= 1, iterations >= 1
 *   sink float32 [workgroups * 256] device (written; content meaningless) */
ha_status ha_probe_mfma_bf16(int32_t workgroups, int32_t iterations, float* sink, void* stream);

/* Matrix cores beside vector ALU work: whether one wavefront's products and
 * another's vector instructions on the same SIMD run at the same time, which
 * decides how much of prefill's softmax can hide under its products.
 * `workgroups` workgroups of 8 wavefronts (two per SIMD); per iteration a
 * "matrix block" is 96 v_mfma_f32_16x16x32_bf16 on register operands and a
 * "vector block" 96 dependent (FMA, exp2) pairs, no memory traffic.
 *   mode 0  every wave: matrix blocks only
 *   mode 1  waves 0-3: matrix blocks; waves 4-7: vector blocks
 *   mode 2  every wave: a matrix block, barrier, a vector block, barrier
 *   mode 3  waves 0-3 as mode 2; waves 4-7 vector first, then matrix
 *   mode 4  every wave: vector blocks only
 *   workgroups >= 1, iterations >= 1
 *   sink float32 [workgroups * 512] device (written; content meaningless) */
ha_status ha_probe_coissue(int32_t mode, int32_t workgroups, int32_t iterations, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HA_PROBE_H */
