// C ABI of the hybrid attention library: argument validation, error
// reporting, the host-side window-safe prefix matcher, and dispatch to the
// kernel launchers. Every check runs on the host before any HIP call, so a
// rejected call never touches the device.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/hybrid_attn.h"
#include "kernels.hpp"
#include "status.hpp"

namespace {

thread_local std::string g_last_error;

ha_status fail(ha_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

ha_status ok() {
  g_last_error.clear();
  return HA_OK;
}

ha_status check_shape(const ha_shape* s, ha::Geometry* geo) {
  if (!s) return fail(HA_ERR_NULL, "shape is NULL");
  if (s->num_q_heads <= 0 || s->num_kv_heads <= 0)
    return fail(HA_ERR_SHAPE, "head counts must be positive (got %d q, %d kv)", s->num_q_heads, s->num_kv_heads);
  if (s->num_q_heads % s->num_kv_heads != 0)
    return fail(HA_ERR_SHAPE, "num_q_heads %d is not a multiple of num_kv_heads %d", s->num_q_heads,
                s->num_kv_heads);
  const int group = s->num_q_heads / s->num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8 && group != 16)
    return fail(HA_ERR_SHAPE, "query heads per kv head must be 1, 2, 4, 8 or 16 (got %d)", group);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(HA_ERR_SHAPE, "head_dim must be 64 or 128 (got %d)", s->head_dim);
  if (s->window < 1 || s->window > (1 << 24))
    return fail(HA_ERR_SHAPE, "window must be in [1, 2^24] (got %d)", s->window);
  if (s->page_size < 16 || s->page_size > (1 << 20) || (s->page_size & (s->page_size - 1)) != 0)
    return fail(HA_ERR_SHAPE, "page_size must be a power of two in [16, 2^20] (got %d)", s->page_size);
  if (!(std::isfinite(s->softmax_scale))) return fail(HA_ERR_SHAPE, "softmax_scale is not finite");
  geo->hq = s->num_q_heads;
  geo->hkv = s->num_kv_heads;
  geo->d = s->head_dim;
  geo->window = s->window;
  geo->ring = (s->window + 15) / 16 * 16;
  geo->page_shift = __builtin_ctz(static_cast<unsigned>(s->page_size)) - 4;
  geo->group = group;
  geo->scale = s->softmax_scale > 0.0f ? s->softmax_scale : 1.0f / std::sqrt(static_cast<float>(s->head_dim));
  return HA_OK;
}

ha_status check_view(const ha_kv_view* kv, int batch, const ha::Geometry& geo) {
  if (!kv) return fail(HA_ERR_NULL, "kv view is NULL");
  if (kv->kind != HA_SWA && kv->kind != HA_FULL) return fail(HA_ERR_UNSUPPORTED, "unknown layer kind %d", kv->kind);
  if (kv->num_blocks < 0) return fail(HA_ERR_RANGE, "num_blocks is negative");
  if (kv->kv_dtype != HA_KV_BF16 && kv->kv_dtype != HA_KV_INT8)
    return fail(HA_ERR_UNSUPPORTED, "unknown pool format %d", kv->kv_dtype);
  if (batch > 0) {
    if (!kv->k || !kv->v) return fail(HA_ERR_NULL, "pool K or V pointer is NULL");
    if (kv->kv_dtype == HA_KV_INT8 && (!kv->k_scale || !kv->v_scale))
      return fail(HA_ERR_NULL, "an INT8 pool needs k_scale and v_scale");
    if (!kv->table) return fail(HA_ERR_NULL, "%s is NULL", kv->kind == HA_SWA ? "ring id table" : "page table");
    if (kv->kind == HA_FULL && kv->table_stride <= 0)
      return fail(HA_ERR_RANGE, "page table stride must be positive (got %d)", kv->table_stride);
    // a row's 16-token blocks are counted in int; positions are int32, so
    // rows past 2^27 blocks could never be reached anyway
    if (kv->kind == HA_FULL && (static_cast<int64_t>(kv->table_stride) << geo.page_shift) > (int64_t{1} << 27))
      return fail(HA_ERR_RANGE, "page table stride %d x page_size covers more than 2^31 tokens", kv->table_stride);
  }
  return HA_OK;
}

ha_status check_dtype(int32_t dt) {
  if (dt != HA_BF16 && dt != HA_F32) return fail(HA_ERR_UNSUPPORTED, "unsupported dtype %d", dt);
  return HA_OK;
}

ha_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(HA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

ha_status append_common(const ha_shape* shape, const ha_kv_view* view, int32_t want_kind, const int32_t* pos0,
                        const int32_t* cu_new, int32_t batch, int32_t num_tokens, const void* k_new,
                        const void* v_new, int32_t src_dtype, void* stream) {
  ha::Geometry geo;
  ha_status st = check_shape(shape, &geo);
  if (st != HA_OK) return st;
  if (batch < 0 || num_tokens < 0) return fail(HA_ERR_RANGE, "batch and num_tokens must be >= 0");
  st = check_view(view, batch, geo);
  if (st != HA_OK) return st;
  if (view->kind != want_kind)
    return fail(HA_ERR_UNSUPPORTED, "%s needs a %s view", want_kind == HA_SWA ? "swa_ring_append" : "full_pool_append",
                want_kind == HA_SWA ? "HA_SWA" : "HA_FULL");
  if ((st = check_dtype(src_dtype)) != HA_OK) return st;
  if (batch == 0 || num_tokens == 0) return ok();
  if (!pos0 || !cu_new) return fail(HA_ERR_NULL, "pos0 or cu_new is NULL");
  if (!k_new || !v_new) return fail(HA_ERR_NULL, "k_new or v_new is NULL");
  ha::AppendArgs a{};
  a.geo = geo;
  a.full = want_kind == HA_FULL;
  a.k_pool = static_cast<uint16_t*>(view->k);
  a.v_pool = static_cast<uint16_t*>(view->v);
  a.num_blocks = view->num_blocks;
  a.table = view->table;
  a.table_stride = view->table_stride;
  a.pos0 = pos0;
  a.cu_new = cu_new;
  a.batch = batch;
  a.num_tokens = num_tokens;
  a.k_new = k_new;
  a.v_new = v_new;
  a.src_f32 = src_dtype == HA_F32;
  a.kv8 = view->kv_dtype == HA_KV_INT8;
  a.k_scale = view->k_scale;
  a.v_scale = view->v_scale;
  return hip_status(ha::launch_append(a, static_cast<hipStream_t>(stream)), "append launch");
}

ha_status read_common(const ha_shape* shape, const ha_kv_view* view, int32_t want_kind, const int32_t* pos0,
                      const int32_t* cu, int32_t batch, int32_t num_tokens, void* k_out, void* v_out,
                      void* stream) {
  ha::Geometry geo;
  ha_status st = check_shape(shape, &geo);
  if (st != HA_OK) return st;
  if (batch < 0 || num_tokens < 0) return fail(HA_ERR_RANGE, "batch and num_tokens must be >= 0");
  st = check_view(view, batch, geo);
  if (st != HA_OK) return st;
  if (view->kind != want_kind)
    return fail(HA_ERR_UNSUPPORTED, "%s needs a %s view", want_kind == HA_SWA ? "swa_ring_read" : "full_pool_read",
                want_kind == HA_SWA ? "HA_SWA" : "HA_FULL");
  if (view->kv_dtype != HA_KV_BF16) return fail(HA_ERR_UNSUPPORTED, "reads return bf16 rows of bf16 pools only");
  if (batch == 0 || num_tokens == 0) return ok();
  if (!pos0 || !cu) return fail(HA_ERR_NULL, "pos0 or cu is NULL");
  if (!k_out || !v_out) return fail(HA_ERR_NULL, "k_out or v_out is NULL");
  ha::AppendArgs a{};
  a.geo = geo;
  a.full = want_kind == HA_FULL;
  a.k_pool = static_cast<uint16_t*>(view->k);
  a.v_pool = static_cast<uint16_t*>(view->v);
  a.num_blocks = view->num_blocks;
  a.table = view->table;
  a.table_stride = view->table_stride;
  a.pos0 = pos0;
  a.cu_new = cu;
  a.batch = batch;
  a.num_tokens = num_tokens;
  return hip_status(ha::launch_read(a, k_out, v_out, static_cast<hipStream_t>(stream)), "read launch");
}

// Bytes of the staged chunk (K and V of every 16-token block, bf16), rounded
// up to 256 so the full layers' partial rows that follow start aligned.
size_t prefill_stage_bytes(const ha::Geometry& geo, int batch, int num_tokens) {
  const size_t bytes = static_cast<size_t>(ha::prefill_stage_blocks(num_tokens, batch)) * geo.hkv * 16 * geo.d * 2 * 2;
  return (bytes + 255) / 256 * 256;
}

size_t prefill_workspace(const ha::Geometry& geo, bool full, int batch, int num_tokens) {
  if (batch <= 0 || num_tokens <= 0) return 0;
  return prefill_stage_bytes(geo, batch, num_tokens) + (full ? static_cast<size_t>(ha::prefill_partial_bytes(geo.d)) : 0);
}

size_t decode_workspace(const ha::Geometry& geo, bool full, int batch, int max_kv_len, int num_splits) {
  if (!full) return 0;
  const int sb = ha::decode_split_blocks(true, geo.window, max_kv_len, batch, geo.hkv, num_splits);
  const int ns = ha::decode_num_splits(true, geo.window, max_kv_len, sb);
  if (ns <= 1) return 0;
  return static_cast<size_t>(batch) * geo.hq * ns * (geo.d + 1) * sizeof(float);
}

size_t verify_workspace(const ha::Geometry& geo, bool full, int batch, int max_kv_len, int nq, int num_splits) {
  if (!full) return 0;
  const int sb = ha::decode_split_blocks(true, geo.window, max_kv_len, batch, geo.hkv, num_splits);
  const int ns = ha::decode_num_splits(true, geo.window, max_kv_len, sb);
  if (ns <= 1) return 0;
  return static_cast<size_t>(batch) * nq * geo.hq * ns * (geo.d + 1) * sizeof(float);
}

ha_status check_nq(const ha::Geometry& geo, int nq) {
  if (nq < 1 || nq > 16) return fail(HA_ERR_RANGE, "nq must be in [1, 16] (got %d)", nq);
  if (nq * geo.group > 32)
    return fail(HA_ERR_SHAPE, "nq * (Hq / Hkv) must be <= 32 (got %d * %d)", nq, geo.group);
  return ok();
}

// Where the split-K partials of a decode call live.
enum class Scratch { kCallerWorkspace, kLibraryStatic };

ha_status decode_common(const ha_shape* shape, const ha_kv_view* kv, const int32_t* kv_len, int32_t batch,
                        int32_t max_kv_len, const void* q, const void* k_new, const void* v_new, int32_t in_dtype,
                        float* out, float* lse, int32_t num_splits, Scratch where, void* workspace,
                        size_t workspace_bytes, void* stream) {
  ha::Geometry geo;
  ha_status st = check_shape(shape, &geo);
  if (st != HA_OK) return st;
  if (batch < 0 || max_kv_len < 0 || num_splits < 0)
    return fail(HA_ERR_RANGE, "batch, max_kv_len and num_splits must be >= 0");
  if ((st = check_view(kv, batch, geo)) != HA_OK) return st;
  if ((st = check_dtype(in_dtype)) != HA_OK) return st;
  if (batch == 0) return ok();
  if (batch > 65535) return fail(HA_ERR_RANGE, "decode batch %d exceeds 65535", batch);
  if (!kv_len || !q || !out || !lse) return fail(HA_ERR_NULL, "kv_len, q, out or lse is NULL");
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(HA_ERR_NULL, "k_new and v_new must both be given (fused append) or both be NULL");
  const bool kv8 = kv->kv_dtype == HA_KV_INT8;
  const bool full = kv->kind == HA_FULL;
  const size_t need = decode_workspace(geo, full, batch, max_kv_len, num_splits);
  if (where == Scratch::kCallerWorkspace) {
    if (need > 0 && (!workspace || workspace_bytes < need))
      return fail(HA_ERR_WORKSPACE, "decode needs %zu workspace bytes, got %zu", need, workspace ? workspace_bytes : 0);
  } else if (need > HA_DECODE_SCRATCH_BYTES) {
    return fail(HA_ERR_WORKSPACE,
                "decode needs %zu scratch bytes; the library's static scratch holds %zu: pass a smaller num_splits "
                "or use hybrid_attn_decode with a workspace",
                need, static_cast<size_t>(HA_DECODE_SCRATCH_BYTES));
  }
  ha::DecodeArgs a{};
  a.geo = geo;
  a.full = full;
  a.k_pool = static_cast<const uint16_t*>(kv->k);
  a.v_pool = static_cast<const uint16_t*>(kv->v);
  a.num_blocks = kv->num_blocks;
  a.table = kv->table;
  a.table_stride = kv->table_stride;
  a.kv_len = kv_len;
  a.batch = batch;
  a.q = q;
  a.q_f32 = in_dtype == HA_F32;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_pool_w = static_cast<uint16_t*>(kv->k);
  a.v_pool_w = static_cast<uint16_t*>(kv->v);
  a.kv8 = kv8;
  a.k_scale = kv->k_scale;
  a.v_scale = kv->v_scale;
  a.out = out;
  a.lse = lse;
  a.split_blocks = ha::decode_split_blocks(full, geo.window, max_kv_len, batch, geo.hkv, num_splits);
  a.splits = ha::decode_num_splits(full, geo.window, max_kv_len, a.split_blocks);
  if (a.splits > 65535) return fail(HA_ERR_RANGE, "too many key splits (%d); pass a smaller num_splits", a.splits);
  if (need > 0 && where == Scratch::kLibraryStatic) {
    // The partials go to the current device's copy of the static array; the
    // stream must belong to that device.
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (stream != nullptr) {
      hipDevice_t sdev = -1;
      e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
      if (e != hipSuccess) return hip_status(e, "hipStreamGetDevice");
      if (sdev != dev)
        return fail(HA_ERR_RANGE, "the stream belongs to device %d, the current device is %d", sdev, dev);
    }
    e = ha::decode_scratch(dev, &workspace);
    if (e != hipSuccess) return hip_status(e, "static scratch lookup");
  }
  if (need > 0) {
    float* ws = static_cast<float*>(workspace);
    a.part_o = ws;
    a.part_lse = ws + static_cast<size_t>(batch) * geo.hq * a.splits * geo.d;
  }
  return hip_status(ha::launch_decode(a, static_cast<hipStream_t>(stream)), "decode launch");
}

}  // namespace

namespace ha {

ha_status set_error(ha_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

ha_status clear_error() {
  g_last_error.clear();
  return HA_OK;
}

}  // namespace ha

extern "C" {

ha_status swa_ring_append(const ha_shape* shape, const ha_kv_view* ring, const int32_t* pos0, const int32_t* cu_new,
                          int32_t batch, int32_t num_tokens, const void* k_new, const void* v_new,
                          int32_t src_dtype, void* stream) {
  return append_common(shape, ring, HA_SWA, pos0, cu_new, batch, num_tokens, k_new, v_new, src_dtype, stream);
}

ha_status full_pool_append(const ha_shape* shape, const ha_kv_view* pages, const int32_t* pos0,
                           const int32_t* cu_new, int32_t batch, int32_t num_tokens, const void* k_new,
                           const void* v_new, int32_t src_dtype, void* stream) {
  return append_common(shape, pages, HA_FULL, pos0, cu_new, batch, num_tokens, k_new, v_new, src_dtype, stream);
}

ha_status swa_ring_read(const ha_shape* shape, const ha_kv_view* ring, const int32_t* pos0, const int32_t* cu,
                        int32_t batch, int32_t num_tokens, void* k_out, void* v_out, void* stream) {
  return read_common(shape, ring, HA_SWA, pos0, cu, batch, num_tokens, k_out, v_out, stream);
}

ha_status full_pool_read(const ha_shape* shape, const ha_kv_view* pages, const int32_t* pos0, const int32_t* cu,
                         int32_t batch, int32_t num_tokens, void* k_out, void* v_out, void* stream) {
  return read_common(shape, pages, HA_FULL, pos0, cu, batch, num_tokens, k_out, v_out, stream);
}

ha_status window_safe_match(const int32_t* req_tokens, int64_t req_len, const int32_t* cached_tokens,
                            int64_t cached_len, const uint8_t* swa_valid, int32_t window, int64_t* out_len) {
  if (!out_len) return fail(HA_ERR_NULL, "out_len is NULL");
  if (req_len < 0 || cached_len < 0) return fail(HA_ERR_RANGE, "lengths must be >= 0");
  if (window < 1) return fail(HA_ERR_SHAPE, "window must be >= 1 (got %d)", window);
  if ((req_len > 0 && !req_tokens) || (cached_len > 0 && (!cached_tokens || !swa_valid)))
    return fail(HA_ERR_NULL, "token or validity array is NULL");
  const int64_t n = req_len < cached_len ? req_len : cached_len;
  int64_t m = 0;
  while (m < n && req_tokens[m] == cached_tokens[m]) ++m;
  // Walk back from m: if an invalid slot x lies in the candidate's last window
  // [L - W, L), no length in (x, L] can be safe, so the next candidate is x.
  int64_t len = m;
  for (;;) {
    const int64_t lo = len - window > 0 ? len - window : 0;
    int64_t bad = -1;
    for (int64_t p = len - 1; p >= lo; --p) {
      if (!swa_valid[p]) {
        bad = p;
        break;
      }
    }
    if (bad < 0) break;
    len = bad;
  }
  *out_len = len;
  return ok();
}

ha_status hybrid_attn_prefill(const ha_shape* shape, const ha_kv_view* kv, const int32_t* hist_len,
                              const int32_t* cu_new, int32_t batch, int32_t num_tokens, int32_t max_new,
                              const void* q, const void* k_new, const void* v_new, int32_t in_dtype, float* out,
                              float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  ha::Geometry geo;
  ha_status st = check_shape(shape, &geo);
  if (st != HA_OK) return st;
  if (batch < 0 || num_tokens < 0 || max_new < 0)
    return fail(HA_ERR_RANGE, "batch, num_tokens and max_new must be >= 0");
  if ((st = check_view(kv, batch, geo)) != HA_OK) return st;
  if (kv->kv_dtype != HA_KV_BF16) return fail(HA_ERR_UNSUPPORTED, "prefill reads bf16 pools only");
  if ((st = check_dtype(in_dtype)) != HA_OK) return st;
  if (batch == 0 || num_tokens == 0 || max_new == 0) return ok();
  if (max_new > num_tokens) return fail(HA_ERR_RANGE, "max_new %d exceeds num_tokens %d", max_new, num_tokens);
  if (!hist_len || !cu_new) return fail(HA_ERR_NULL, "hist_len or cu_new is NULL");
  if (!q || !k_new || !v_new) return fail(HA_ERR_NULL, "q, k_new or v_new is NULL");
  if (!out || !lse) return fail(HA_ERR_NULL, "out or lse is NULL");
  const size_t need = prefill_workspace(geo, kv->kind == HA_FULL, batch, num_tokens);
  if (!workspace || workspace_bytes < need)
    return fail(HA_ERR_WORKSPACE, "prefill needs %zu workspace bytes, got %zu", need, workspace ? workspace_bytes : 0);
  ha::PrefillArgs a{};
  a.geo = geo;
  a.full = kv->kind == HA_FULL;
  a.k_pool = static_cast<const uint16_t*>(kv->k);
  a.v_pool = static_cast<const uint16_t*>(kv->v);
  a.num_blocks = kv->num_blocks;
  a.table = kv->table;
  a.table_stride = kv->table_stride;
  a.hist_len = hist_len;
  a.cu_new = cu_new;
  a.batch = batch;
  a.num_tokens = num_tokens;
  a.max_new = max_new;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.in_f32 = in_dtype == HA_F32;
  a.out = out;
  a.lse = lse;
  a.stage = static_cast<uint16_t*>(workspace);
  a.stage_blocks = ha::prefill_stage_blocks(num_tokens, batch);
  a.part = a.full ? reinterpret_cast<float*>(static_cast<char*>(workspace) + prefill_stage_bytes(geo, batch, num_tokens))
                  : nullptr;
  return hip_status(ha::launch_prefill(a, static_cast<hipStream_t>(stream)), "prefill launch");
}

ha_status hybrid_attn_decode(const ha_shape* shape, const ha_kv_view* kv, const int32_t* kv_len, int32_t batch,
                             int32_t max_kv_len, const void* q, const void* k_new, const void* v_new,
                             int32_t in_dtype, float* out, float* lse, int32_t num_splits, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return decode_common(shape, kv, kv_len, batch, max_kv_len, q, k_new, v_new, in_dtype, out, lse, num_splits,
                       Scratch::kCallerWorkspace, workspace, workspace_bytes, stream);
}

ha_status hybrid_attn_decode_noalloc(const ha_shape* shape, const ha_kv_view* kv, const int32_t* kv_len,
                                     int32_t batch, int32_t max_kv_len, const void* q, const void* k_new,
                                     const void* v_new, int32_t in_dtype, float* out, float* lse,
                                     int32_t num_splits, void* stream) {
  return decode_common(shape, kv, kv_len, batch, max_kv_len, q, k_new, v_new, in_dtype, out, lse, num_splits,
                       Scratch::kLibraryStatic, nullptr, 0, stream);
}

ha_status hybrid_attn_verify(const ha_shape* shape, const ha_kv_view* kv, const int32_t* kv_len, int32_t batch,
                             int32_t max_kv_len, int32_t nq, const void* q, const void* k_new, const void* v_new,
                             int32_t in_dtype, float* out, float* lse, int32_t num_splits, void* workspace,
                             size_t workspace_bytes, void* stream) {
  ha::Geometry geo;
  ha_status st = check_shape(shape, &geo);
  if (st != HA_OK) return st;
  if (batch < 0 || max_kv_len < 0 || num_splits < 0)
    return fail(HA_ERR_RANGE, "batch, max_kv_len and num_splits must be >= 0");
  if ((st = check_nq(geo, nq)) != HA_OK) return st;
  if ((st = check_view(kv, batch, geo)) != HA_OK) return st;
  if ((st = check_dtype(in_dtype)) != HA_OK) return st;
  if (batch == 0) return ok();
  if (batch > 65535) return fail(HA_ERR_RANGE, "verify batch %d exceeds 65535", batch);
  if (!kv_len || !q || !out || !lse) return fail(HA_ERR_NULL, "kv_len, q, out or lse is NULL");
  if (!k_new || !v_new) return fail(HA_ERR_NULL, "k_new and v_new (the new tokens' K/V) are required");
  const bool full = kv->kind == HA_FULL;
  const size_t need = verify_workspace(geo, full, batch, max_kv_len, nq, num_splits);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(HA_ERR_WORKSPACE, "verify needs %zu workspace bytes, got %zu", need, workspace ? workspace_bytes : 0);
  ha::VerifyArgs a{};
  a.geo = geo;
  a.full = full;
  a.k_pool = static_cast<const uint16_t*>(kv->k);
  a.v_pool = static_cast<const uint16_t*>(kv->v);
  a.k_pool_w = static_cast<uint16_t*>(kv->k);
  a.v_pool_w = static_cast<uint16_t*>(kv->v);
  a.num_blocks = kv->num_blocks;
  a.table = kv->table;
  a.table_stride = kv->table_stride;
  a.kv_len = kv_len;
  a.batch = batch;
  a.nq = nq;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.in_f32 = in_dtype == HA_F32;
  a.kv8 = kv->kv_dtype == HA_KV_INT8;
  a.k_scale = kv->k_scale;
  a.v_scale = kv->v_scale;
  a.out = out;
  a.lse = lse;
  a.split_blocks = ha::decode_split_blocks(full, geo.window, max_kv_len, batch, geo.hkv, num_splits);
  a.splits = ha::decode_num_splits(full, geo.window, max_kv_len, a.split_blocks);
  if (a.splits > 65535) return fail(HA_ERR_RANGE, "too many key splits (%d); pass a smaller num_splits", a.splits);
  if (need > 0) {
    float* ws = static_cast<float*>(workspace);
    a.part_o = ws;
    a.part_lse = ws + static_cast<size_t>(batch) * nq * geo.hq * a.splits * geo.d;
  }
  return hip_status(ha::launch_verify(a, static_cast<hipStream_t>(stream)), "verify launch");
}

size_t hybrid_attn_verify_workspace_size(const ha_shape* shape, int32_t kind, int32_t batch, int32_t max_kv_len,
                                         int32_t nq, int32_t num_splits) {
  ha::Geometry geo;
  if (check_shape(shape, &geo) != HA_OK) return 0;
  if ((kind != HA_SWA && kind != HA_FULL) || batch < 0 || max_kv_len < 0 || num_splits < 0) return 0;
  if (check_nq(geo, nq) != HA_OK) return 0;
  return verify_workspace(geo, kind == HA_FULL, batch, max_kv_len, nq, num_splits);
}

size_t hybrid_attn_workspace_size(const ha_shape* shape, int32_t kind, int32_t decode, int32_t batch,
                                  int32_t max_kv_len, int32_t num_splits) {
  ha::Geometry geo;
  if (check_shape(shape, &geo) != HA_OK) return 0;
  if ((kind != HA_SWA && kind != HA_FULL) || batch < 0 || max_kv_len < 0 || num_splits < 0) return 0;
  if (!decode) return prefill_workspace(geo, kind == HA_FULL, batch, max_kv_len);
  return decode_workspace(geo, kind == HA_FULL, batch, max_kv_len, num_splits);
}

int32_t hybrid_attn_decode_splits(const ha_shape* shape, int32_t kind, int32_t batch, int32_t max_kv_len,
                                  int32_t num_splits) {
  ha::Geometry geo;
  if (check_shape(shape, &geo) != HA_OK) return 0;
  if ((kind != HA_SWA && kind != HA_FULL) || batch < 0 || max_kv_len < 0 || num_splits < 0) return 0;
  const bool full = kind == HA_FULL;
  const int sb = ha::decode_split_blocks(full, geo.window, max_kv_len, batch, geo.hkv, num_splits);
  return ha::decode_num_splits(full, geo.window, max_kv_len, sb);
}

const char* ha_status_str(int32_t status) {
  switch (status) {
    case HA_OK: return "HA_OK";
    case HA_ERR_NULL: return "HA_ERR_NULL";
    case HA_ERR_SHAPE: return "HA_ERR_SHAPE";
    case HA_ERR_RANGE: return "HA_ERR_RANGE";
    case HA_ERR_WORKSPACE: return "HA_ERR_WORKSPACE";
    case HA_ERR_UNSUPPORTED: return "HA_ERR_UNSUPPORTED";
    case HA_ERR_HIP: return "HA_ERR_HIP";
    default: return "HA_ERR_UNKNOWN";
  }
}

const char* ha_last_error(void) { return g_last_error.c_str(); }

int32_t ha_abi_version(void) { return HA_ABI_VERSION; }

}  // extern "C"
