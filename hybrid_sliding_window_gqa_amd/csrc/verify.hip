// Multi-token verify decode: nq new tokens per sequence (the positions a
// multi-token-prediction head proposed) attend causally among themselves and
// to the sequence's history in one launch, then are appended to the pool.
// The pages run a three-layer MTP head and verify its 1 + 3 tokens per step
// (htx.com "Xiaomi MiMo's 99% price cut ..." section 工程六; blog.hotdry.top
// 2026-06-09 "MTP 与多模态流水线"). Decode stays bound by the KV it reads
// (youleyou.com "小米MiMo首次公开模型推理系统全链路优化降价99%" section 1), so
// verifying nq tokens costs about one decode step: the K/V bytes are the same
// and the matrix cores see nq times the columns.
//
// Sequence b's new tokens sit at positions t0 .. t0 + nq - 1, t0 = kv_len[b] -
// nq. The pool holds positions < t0; the new tokens' K/V come from k_new /
// v_new. Query token i sees keys [0, t0 + i] (full) or [t0 + i - W + 1,
// t0 + i] (SWA).
//
// Workgroup = one (split, kv head, sequence), 4 waves. The S^T = K Q^T
// columns are (token, head) pairs of the GQA group, 16 per MFMA column group,
// NG groups (nq * G <= 16 * NG). Each wave takes history blocks w, w + 4, ...
// of its split and keeps two in flight (ping-pong operand registers), like
// decode; split 0's wave 0 also consumes one extra block holding the new
// tokens, built from k_new / v_new. The new tokens are not patched into the
// ring slots they will occupy: with nq > 1 an earlier query still needs the
// key a later token overwrites. Every key that does not exist (pool slots at
// or past t0, unwritten ring slots, rows past nq in the new block) has its V
// zeroed and its score masked; per-column masks apply the causal and window
// bounds. Waves merge through LDS; the workgroup writes final rows (one split)
// or partials for verify_reduce_kernel. After the merge barrier, split 0
// writes the new tokens into the pool: nothing in the launch reads those
// slots as keys (they are at or past t0, or, for the ring, read by this
// workgroup only, before the barrier).
//
// INT8 pools (include/hybrid_attn.h): history blocks are loaded as codes and
// scales and widened to the bf16 operands right before use; the K scale
// multiplies the scores and the V scale each probability (P' in two bf16
// parts, as in decode). The new tokens' block is quantized in registers with
// the appends' arithmetic (row absmax butterflies over the lanes that hold a
// K row or a V row), so they attend as the codes they are stored with; the
// append after the merge quantizes them again, one 8-channel chunk per lane,
// with the same operations.
#include <cmath>

#include "common.hpp"
#include "kernels.hpp"

namespace ha {

namespace {

constexpr int kVerifyWaves = 4;
// Slack of the exp2 reference (log2 units); see the consume step.
constexpr float kVerifySlack = 8.0f;

template <int D>
struct VBlock {
  u32x4 k[D / 32];
  u32x2 v[D / 16];
};

template <int D>
__device__ __forceinline__ void vload_block(VBlock<D>& ops, const uint16_t* kp, const uint16_t* vp, int64_t base,
                                            int lane) {
  const bool ok = base >= 0;
  const int64_t b0 = ok ? base : 0;
  const uint32_t bytes = ok ? kBlock * D * 2 : 0;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kp + b0, bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vp + b0, bytes);
#pragma unroll
  for (int m = 0; m < D / 32; ++m) ops.k[m] = buf_load16_stream(rk, 16 * (64 * m + lane));
#pragma unroll
  for (int p = 0; p < D / 32; ++p) {
    const u32x4 w = buf_load16_stream(rv, 16 * (64 * p + lane));
    ops.v[2 * p] = u32x2{w.x, w.y};
    ops.v[2 * p + 1] = u32x2{w.z, w.w};
  }
}

// One history block as loaded: bf16 operands, or INT8 codes and scales.
template <int D, bool kKv8>
struct VBuf;
template <int D>
struct VBuf<D, false> {
  VBlock<D> ops;
};
template <int D>
struct VBuf<D, true> {
  RawBlock8<D> raw;
};

template <int D, bool kKv8>
__device__ __forceinline__ void vload_buf(VBuf<D, kKv8>& b, const VerifyArgs& a, int64_t base, int lane) {
  if constexpr (kKv8) load_block8<D>(b.raw, a.k_pool, a.v_pool, a.k_scale, a.v_scale, base, lane);
  else vload_block<D>(b.ops, a.k_pool, a.v_pool, base, lane);
}

// bf16 bits of an INT8 code (exact).
__device__ __forceinline__ uint32_t code_bf16(uint32_t code) {
  return __float_as_uint(static_cast<float>(static_cast<int8_t>(code))) >> 16;
}

template <bool kF32>
__device__ __forceinline__ uint32_t bf16_at(const void* src, int64_t elem) {
  if constexpr (kF32) return f32_to_bf16_bits(static_cast<const float*>(src)[elem]);
  else return static_cast<const uint16_t*>(src)[elem];
}

// Per-wave softmax state of one column group: lane (q4, c16) holds column c16.
template <int D>
struct ColState {
  float m_run;     // running max (log2 domain), the same in the column's four lanes
  float l_run;     // partial sum over this lane's keys
  f32x4 o[D / 16];
};

}  // namespace

template <int D, bool kFull, bool kF32, int NG, bool kKv8>
__global__ __launch_bounds__(64 * kVerifyWaves, 2) void verify_kernel(VerifyArgs a) {
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int kPad = 4;
  constexpr int kCols = 16 * NG;
  __shared__ float sm_o[kVerifyWaves][kCols][D + kPad];
  __shared__ float sm_m[kVerifyWaves][kCols];
  __shared__ float sm_l[kVerifyWaves][kCols];

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
  // The group is a power of two (1..16, checked at the boundary): column ->
  // (token, head) by shift and mask, not by integer division.
  const int gsh = __builtin_ctz(static_cast<unsigned>(G));
  constexpr int kLog2D = D == 128 ? 7 : 6;
  const int nq = a.nq;

  const int len = a.kv_len[b];
  // The SWA ring id is read beside the length (one memory round trip), and
  // the pointers the first loads need are fetched in the same batch; the
  // compiler-only statement keeps them above the branch below.
  const int ring_id = kFull ? 0 : a.table[b];
  if constexpr (!kFull) asm volatile("" ::"s"(ring_id), "s"(a.q), "s"(a.k_pool), "s"(a.v_pool));
  const int t0 = len - nq;   // position of the first new token
  if (t0 < 0) {
    // kv_len below nq: no valid query position; rows are zero, LSE -inf.
    if (split == 0) {
      for (int e = threadIdx.x; e < nq * G * D; e += blockDim.x) {
        const int i = e >> (gsh + kLog2D);
        const int r = e - i * G * D;
        a.out[((static_cast<int64_t>(b) * nq + i) * hq + g * G) * D + r] = 0.0f;
      }
      for (int e = threadIdx.x; e < nq * G; e += blockDim.x)
        a.lse[(static_cast<int64_t>(b) * nq + (e >> gsh)) * hq + g * G + (e & (G - 1))] = -INFINITY;
    }
    return;
  }

  // Ring slot of the newest history position (t0 - 1), in [0, W).
  const int last_slot = kFull ? 0 : ((t0 - 1) % W + W) % W;

  // History blocks of this split (pool blocks holding positions < t0).
  int first, last, nsplit;
  if constexpr (kFull) {
    const int nblk = min((t0 + kBlock - 1) / kBlock, a.table_stride << a.geo.page_shift);
    nsplit = max(1, min((nblk + a.split_blocks - 1) / a.split_blocks, a.splits));
    first = split * a.split_blocks;
    last = min(nblk, first + a.split_blocks);
  } else {
    nsplit = 1;
    first = 0;
    last = (t0 >= W) ? a.geo.ring / kBlock : (t0 + kBlock - 1) / kBlock;   // ring blocks with a written slot
  }
  if (split >= nsplit) return;
  const int ring = ring_id;
  if constexpr (!kFull) {
    if (ring < 0 || ring >= a.num_blocks) last = first;  // invalid ring id: no history
  }
  const int32_t* page_row = a.table + static_cast<int64_t>(b) * a.table_stride;
  const int psh = a.geo.page_shift;
  auto page_of = [&](int i) -> int { return (kFull && i < last) ? page_row[i >> psh] : -1; };
  auto base_of = [&](int i, int pg) -> int64_t {
    if (i >= last) return -1;
    if constexpr (kFull) {
      if (pg < 0 || pg >= a.num_blocks) return -1;
      return page_block_offset(pg, g, hkv, i & ((1 << psh) - 1), psh, kBlock * D);
    } else {
      return ((static_cast<int64_t>(ring) * hkv + g) * a.geo.ring + kBlock * i) * D;
    }
  };
  // Position of key k (0..15) of history block i, or -1 if that slot holds
  // no key a query can see. Ring slots hold positions [t0 - W, t0) at most;
  // t0 - W is outside every query's window and its slot need not hold it
  // (the caller only has to keep [t0 - W + 1, t0)), so it counts as no key
  // and its V is zeroed like any other missing key's.
  auto hist_pos = [&](int i, int k) -> int {
    if constexpr (kFull) {
      const int p = kBlock * i + k;
      return p < t0 ? p : -1;
    } else {
      const int s = kBlock * i + k;   // ring slot
      if (s >= W) return -1;          // padding slots of the last ring block
      int d = last_slot - s;          // slots back from the newest history position
      if (d < 0) d += W;
      const int p = t0 - 1 - d;
      return (p >= 0 && p > t0 - W) ? p : -1;
    }
  };

  // Columns of group gr: column c = 16 gr + c16 = (token i = c / G, head c % G).
  u32x4 qop[NG][KS];
  int tcol[NG];   // query position of this lane's column (INT_MIN: padding column)
#pragma unroll
  for (int gr = 0; gr < NG; ++gr) {
    const int c = 16 * gr + c16;
    const int i = c >> gsh;
    const bool ok = i < nq;
    tcol[gr] = ok ? t0 + i : -0x40000000;
    if constexpr (kF32) {
      const int64_t qoff = ((static_cast<int64_t>(b) * nq + (ok ? i : 0)) * hq + g * G + (c & (G - 1))) * D + 8 * q4;
#pragma unroll
      for (int m = 0; m < KS; ++m) {
        qop[gr][m] = load8_as_bf16<kF32>(a.q, qoff + 32 * m);
        if (!ok) qop[gr][m] = u32x4{0u, 0u, 0u, 0u};
      }
    } else {
      // One buffer over the sequence's nq query rows; padding columns read
      // past its end and get zeros from the range check (no select that
      // would wait for the load).
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(static_cast<const uint16_t*>(a.q) + static_cast<int64_t>(b) * nq * hq * D,
                                                  static_cast<uint32_t>(nq * hq * D * 2));
      const uint32_t off = ok ? 2u * static_cast<uint32_t>((i * hq + g * G + (c & (G - 1))) * D + 8 * q4) : 0x40000000u;
#pragma unroll
      for (int m = 0; m < KS; ++m) qop[gr][m] = buf_load16(rq, off + 64 * m);
    }
  }

  // The new tokens' K/V elements this thread appends after the merge
  // (element e = threadIdx.x + 256 j of the nq x D rows), loaded up front so
  // that their latency overlaps the attention instead of following the
  // merge. Elements past nq x D read past the buffer's end and get zeros.
  constexpr int kAppendRegs = 4;
  uint32_t app_k[kAppendRegs], app_v[kAppendRegs];
  const bool app_pre = !kF32 && !kKv8 && split == 0 && nq * D <= kAppendRegs * 64 * kVerifyWaves;
  if constexpr (!kF32 && !kKv8) {
    if (app_pre) {
      const int64_t row0 = static_cast<int64_t>(b) * nq * hkv * D;
      const uint32_t bytes = static_cast<uint32_t>(nq * hkv * D * 2);
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<const uint16_t*>(a.k_new) + row0, bytes);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(static_cast<const uint16_t*>(a.v_new) + row0, bytes);
#pragma unroll
      for (int j = 0; j < kAppendRegs; ++j) {
        const int e = threadIdx.x + 64 * kVerifyWaves * j;
        const uint32_t off = e < nq * D ? 2u * static_cast<uint32_t>(((e / D) * hkv + g) * D + e % D) : 0x40000000u;
        app_k[j] = __builtin_amdgcn_raw_buffer_load_b16(rk, off, 0, 0);
        app_v[j] = __builtin_amdgcn_raw_buffer_load_b16(rv, off, 0, 0);
      }
    }
  }

  const float sl2 = a.geo.scale * kLog2e;
  ColState<D> st[NG];
#pragma unroll
  for (int gr = 0; gr < NG; ++gr) {
    st[gr].m_run = -INFINITY;
    st[gr].l_run = 0.0f;
#pragma unroll
    for (int d = 0; d < DT; ++d) st[gr].o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One block: keys at positions kp[r] (key 4 q4 + r; -1: no key), shared
  // by every column group. INT8 pools: ops holds the widened codes, ks / vs
  // the keys' K and V scales (the K scale multiplies the scores, the V scale
  // each probability, l sums the unscaled ones); a key that does not exist
  // gets a zero V scale, so its slot's scale cannot reach O.
  auto consume_ops = [&](VBlock<D>& ops, const int (&kp)[4], const float (&ks)[4], const float (&vs)[4]) {
    float vsk[4];
    if constexpr (kKv8) {
#pragma unroll
      for (int r = 0; r < 4; ++r) vsk[r] = kp[r] >= 0 ? vs[r] : 0.0f;
    } else if (!__all(kp[0] >= 0 && kp[1] >= 0 && kp[2] >= 0 && kp[3] >= 0)) {
      // zero V of keys that do not exist (their pool slots may hold anything);
      // blocks whose keys all exist (every full history block) skip it
      uint32_t keep[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) keep[r] = kp[r] >= 0 ? 0xffffu : 0u;
      const uint32_t mlo = keep[0] | (keep[1] << 16);
      const uint32_t mhi = keep[2] | (keep[3] << 16);
#pragma unroll
      for (int d = 0; d < DT; ++d) {
        ops.v[d].x &= mlo;
        ops.v[d].y &= mhi;
      }
    }
#pragma unroll
    for (int gr = 0; gr < NG; ++gr) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < KS; ++m) s = mfma_16x16x32(ops.k[m], qop[gr][m], s);
      if constexpr (kKv8) {
#pragma unroll
        for (int r = 0; r < 4; ++r) s[r] *= ks[r];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bool ok = kp[r] >= 0 && kp[r] <= tcol[gr];
        if constexpr (!kFull) ok = ok && kp[r] > tcol[gr] - W;
        s[r] = ok ? s[r] : -INFINITY;
      }
      ColState<D>& cs = st[gr];
      // The exp2 reference is raised only when a column's block max passes it
      // by more than kVerifySlack (log2 units): probabilities stay at most
      // 2^kVerifySlack, and O and l are rescaled on those blocks only.
      const float tmax = group4_max(max_prop(max_prop(s[0], s[1]), max_prop(s[2], s[3]))) * sl2;
      if (__any(tmax > cs.m_run + kVerifySlack)) {
        const float m_new = (tmax > cs.m_run + kVerifySlack) ? tmax : cs.m_run;
        const float alpha =
            (m_new == cs.m_run) ? 1.0f : (cs.m_run == -INFINITY ? 0.0f : fast_exp2(cs.m_run - m_new));
        cs.l_run *= alpha;
#pragma unroll
        for (int d = 0; d < DT; ++d) cs.o[d] *= alpha;
        cs.m_run = m_new;
      }
      const float m_use = (cs.m_run == -INFINITY) ? 0.0f : cs.m_run;
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = fast_exp2(s[r] * sl2 - m_use);
      cs.l_run += (p[0] + p[1]) + (p[2] + p[3]);
      if constexpr (kKv8) {
        float pv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pv[r] = p[r] * vsk[r];
        pv8<D>(ops.v, pv, cs.o);
      } else {
        const u32x2 pb = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
#pragma unroll
        for (int d = 0; d < DT; ++d) cs.o[d] = mfma_16x16x16(ops.v[d], pb, cs.o[d]);
      }
    }
  };
  auto consume = [&](VBuf<D, kKv8>& buf, const int (&kp)[4]) {
    if constexpr (kKv8) {
      VBlock<D> ops;
      widen_k8<D>(buf.raw, ops.k);
      widen_v8<D>(buf.raw, ops.v);
      const float ks[4] = {buf.raw.ks[0], buf.raw.ks[1], buf.raw.ks[2], buf.raw.ks[3]};
      const float vs[4] = {buf.raw.vs[0], buf.raw.vs[1], buf.raw.vs[2], buf.raw.vs[3]};
      consume_ops(ops, kp, ks, vs);
    } else {
      const float none[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      consume_ops(buf.ops, kp, none, none);
    }
  };
  auto hist_keys = [&](int i, int (&kp)[4]) {
#pragma unroll
    for (int r = 0; r < 4; ++r) kp[r] = hist_pos(i, 4 * q4 + r);
  };

  // The new tokens as one more block (split 0, wave 0): key k = token k < nq.
  // Its loads go out first and it is consumed first, so its gathers overlap
  // the history loads rather than following them.
  const bool has_new = split == 0 && wave == 0;
  VBlock<D> N;
  // V^T operand of the new block: lane (q4, c16), dim tile d holds tokens
  // 4 q4 .. 4 q4 + 3 of channel 16 d + c16. Packed only right before the
  // block is consumed, so that no wait on these loads precedes the history
  // loads.
  uint16_t vb[4][DT];
  if (has_new) {
    if constexpr (kF32) {
      const bool krow = c16 < nq;
      const int64_t ksrc = ((static_cast<int64_t>(b) * nq + (krow ? c16 : 0)) * hkv + g) * D + 8 * q4;
#pragma unroll
      for (int m = 0; m < KS; ++m) {
        N.k[m] = load8_as_bf16<kF32>(a.k_new, ksrc + 32 * m);
        if (!krow) N.k[m] = u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = 4 * q4 + r;
        const bool ok = tok < nq;
        const int64_t vsrc = ((static_cast<int64_t>(b) * nq + (ok ? tok : 0)) * hkv + g) * D + c16;
#pragma unroll
        for (int d = 0; d < DT; ++d) vb[r][d] = ok ? static_cast<uint16_t>(bf16_at<kF32>(a.v_new, vsrc + 16 * d)) : 0;
      }
    } else {
      // Buffers over the sequence's nq new rows: lanes of tokens >= nq read
      // past the end and get zeros from the range check, so the loads need
      // no branch or select and all of them are in flight at once.
      const int64_t row0 = static_cast<int64_t>(b) * nq * hkv * D;
      const uint32_t bytes = static_cast<uint32_t>(nq * hkv * D * 2);
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<const uint16_t*>(a.k_new) + row0, bytes);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(static_cast<const uint16_t*>(a.v_new) + row0, bytes);
      const uint32_t koff = c16 < nq ? 2u * static_cast<uint32_t>((c16 * hkv + g) * D + 8 * q4) : 0x40000000u;
#pragma unroll
      for (int m = 0; m < KS; ++m) N.k[m] = buf_load16(rk, koff + 64 * m);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = 4 * q4 + r;
        const uint32_t voff = tok < nq ? 2u * static_cast<uint32_t>((tok * hkv + g) * D + c16) : 0x40000000u;
#pragma unroll
        for (int d = 0; d < DT; ++d)
          vb[r][d] = __builtin_amdgcn_raw_buffer_load_b16(rv, voff + 32 * d, 0, 0);
      }
    }
  }

  // History blocks of this wave: first + wave + 4k, two in flight.
  {
    int ia = first + wave;
    int ib = ia + kVerifyWaves;
    int pg_a2 = 0, pg_b2 = 0;
    int64_t base_a = base_of(ia, page_of(ia));
    int64_t base_b = base_of(ib, page_of(ib));
    VBuf<D, kKv8> A, B;
    vload_buf<D, kKv8>(A, a, base_a, lane);
    vload_buf<D, kKv8>(B, a, base_b, lane);
    pg_a2 = page_of(ia + 2 * kVerifyWaves);
    pg_b2 = page_of(ib + 2 * kVerifyWaves);
    if (has_new) {
      // Compiler-only: the values pass through these statements after the
      // history loads above are issued, so the packing (and its wait for the
      // new-token loads) cannot be hoisted in front of them.
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        static_assert(DT == 4 || DT == 8, "pinned as 8 or 4 registers per token");
        if constexpr (DT == 8)
          asm volatile("" : "+v"(vb[r][0]), "+v"(vb[r][1]), "+v"(vb[r][2]), "+v"(vb[r][3]), "+v"(vb[r][4]),
                       "+v"(vb[r][5]), "+v"(vb[r][6]), "+v"(vb[r][7])::"memory");
        else
          asm volatile("" : "+v"(vb[r][0]), "+v"(vb[r][1]), "+v"(vb[r][2]), "+v"(vb[r][3])::"memory");
      }
      float ksn[4] = {0.0f, 0.0f, 0.0f, 0.0f}, vsn[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (kKv8) {
        // INT8 pools: the new tokens attend as the codes and scales they are
        // appended with, computed with append8_kernel's float32 operations.
        // K row of token c16: the 4 lanes of column c16; V row of token
        // 4 q4 + r: element r of the 16 lanes of row group q4.
        float ka = 0.0f;
#pragma unroll
        for (int m = 0; m < KS; ++m) {
          const uint32_t w4[4] = {N.k[m].x, N.k[m].y, N.k[m].z, N.k[m].w};
#pragma unroll
          for (int j = 0; j < 4; ++j)
            ka = max_prop(ka, max_prop(fabsf(__uint_as_float(w4[j] << 16)), fabsf(__uint_as_float(w4[j] & 0xffff0000u))));
        }
        ka = max_prop(ka, __shfl_xor(ka, 16));
        ka = max_prop(ka, __shfl_xor(ka, 32));
        const float ks_tok = ka / 127.0f;
#pragma unroll
        for (int m = 0; m < KS; ++m) {
          uint32_t w4[4] = {N.k[m].x, N.k[m].y, N.k[m].z, N.k[m].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t lo = code_bf16(code8(__uint_as_float(w4[j] << 16), ks_tok));
            const uint32_t hi = code_bf16(code8(__uint_as_float(w4[j] & 0xffff0000u), ks_tok));
            w4[j] = lo | (hi << 16);
          }
          N.k[m] = u32x4{w4[0], w4[1], w4[2], w4[3]};
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          ksn[r] = __shfl(ks_tok, 4 * q4 + r);   // key 4 q4 + r = token of column 4 q4 + r
          float va = 0.0f;
#pragma unroll
          for (int d = 0; d < DT; ++d) va = max_prop(va, fabsf(__uint_as_float(static_cast<uint32_t>(vb[r][d]) << 16)));
#pragma unroll
          for (int mask = 1; mask < 16; mask <<= 1) va = max_prop(va, __shfl_xor(va, mask));
          vsn[r] = va / 127.0f;
#pragma unroll
          for (int d = 0; d < DT; ++d)
            vb[r][d] = static_cast<uint16_t>(code_bf16(code8(__uint_as_float(static_cast<uint32_t>(vb[r][d]) << 16), vsn[r])));
        }
      }
#pragma unroll
      for (int d = 0; d < DT; ++d)
        N.v[d] = u32x2{static_cast<uint32_t>(vb[0][d]) | (static_cast<uint32_t>(vb[1][d]) << 16),
                       static_cast<uint32_t>(vb[2][d]) | (static_cast<uint32_t>(vb[3][d]) << 16)};
      int kpn[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) kpn[r] = (4 * q4 + r < nq) ? t0 + 4 * q4 + r : -1;
      consume_ops(N, kpn, ksn, vsn);
    }
    const int nmine = (last > ia) ? (last - ia + kVerifyWaves - 1) / kVerifyWaves : 0;
    int kp[4];
    for (int k = 0; k + 1 < nmine; k += 2) {
      if (base_a >= 0) {
        hist_keys(ia, kp);
        consume(A, kp);
      }
      ia += 2 * kVerifyWaves;
      base_a = base_of(ia, pg_a2);
      vload_buf<D, kKv8>(A, a, base_a, lane);
      pg_a2 = page_of(ia + 2 * kVerifyWaves);
      if (base_b >= 0) {
        hist_keys(ib, kp);
        consume(B, kp);
      }
      ib += 2 * kVerifyWaves;
      base_b = base_of(ib, pg_b2);
      vload_buf<D, kKv8>(B, a, base_b, lane);
      pg_b2 = page_of(ib + 2 * kVerifyWaves);
    }
    if ((nmine & 1) && base_a >= 0) {
      hist_keys(ia, kp);
      consume(A, kp);
    }
  }

  // Merge the four waves.
#pragma unroll
  for (int gr = 0; gr < NG; ++gr) {
    const float l = group4_sum(st[gr].l_run);
#pragma unroll
    for (int d = 0; d < DT; ++d)
      *reinterpret_cast<f32x4*>(&sm_o[wave][16 * gr + c16][16 * d + 4 * q4]) = st[gr].o[d];
    if (q4 == 0) {
      sm_m[wave][16 * gr + c16] = st[gr].m_run;
      sm_l[wave][16 * gr + c16] = l;
    }
  }
  __syncthreads();

  // Per column: the merged max, the four waves' weights 2^(m_w - mu) / l and
  // the LSE, once; then the rows as float4 weighted sums of the waves' O.
  const bool final_row = (nsplit == 1);
  const int ncols = nq * G;
  __shared__ float sm_f[kVerifyWaves][kCols];
  if (threadIdx.x < ncols) {
    const int c = threadIdx.x;
    float mx = sm_m[0][c];
#pragma unroll
    for (int w = 1; w < kVerifyWaves; ++w) mx = max_prop(mx, sm_m[w][c]);
    const float mu = (mx == -INFINITY) ? 0.0f : mx;
    float f[kVerifyWaves], l = 0.0f;
#pragma unroll
    for (int w = 0; w < kVerifyWaves; ++w) {
      f[w] = fast_exp2(sm_m[w][c] - mu);
      l += sm_l[w][c] * f[w];
    }
    const float inv = 1.0f / l;
#pragma unroll
    for (int w = 0; w < kVerifyWaves; ++w) sm_f[w][c] = f[w] * inv;
    const int64_t row = (static_cast<int64_t>(b) * nq + (c >> gsh)) * hq + g * G + (c & (G - 1));
    const float lse2 = mu + fast_log2(l);
    if (final_row) a.lse[row] = lse2 * kLn2;
    else a.part_lse[row * a.splits + split] = lse2;
  }
  __syncthreads();
  constexpr int kD4 = D / 4;
  for (int e = threadIdx.x; e < ncols * kD4; e += blockDim.x) {
    const int c = e / kD4;
    const int d4 = e - c * kD4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kVerifyWaves; ++w) acc += *reinterpret_cast<const f32x4*>(&sm_o[w][c][4 * d4]) * sm_f[w][c];
    const int64_t row = (static_cast<int64_t>(b) * nq + (c >> gsh)) * hq + g * G + (c & (G - 1));
    float* dst = final_row ? a.out + row * D : a.part_o + (row * a.splits + split) * D;
    *reinterpret_cast<f32x4*>(dst + 4 * d4) = acc;
  }

  // Append the new tokens (split 0; every read of this workgroup is done).
  // Pool block (element offset) and row of new token j, or false when it is
  // not written (no valid page or ring, or a ring slot a later token of this
  // call writes again).
  auto new_slot = [&](int j, int64_t& blk, int& row) -> bool {
    const int p = t0 + j;
    if constexpr (kFull) {
      const int lb = p / kBlock;
      const int pg = (lb >> psh) < a.table_stride ? page_row[lb >> psh] : -1;
      if (pg < 0 || pg >= a.num_blocks) return false;
      blk = page_block_offset(pg, g, hkv, lb & ((1 << psh) - 1), psh, kBlock * D);
      row = p % kBlock;
    } else {
      if (ring < 0 || ring >= a.num_blocks) return false;
      if (j < nq - W) return false;
      const int s = p % W;
      blk = ((static_cast<int64_t>(ring) * hkv + g) * a.geo.ring + kBlock * (s / kBlock)) * D;
      row = s % kBlock;
    }
    return true;
  };
  if constexpr (kKv8) {
    // INT8 pools: append8_kernel's arithmetic, D/8 lanes per token row (one
    // 8-channel chunk each), the row's absmax a butterfly over those lanes.
    if (split == 0) {
      constexpr int kChunks = D / 8;
      constexpr int kRowsPerPass = 64 * kVerifyWaves / kChunks;
      const int c = static_cast<int>(threadIdx.x) % kChunks;
      for (int j = static_cast<int>(threadIdx.x) / kChunks; j < nq; j += kRowsPerPass) {
        int64_t blk;
        int row;
        if (!new_slot(j, blk, row)) continue;   // uniform over the row's lanes
        const int64_t src = ((static_cast<int64_t>(b) * nq + j) * hkv + g) * D + c * 8;
        const u32x4 kraw = load8_as_bf16<kF32>(a.k_new, src);
        const u32x4 vraw = load8_as_bf16<kF32>(a.v_new, src);
        const uint32_t kw[4] = {kraw.x, kraw.y, kraw.z, kraw.w};
        const uint32_t vw[4] = {vraw.x, vraw.y, vraw.z, vraw.w};
        float kx[8], vx[8];
        float ka = 0.0f, va = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kx[2 * e] = __uint_as_float(kw[e] << 16);
          kx[2 * e + 1] = __uint_as_float(kw[e] & 0xffff0000u);
          vx[2 * e] = __uint_as_float(vw[e] << 16);
          vx[2 * e + 1] = __uint_as_float(vw[e] & 0xffff0000u);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ka = max_prop(ka, fabsf(kx[e]));
          va = max_prop(va, fabsf(vx[e]));
        }
#pragma unroll
        for (int mask = kChunks / 2; mask >= 1; mask >>= 1) {
          ka = max_prop(ka, __shfl_xor(ka, mask));
          va = max_prop(va, __shfl_xor(va, mask));
        }
        const float ks = ka / 127.0f;
        const float vs = va / 127.0f;
        uint8_t* kb = reinterpret_cast<uint8_t*>(a.k_pool_w) + blk;
        uint8_t* vbk = reinterpret_cast<uint8_t*>(a.v_pool_w) + blk;
        uint32_t kq[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kq[e >> 2] |= code8(kx[e], ks) << (8 * (e & 3));
          vbk[v8_elem(row, c * 8 + e)] = static_cast<uint8_t>(code8(vx[e], vs));
        }
        *reinterpret_cast<u32x2*>(kb + k8_elem(row, c * 8)) = u32x2{kq[0], kq[1]};
        if (c == 0) {
          a.k_scale[blk / D + row] = ks;
          a.v_scale[blk / D + row] = vs;
        }
      }
    }
    return;
  }
  auto append_elem = [&](int e, uint32_t kv, uint32_t vv) {
    const int j = e / D;
    const int dd = e - j * D;
    int64_t blk;
    int row;
    if (!new_slot(j, blk, row)) return;
    a.k_pool_w[blk + k_elem(row, dd)] = static_cast<uint16_t>(kv);
    a.v_pool_w[blk + v_elem(row, dd)] = static_cast<uint16_t>(vv);
  };
  if (app_pre) {
#pragma unroll
    for (int j = 0; j < kAppendRegs; ++j) {
      const int e = threadIdx.x + 64 * kVerifyWaves * j;
      if (e < nq * D) append_elem(e, app_k[j], app_v[j]);
    }
  } else if (split == 0) {
    for (int e = threadIdx.x; e < nq * D; e += blockDim.x) {
      const int64_t src = ((static_cast<int64_t>(b) * nq + e / D) * hkv + g) * D + e % D;
      append_elem(e, bf16_at<kF32>(a.k_new, src), bf16_at<kF32>(a.v_new, src));
    }
  }
}

// Split-K merge of verify partials: one thread per output element of a
// sequence's nq * Hq rows, splits folded with a running max (log2 domain).
template <int D>
__global__ __launch_bounds__(256) void verify_reduce_kernel(VerifyArgs a) {
  const int b = blockIdx.y;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  const int nq = a.nq;
  if (e >= nq * a.geo.hq * D) return;
  const int t0 = a.kv_len[b] - nq;
  if (t0 < 0) return;
  const int nblk = min((t0 + kBlock - 1) / kBlock, a.table_stride << a.geo.page_shift);
  const int nsplit = max(1, min((nblk + a.split_blocks - 1) / a.split_blocks, a.splits));
  if (nsplit <= 1) return;
  const int r = e / D;               // row of the sequence: token * hq + head
  const int dd = e - r * D;
  const int64_t row = static_cast<int64_t>(b) * nq * a.geo.hq + r;
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
  a.out[row * D + dd] = acc / l;
  if (dd == 0) a.lse[row] = ((m == -INFINITY ? 0.0f : m) + fast_log2(l)) * kLn2;
}

int verify_column_groups(int nq, int group) { return (nq * group + 15) / 16; }

template <int D, bool kFull, int NG>
static void launch_verify_k(const VerifyArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 block(64 * kVerifyWaves);
  if (a.kv8) {
    if (a.in_f32) hipLaunchKernelGGL((verify_kernel<D, kFull, true, NG, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((verify_kernel<D, kFull, false, NG, true>), grid, block, 0, stream, a);
  } else {
    if (a.in_f32) hipLaunchKernelGGL((verify_kernel<D, kFull, true, NG, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((verify_kernel<D, kFull, false, NG, false>), grid, block, 0, stream, a);
  }
}

template <int D>
static hipError_t launch_verify_d(const VerifyArgs& a, hipStream_t stream) {
  const dim3 grid(a.full ? a.splits : 1, a.geo.hkv, a.batch);
  const int ng = verify_column_groups(a.nq, a.geo.group);
  if (a.full) {
    if (ng == 1) launch_verify_k<D, true, 1>(a, grid, stream);
    else launch_verify_k<D, true, 2>(a, grid, stream);
  } else {
    if (ng == 1) launch_verify_k<D, false, 1>(a, grid, stream);
    else launch_verify_k<D, false, 2>(a, grid, stream);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (a.full && a.splits > 1) {
    const dim3 rgrid((a.nq * a.geo.hq * D + 255) / 256, a.batch);
    hipLaunchKernelGGL((verify_reduce_kernel<D>), rgrid, dim3(256), 0, stream, a);
    err = hipGetLastError();
  }
  return err;
}

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream) {
  if (a.batch == 0 || a.nq == 0) return hipSuccess;
  if (a.geo.d == 64) return launch_verify_d<64>(a, stream);
  return launch_verify_d<128>(a, stream);
}

}  // namespace ha
