// Host-side sizing policies shared by the workspace queries (api.cpp) and the
// kernel launchers: how decode splits a sequence's keys over workgroups, and
// how many 16-token blocks prefill's chunk staging needs. Plain host code, so
// the host-only sanitizer build of the library links it unchanged.
#include <climits>

#include "kernels.hpp"

namespace ha {

namespace {
constexpr int kBlockTokens = 16;   // tokens per page / ring block
template <typename T>
T max_of(T a, T b) { return a > b ? a : b; }
template <typename T>
T min_of(T a, T b) { return a < b ? a : b; }
}  // namespace

// Workspace of hybrid_attn_prefill: sequence b's staged blocks start at
// ceil(cu_new[b] / 16) + b, so every sequence's first block is its own.
int64_t prefill_stage_blocks(int num_tokens, int batch) {
  return (static_cast<int64_t>(num_tokens) + kBlockTokens - 1) / kBlockTokens + batch;
}

// Full-layer prefill split. A call's work items are whole query blocks of
// different key counts, list-scheduled over each XCD's 32 CUs.
//  * More than 32 items per XCD: the last round leaves CUs idle while the
//    final items finish. A simulation with the kernel's measured per-item and
//    per-tile costs puts that at about 2% of the full layers of the chunked
//    workload (4 x 32768 tokens, 8192-token chunks). Running each XCD's last
//    12 items in two key parts, the final 4 of them in four, brings it to
//    0.4%; over chunk sizes of 3000 to 16384 tokens and 2 or 4 sequences the
//    same rule averaged 1.3% against 2.6% unsplit (every split part counted
//    with the per-item fixed cost).
//  * At most 16 items per XCD (short chunks of few sequences over long
//    histories): most CUs would have no item at all, so every item is split,
//    into 32 / items parts (the first, heaviest, one more): one round of 32
//    workgroups.
//  * 17 to 21 items: one round of whole items leaves 11 to 15 CUs idle, and
//    the round lasts a whole item. In three parts each, the items take two
//    rounds of a third: 2/3 of the time.
//  * 22 to 32 items: two rounds of parts would need more than three parts
//    for some items, or end no earlier than a whole item; items stay whole.
void prefill_split_policy(int64_t items_per_xcd, int* n1, int* p1, int* n2, int* p2) {
  constexpr int kCusPerXcd = 32;
  *n1 = *p1 = *n2 = *p2 = 0;
  if (items_per_xcd <= 0) return;
  const int items = static_cast<int>(min_of<int64_t>(items_per_xcd, 1 << 20));
  if (items <= kCusPerXcd / 2) {
    const int parts = kCusPerXcd / items;              // >= 2
    *n1 = kCusPerXcd - items * parts;                  // heaviest items get one more part
    *p1 = parts + 1;
    *n2 = items - *n1;
    *p2 = parts;
  } else if (3 * items <= kPrefillPartsPerXcd) {
    *n2 = items;
    *p2 = 3;
  } else if (items > kCusPerXcd) {
    const int tail = min_of(12, items / 4);
    const int quads = tail / 3;
    *n1 = tail - quads;
    *p1 = 2;
    *n2 = quads;
    *p2 = 4;
  }
}

int64_t prefill_partial_bytes(int d) {
  return static_cast<int64_t>(kPrefillPartEntries) * kPrefillFullRows * (d + 1) * 4;
}

// Split policy. Every split of the longest sequence is equally long. Decode
// is bound by HBM, and two resident 4-wave workgroups per CU already keep a
// CU's share of the bandwidth busy (measured: a third one adds nothing), so
// a round is 256 CUs x 2 workgroups. The split count minimises
// (rounds) x (blocks per workgroup + a fixed cost), plus the merge's cost
// when there is more than one split (the reduce launch and the partial rows,
// about 8 blocks' worth at full load on MI355X). Equal workgroups and whole rounds avoid
// a tail of partly idle CUs. When one split per sequence cannot give every
// CU two workgroups, workgroups are capped at 208 blocks (1.6 MiB of K/V) so
// ragged batches still spread over the chip. (Ragged decode workload, 24
// sequences of 1K to 1M tokens, full-layer call on one MI355X: 224 splits
// of up to 256 blocks 2651 us; 255 to 320 splits 2547 to 2575 us.)
// Batches with enough pairs for every CU are capped at 1024 blocks (8 MiB)
// per workgroup. The policy sees only the longest sequence, and a batch of
// many short sequences plus one long one would otherwise leave the long
// sequence to its own Hkv workgroups (one MI355X: 255 one-token sequences
// and one of 900K tokens took 14.9 ms in one split per sequence, 0.79 ms
// with the cap (55 splits), 0.63 ms for the long sequence alone); the
// decode workload's 513-block sequences stay at one split.
int decode_split_blocks(bool full, int window, int max_kv_len, int batch, int hkv, int requested_splits) {
  if (!full) return (window + kBlockTokens - 1) / kBlockTokens;
  const int nblk = (max_of(max_kv_len, 1) + kBlockTokens - 1) / kBlockTokens;
  if (requested_splits > 0) return max_of(1, (nblk + requested_splits - 1) / requested_splits);
  constexpr int64_t kSlots = 256 * 2;
  constexpr int kMaxBlocks = 208, kMaxBlocksFilled = 1024, kMinBlocks = 4, kFixedCost = 4, kMergeCost = 8;
  const int64_t pairs = static_cast<int64_t>(max_of(batch, 1)) * max_of(hkv, 1);
  const int cap = pairs >= kSlots ? kMaxBlocksFilled : kMaxBlocks;
  const int s_lo = max_of(1, (nblk + cap - 1) / cap);
  const int s_hi = min_of(max_of(s_lo, nblk / kMinBlocks), s_lo + 512);
  int best_sb = (nblk + s_lo - 1) / s_lo;
  int64_t best_cost = INT64_MAX;
  for (int s = s_lo; s <= s_hi; ++s) {
    const int sb = (nblk + s - 1) / s;
    const int64_t s_eff = (nblk + sb - 1) / sb;
    const int64_t rounds = (pairs * s_eff + kSlots - 1) / kSlots;
    const int64_t cost = rounds * (sb + kFixedCost) + (s_eff > 1 ? kMergeCost : 0);
    if (cost < best_cost) {
      best_cost = cost;
      best_sb = sb;
    }
  }
  return best_sb;
}

int decode_num_splits(bool full, int window, int max_kv_len, int split_blocks) {
  if (!full) return 1;
  const int nblk = (max_of(max_kv_len, 1) + kBlockTokens - 1) / kBlockTokens;
  return (nblk + split_blocks - 1) / split_blocks;
}

}  // namespace ha
