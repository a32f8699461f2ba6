// Host-side work plan for lazyattn_decode_planned: decode work cut at
// document boundaries, with the sequences that share a cached document
// reading it together.
//
// A position-free cache keeps one physical copy of a document for every
// request that places it, at any position (gist.science, "Resumo Técnico:
// LazyAttention", "Metodologia"; the Zipf-skewed reuse of "Resultados
// Experimentais").  Per-sequence decode reads that copy once per sequence.
// Here each sequence's table is cut into runs (one document each, where the
// table allows); the runs of up to kPlanMembers sequences that hold the same
// blocks (wherever they sit in each row) become one work item, whose
// workgroup reads those blocks once for all of them (its 16 matrix-core columns are (sequence, query head)
// pairs).  Items of one (document, KV head) go to the same XCD (workgroup i
// runs on XCD i mod 8) in consecutive places, so the L2 of that XCD serves
// the document's further readers.  Every run writes a split-K partial into
// its own slot, which the combine kernel merges per sequence.
#include "lazyattn.h"

#include <stddef.h>

#include <algorithm>
#include <map>
#include <vector>

namespace {

constexpr int kBlockTokens = 16;
constexpr int kXcds = 8;
constexpr int kMinItemBlocks = 4;        // a document edge cuts a run once it holds this many blocks
constexpr int kDefaultItemBlocks = 128;  // documents up to 2048 tokens stay whole
constexpr int kItemCost = 2;             // a workgroup's fixed cost, in blocks
constexpr int kPlanMembers = 4;          // sequences per item at most
constexpr int kPlanInts = 12;            // ints per item

struct Run {
  int b, slot, blk0, blk1;  // blocks [blk0, blk1) of sequence b's row
  bool one_offset;          // the same offset throughout
  bool last;                // the sequence's last run
  bool shareable() const { return one_offset && !last; }
};

struct Item {
  int g, blk0, blk1, weight;
  int nmem;
  uint32_t mem[kPlanMembers];  // sequence | slot << 16
  int start[kPlanMembers];     // where the run starts in each member's row
  long long key;               // first block id (or a unique negative id)
};

inline int word_offset(uint32_t w) { return (int)(w >> 16); }
inline uint32_t word_block(uint32_t w) { return w & 0xffffu; }

}  // namespace

extern "C" size_t lazyattn_decode_plan_ints(int batch, int max_blocks_per_seq, int num_kv_heads) {
  if (batch <= 0 || max_blocks_per_seq <= 0 || num_kv_heads <= 0) return 0;
  const size_t counts = ((size_t)batch + 3) / 4 * 4;
  return counts + kPlanInts * (size_t)batch * (size_t)max_blocks_per_seq * (size_t)num_kv_heads;
}

extern "C" int lazyattn_decode_plan(const uint32_t *block_table, const int32_t *seq_lens, int batch,
                                    int max_blocks_per_seq, int num_q_heads, int num_kv_heads,
                                    int max_item_blocks, int32_t *plan, size_t plan_ints, int *num_items,
                                    int *max_items_per_seq) {
  if (batch < 1 || batch > 65535 || num_kv_heads < 1 || num_kv_heads > 65535 || num_q_heads < 1 ||
      num_q_heads % num_kv_heads || num_q_heads / num_kv_heads > 16 ||
      ((num_q_heads / num_kv_heads) & (num_q_heads / num_kv_heads - 1)) || max_blocks_per_seq < 1 ||
      max_blocks_per_seq > LAZYATTN_MAX_POSITION / LAZYATTN_BLOCK_TOKENS + 1 || max_item_blocks < 0 ||
      max_item_blocks > 4096)
    return LAZYATTN_ERR_SHAPE;
  if (!block_table || !seq_lens || !plan || !num_items || !max_items_per_seq) return LAZYATTN_ERR_NULL;
  const int item_max = max_item_blocks ? max_item_blocks : kDefaultItemBlocks;
  const int group = num_q_heads / num_kv_heads;
  const int members = std::min(kPlanMembers, 16 / group);

  // 1. each sequence's table cut into runs: a new run where the offset
  // changes (a document edge) once the run holds kMinItemBlocks blocks, and
  // wherever a run reaches item_max.  An empty (or invalid-length) sequence
  // keeps one empty run, through which the kernel writes its zeros (or NaN).
  std::vector<Run> runs;
  std::vector<int> counts((size_t)batch, 0);
  int max_items = 1;
  for (int b = 0; b < batch; ++b) {
    const int len = seq_lens[b];
    const int nblk =
        (len < 0 || len > max_blocks_per_seq * kBlockTokens) ? 0 : (len + kBlockTokens - 1) / kBlockTokens;
    const uint32_t *row = block_table + (size_t)b * max_blocks_per_seq;
    const size_t first = runs.size();
    int start = 0;
    bool one_offset = true;
    for (int j = 1; j <= nblk; ++j) {
      const bool edge = j < nblk && word_offset(row[j]) != word_offset(row[j - 1]);
      const int run = j - start;
      if (j == nblk || (edge && run >= kMinItemBlocks) || run >= item_max) {
        runs.push_back(Run{b, (int)(runs.size() - first), start, j, one_offset, false});
        start = j;
        one_offset = true;
      } else if (edge) {
        one_offset = false;
      }
    }
    if (runs.size() == first) runs.push_back(Run{b, 0, 0, 0, true, false});
    runs.back().last = true;  // grows with the sequence
    counts[b] = (int)(runs.size() - first);
    max_items = std::max(max_items, counts[b]);
  }

  // 2. runs that hold the same blocks (shareable ones) become items of up to
  // `members` sequences; every other run is an item of its own
  std::map<std::vector<uint32_t>, std::vector<int>> same;
  std::vector<std::vector<int>> sets;
  for (int r = 0; r < (int)runs.size(); ++r) {
    const Run &u = runs[(size_t)r];
    if (members > 1 && u.shareable()) {
      const uint32_t *row = block_table + (size_t)u.b * max_blocks_per_seq;
      std::vector<uint32_t> ids((size_t)(u.blk1 - u.blk0));
      for (int j = u.blk0; j < u.blk1; ++j) ids[(size_t)(j - u.blk0)] = word_block(row[j]);
      same[ids].push_back(r);
    } else {
      sets.push_back(std::vector<int>{r});
    }
  }
  for (auto &kv : same)
    for (size_t i = 0; i < kv.second.size(); i += (size_t)members)
      sets.emplace_back(kv.second.begin() + (long)i,
                        kv.second.begin() + (long)std::min(kv.second.size(), i + (size_t)members));
  std::vector<Item> items;
  for (const auto &set : sets) {
    const Run &u = runs[(size_t)set[0]];
    const uint32_t *row = block_table + (size_t)u.b * max_blocks_per_seq;
    Item it{};
    it.blk0 = u.blk0;
    // a last run reaches the end of the row: the kernel clips it to the
    // sequence's length, so the plan stays valid while the sequence grows
    // into blocks appended to its row
    it.blk1 = u.last ? max_blocks_per_seq : u.blk1;
    it.weight = u.blk1 - u.blk0 + kItemCost;
    it.nmem = (int)set.size();
    for (int k = 0; k < it.nmem; ++k) {
      const Run &v = runs[(size_t)set[(size_t)k]];
      it.mem[k] = (uint32_t)v.b | ((uint32_t)v.slot << 16);
      it.start[k] = v.blk0;
    }
    it.key = u.blk1 > u.blk0 ? (long long)word_block(row[u.blk0]) : -1 - (long long)u.b;
    for (int g = 0; g < num_kv_heads; ++g) {
      it.g = g;
      items.push_back(it);
    }
  }
  const size_t base = ((size_t)batch + 3) / 4 * 4;
  if (plan_ints < base + kPlanInts * items.size() || items.size() > 0x7fffffffu) return LAZYATTN_ERR_WORKSPACE;

  // 3. groups: the items of one (first block, KV head), heaviest first, each
  // to the least loaded XCD so far
  std::vector<int> order(items.size());
  for (size_t i = 0; i < items.size(); ++i) order[i] = (int)i;
  std::sort(order.begin(), order.end(), [&](int x, int y) {
    if (items[(size_t)x].key != items[(size_t)y].key) return items[(size_t)x].key < items[(size_t)y].key;
    if (items[(size_t)x].g != items[(size_t)y].g) return items[(size_t)x].g < items[(size_t)y].g;
    return x < y;
  });
  struct Group {
    long long weight = 0;
    std::vector<int> items;
  };
  std::vector<Group> groups;
  for (size_t i = 0; i < order.size(); ++i) {
    const Item &it = items[(size_t)order[i]];
    if (i == 0 || it.key != items[(size_t)order[i - 1]].key || it.g != items[(size_t)order[i - 1]].g)
      groups.emplace_back();
    groups.back().items.push_back(order[i]);
    groups.back().weight += it.weight;
  }
  std::stable_sort(groups.begin(), groups.end(),
                   [](const Group &x, const Group &y) { return x.weight > y.weight; });
  std::vector<std::vector<int>> queue(kXcds);
  long long load[kXcds] = {};
  for (const Group &gr : groups) {
    int x = 0;
    for (int c = 1; c < kXcds; ++c)
      if (load[c] < load[x]) x = c;
    load[x] += gr.weight;
    queue[(size_t)x].insert(queue[(size_t)x].end(), gr.items.begin(), gr.items.end());
  }

  // 4. workgroup i takes the next item of XCD i mod 8's queue; a queue that
  // has run dry borrows from the fullest one
  for (int b = 0; b < batch; ++b) plan[b] = counts[(size_t)b];
  for (size_t i = (size_t)batch; i < base; ++i) plan[i] = 0;
  size_t head[kXcds] = {};
  for (size_t p = 0; p < items.size(); ++p) {
    int x = (int)(p % kXcds);
    if (head[x] == queue[(size_t)x].size()) {
      for (int c = 0; c < kXcds; ++c)
        if (queue[(size_t)c].size() - head[c] > queue[(size_t)x].size() - head[x]) x = c;
    }
    const Item &it = items[(size_t)queue[(size_t)x][head[x]++]];
    int32_t *dst = plan + base + kPlanInts * p;
    dst[0] = (int32_t)((uint32_t)it.g | ((uint32_t)it.nmem << 16));
    dst[1] = it.blk0;
    dst[2] = it.blk1;
    dst[3] = 0;
    for (int k = 0; k < kPlanMembers; ++k) {
      dst[4 + k] = k < it.nmem ? (int32_t)it.mem[k] : 0;
      dst[8 + k] = k < it.nmem ? it.start[k] : 0;
    }
  }
  *num_items = (int)items.size();
  *max_items_per_seq = max_items;
  return LAZYATTN_OK;
}
