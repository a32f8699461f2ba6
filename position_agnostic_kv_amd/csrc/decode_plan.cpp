// Host-side work plan for lazyattn_decode_planned: decode work cut at
// document boundaries and ordered so that the sequences that share a cached
// document read it at the same time on one XCD.
//
// A position-free cache keeps one physical copy of a document for every
// request that places it, at any position (gist.science, "Resumo Técnico:
// LazyAttention", "Metodologia"; the Zipf-skewed reuse of "Resultados
// Experimentais").  Per-sequence decode reads that copy once per sequence.
// Here each (sequence, document, KV head) is one work item; items of one
// (document, KV head) go to the same XCD (workgroup i runs on XCD i mod 8)
// in consecutive places, so the first reader brings the blocks into that
// XCD's L2 and the others find them there.  Items write split-K partials
// (one slot per document of a sequence), which the combine kernel merges.
#include "lazyattn.h"

#include <stddef.h>

#include <algorithm>
#include <vector>

namespace {

constexpr int kBlockTokens = 16;
constexpr int kXcds = 8;
constexpr int kMinItemBlocks = 4;       // shorter runs join their neighbour
constexpr int kDefaultItemBlocks = 128;  // documents up to 2048 tokens stay whole
constexpr int kItemCost = 2;            // a workgroup's fixed cost, in blocks

struct Item {
  int b, g, slot, blk0, blk1;
  int blocks;  // blocks the item reads now (its weight)
};

struct Group {
  long long key;              // first block id (shared) or a unique negative id
  int g;                      // KV head
  long long weight = 0;       // blocks + fixed cost of its items
  std::vector<int> items;     // indices into the item list
};

inline int word_offset(uint32_t w) { return (int)(w >> 16); }

}  // namespace

extern "C" size_t lazyattn_decode_plan_ints(int batch, int max_blocks_per_seq, int num_kv_heads) {
  if (batch <= 0 || max_blocks_per_seq <= 0 || num_kv_heads <= 0) return 0;
  const size_t counts = ((size_t)batch + 3) / 4 * 4;
  return counts + 4 * (size_t)batch * (size_t)max_blocks_per_seq * (size_t)num_kv_heads;
}

extern "C" int lazyattn_decode_plan(const uint32_t *block_table, const int32_t *seq_lens, int batch,
                                    int max_blocks_per_seq, int num_kv_heads, int max_item_blocks,
                                    int32_t *plan, size_t plan_ints, int *num_items, int *max_items_per_seq) {
  if (batch < 1 || batch > 65535 || num_kv_heads < 1 || num_kv_heads > 65535 || max_blocks_per_seq < 1 ||
      max_blocks_per_seq > LAZYATTN_MAX_POSITION / LAZYATTN_BLOCK_TOKENS + 1 || max_item_blocks < 0 ||
      max_item_blocks > 4096)
    return LAZYATTN_ERR_SHAPE;
  if (!block_table || !seq_lens || !plan || !num_items || !max_items_per_seq) return LAZYATTN_ERR_NULL;
  const int item_max = max_item_blocks ? max_item_blocks : kDefaultItemBlocks;

  // 1. each sequence's table cut into runs: a new run where the offset
  // changes (a document boundary), once the run holds kMinItemBlocks blocks,
  // and wherever a run reaches item_max; a short last run joins the one
  // before it.  An empty (or invalid-length) sequence keeps one empty run,
  // through which the kernel writes its zeros (or NaN).
  std::vector<Item> items;
  std::vector<int> counts((size_t)batch, 0);
  std::vector<long long> keys;  // per run (of the item list's first head)
  std::vector<std::pair<int, int>> runs;
  int max_items = 1;
  for (int b = 0; b < batch; ++b) {
    const int len = seq_lens[b];
    const int nblk = (len < 0 || len > max_blocks_per_seq * kBlockTokens) ? 0 : (len + kBlockTokens - 1) / kBlockTokens;
    const uint32_t *row = block_table + (size_t)b * max_blocks_per_seq;
    runs.clear();
    if (nblk == 0) {
      runs.emplace_back(0, 0);
    } else {
      int start = 0;
      for (int j = 1; j < nblk; ++j) {
        const int run = j - start;
        if ((word_offset(row[j]) != word_offset(row[j - 1]) && run >= kMinItemBlocks) || run >= item_max) {
          runs.emplace_back(start, j);
          start = j;
        }
      }
      runs.emplace_back(start, nblk);
      if (runs.size() > 1 && runs.back().second - runs.back().first < kMinItemBlocks) {
        runs[runs.size() - 2].second = nblk;
        runs.pop_back();
      }
    }
    counts[b] = (int)runs.size();
    max_items = std::max(max_items, counts[b]);
    for (int s = 0; s < (int)runs.size(); ++s) {
      const long long key = nblk == 0 ? -1 - (long long)b : (long long)(row[runs[s].first] & 0xffffu);
      // the last run reaches the end of the table row: the kernel clips it
      // to the sequence's length, so the plan stays valid while the
      // sequence grows into blocks appended to its row
      const int end = s + 1 == (int)runs.size() ? max_blocks_per_seq : runs[s].second;
      for (int g = 0; g < num_kv_heads; ++g) {
        items.push_back(Item{b, g, s, runs[s].first, end, runs[s].second - runs[s].first});
        keys.push_back(key);
      }
    }
  }
  const size_t base = ((size_t)batch + 3) / 4 * 4;
  if (plan_ints < base + 4 * items.size() || items.size() > 0x7fffffffu) return LAZYATTN_ERR_WORKSPACE;

  // 2. groups: the items of one (first block, KV head); heaviest first
  std::vector<int> order(items.size());
  for (size_t i = 0; i < items.size(); ++i) order[i] = (int)i;
  std::sort(order.begin(), order.end(), [&](int x, int y) {
    if (keys[x] != keys[y]) return keys[x] < keys[y];
    if (items[x].g != items[y].g) return items[x].g < items[y].g;
    return x < y;
  });
  std::vector<Group> groups;
  for (size_t i = 0; i < order.size(); ++i) {
    const int it = order[i];
    if (groups.empty() || groups.back().key != keys[it] || groups.back().g != items[it].g) {
      groups.emplace_back();
      groups.back().key = keys[it];
      groups.back().g = items[it].g;
    }
    groups.back().items.push_back(it);
    groups.back().weight += items[it].blocks + kItemCost;
  }
  std::stable_sort(groups.begin(), groups.end(),
                   [](const Group &x, const Group &y) { return x.weight > y.weight; });

  // 3. groups to XCDs, each to the least loaded so far (longest first)
  std::vector<std::vector<int>> queue(kXcds);
  long long load[kXcds] = {};
  for (const Group &gr : groups) {
    int x = 0;
    for (int c = 1; c < kXcds; ++c)
      if (load[c] < load[x]) x = c;
    load[x] += gr.weight;
    queue[x].insert(queue[x].end(), gr.items.begin(), gr.items.end());
  }

  // 4. workgroup i takes the next item of XCD i mod 8's queue; a queue that
  // has run dry borrows from the fullest one
  for (int b = 0; b < batch; ++b) plan[b] = counts[(size_t)b];
  for (size_t i = (size_t)batch; i < base; ++i) plan[i] = 0;
  size_t head[kXcds] = {};
  for (size_t p = 0; p < items.size(); ++p) {
    int x = (int)(p % kXcds);
    if (head[x] == queue[x].size()) {
      for (int c = 0; c < kXcds; ++c)
        if (queue[c].size() - head[c] > queue[x].size() - head[x]) x = c;
    }
    const Item &it = items[(size_t)queue[x][head[x]++]];
    int32_t *dst = plan + base + 4 * p;
    dst[0] = it.b;
    dst[1] = it.g;
    dst[2] = (int32_t)((uint32_t)it.slot | ((uint32_t)it.blk0 << 16));
    dst[3] = it.blk1;
  }
  *num_items = (int)items.size();
  *max_items_per_seq = max_items;
  return LAZYATTN_OK;
}
