// Work plan of a grouped decode (pa_decode_grouped): which sequences of a batch
// share the leading blocks of their block tables, and how the blocks of each
// group split into work items.  Pure host code.
//
// Sequences forked from one prompt point the logical blocks of that prompt at the
// same physical blocks ("理解 vLLM PagedAttention", section 六; "vLLM 核心概念",
// section "内存共享").  Decode reads every cached token of every sequence, so a
// shared block is read once per sharer; a group's work item instead reads it once
// and scores it against the queries of all the group's sequences, which are the
// columns of its matrix-core tile.
//
// Plan layout (int32, see pa.h): a header of 8 ints, 8 ints per group, 4 per
// member, then one int per (group, partition) item pair, the pairs of all groups
// from the most blocks to the fewest.

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <vector>

#include "pa_internal.h"

namespace {

constexpr int32_t kHeader = 8;
constexpr int32_t kGroupInts = 8;
constexpr int32_t kMemberInts = 4;
constexpr int32_t kMaxColumns = 16;            // one matrix-core tile of query columns
constexpr int32_t kPartTokensMin = 512;        // the workspace holds partitions of this length

int64_t parts_512(int32_t max_ctx) { return (static_cast<int64_t>(max_ctx) + kPartTokensMin - 1) / kPartTokensMin; }

}  // namespace

extern "C" {

size_t pa_group_plan_bytes(int32_t num_seqs, int32_t max_context_len) {
  if (num_seqs <= 0 || max_context_len <= 0) return 0;
  const int64_t n = num_seqs;
  return sizeof(int32_t) * static_cast<size_t>(kHeader + (kGroupInts + kMemberInts) * n +
                                               n * parts_512(max_context_len));
}

pa_status pa_group_plan(const int32_t* tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, int32_t max_context_len, int32_t num_heads,
                        int32_t num_kv_heads, int32_t min_items, int32_t* plan, size_t plan_bytes,
                        int32_t* plan_ints) {
  const char* fn = "pa_group_plan";
  pa::clear_error();
  if (!plan_ints) return pa::fail(PA_ERR_INVALID_ARG, "%s: plan_ints is NULL", fn);
  *plan_ints = 0;
  if (!tables || !context_lens || !plan || num_seqs <= 0 || max_blocks_per_seq <= 0 ||
      max_context_len <= 0 || num_kv_heads <= 0 || num_heads <= 0 || num_heads % num_kv_heads)
    return pa::fail(PA_ERR_INVALID_ARG, "%s: bad arguments", fn);
  if (static_cast<int64_t>(max_blocks_per_seq) * PA_BLOCK_SIZE < max_context_len)
    return pa::fail(PA_ERR_INVALID_ARG, "%s: max_blocks_per_seq %d cannot hold %d tokens", fn,
                    max_blocks_per_seq, max_context_len);
  if (plan_bytes < pa_group_plan_bytes(num_seqs, max_context_len))
    return pa::fail(PA_ERR_INVALID_ARG, "%s: plan buffer %zu bytes, %zu needed", fn, plan_bytes,
                    pa_group_plan_bytes(num_seqs, max_context_len));
  const int32_t G = num_heads / num_kv_heads;
  if (G > kMaxColumns) return PA_OK;                // wider query groups: no grouped decode
  const int32_t max_members = kMaxColumns / G;
  const int64_t B = num_seqs;
  std::vector<int32_t> nblk(B);
  for (int64_t b = 0; b < B; ++b) {
    const int32_t c = context_lens[b];
    if (c < 1 || c > max_context_len)
      return pa::fail(PA_ERR_INVALID_ARG, "%s: context length %d of sequence %lld outside [1, %d]",
                      fn, c, static_cast<long long>(b), max_context_len);
    nblk[b] = (c + PA_BLOCK_SIZE - 1) / PA_BLOCK_SIZE;
  }
  auto row = [&](int64_t b) { return tables + b * max_blocks_per_seq; };

  // Candidate groups: sequences whose first block is the same physical block, in
  // sequence order within a group.
  std::vector<int32_t> order(B);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t x, int32_t y) { return row(x)[0] < row(y)[0]; });
  struct Group {
    int32_t first, count;   // members order[first .. first + count)
    int32_t ns;             // leading blocks all members share
  };
  std::vector<Group> groups;
  int64_t saved = 0, total = 0;
  for (int64_t b = 0; b < B; ++b) total += nblk[b];
  for (int64_t i = 0; i < B;) {
    int64_t e = i + 1;
    while (e < B && row(order[e])[0] == row(order[i])[0]) ++e;
    // chunks of at most max_members; each chunk shares its own longest common prefix
    for (int64_t c = i; c < e; c += max_members) {
      const int32_t cnt = static_cast<int32_t>(std::min<int64_t>(max_members, e - c));
      const int32_t m0 = order[c];
      int32_t ns = nblk[m0];
      for (int32_t k = 1; k < cnt; ++k) {
        const int32_t m = order[c + k];
        const int32_t lim = std::min(ns, nblk[m]);
        int32_t j = 0;
        while (j < lim && row(m)[j] == row(m0)[j]) ++j;
        ns = j;
      }
      groups.push_back({static_cast<int32_t>(c), cnt, ns});
      saved += static_cast<int64_t>(ns) * (cnt - 1);
    }
    i = e;
  }
  // Worth it when the shared blocks read once instead of once per sharer are at
  // least a tenth of all block reads.
  if (saved * 10 < total) return PA_OK;

  // The group's block list: its shared blocks, then each member's own blocks in
  // member order.  Partition length: the longest of 256, 128, 64, 32 blocks for
  // which the list gives at least min_items items (over all KV heads), and no group
  // more partitions than the workspace holds states; else the shortest that fits.
  const int64_t ng = static_cast<int64_t>(groups.size());
  std::vector<int64_t> len(ng);
  int64_t max_len = 0;
  for (int64_t g = 0; g < ng; ++g) {
    int64_t L = groups[g].ns;
    for (int32_t k = 0; k < groups[g].count; ++k) L += nblk[order[groups[g].first + k]] - groups[g].ns;
    len[g] = L;
    max_len = std::max(max_len, L);
  }
  const int64_t cap = parts_512(max_context_len);     // states per (sequence, head) in the workspace
  int32_t pb = 0;
  for (int32_t cand = 256; cand >= 32; cand /= 2) {
    if ((max_len + cand - 1) / cand > cap) break;
    pb = cand;
    int64_t items = 0;
    for (int64_t g = 0; g < ng; ++g) items += (len[g] + cand - 1) / cand;
    if (items * num_kv_heads >= min_items) break;
  }
  if (pb == 0) return PA_OK;                          // the groups' lists are too long
  if (max_len > 4095 * static_cast<int64_t>(pb)) return PA_OK;   // item pair: 12-bit partition

  // Write the plan.
  int64_t pairs = 0;
  for (int64_t g = 0; g < ng; ++g) pairs += (len[g] + pb - 1) / pb;
  int32_t* hdr = plan;
  int32_t* gp = plan + kHeader;
  int32_t* mp = gp + kGroupInts * ng;
  int32_t* ip = mp + kMemberInts * B;
  int32_t max_parts = 0;
  for (int64_t g = 0; g < ng; ++g) {
    const Group& gr = groups[g];
    const int32_t parts = static_cast<int32_t>((len[g] + pb - 1) / pb);
    max_parts = std::max(max_parts, parts);
    int32_t ctx_max = 0;
    int32_t off = 0;
    for (int32_t k = 0; k < gr.count; ++k) {
      const int32_t m = order[gr.first + k];
      int32_t* r = mp + kMemberInts * (gr.first + k);
      r[0] = m;
      r[1] = off;
      r[2] = nblk[m];
      r[3] = context_lens[m];
      off += nblk[m] - gr.ns;
      ctx_max = std::max(ctx_max, context_lens[m]);
    }
    int32_t* r = gp + kGroupInts * g;
    r[0] = gr.first;
    r[1] = gr.count;
    r[2] = gr.ns;
    r[3] = static_cast<int32_t>(len[g]);
    r[4] = parts;
    r[5] = ctx_max;
    r[6] = r[7] = 0;
  }
  // item pairs: (group, partition), partitions with the most blocks first (full ones,
  // then the last ones by size), groups in order within a size
  std::vector<int64_t> keys;
  keys.reserve(pairs);
  for (int64_t g = 0; g < ng; ++g) {
    const int32_t parts = gp[kGroupInts * g + 4];
    for (int32_t p = 0; p < parts; ++p) {
      const int64_t blocks = std::min<int64_t>(pb, len[g] - static_cast<int64_t>(p) * pb);
      keys.push_back(((pb - blocks) << 40) | (g << 12) | p);
    }
  }
  std::sort(keys.begin(), keys.end());
  for (int64_t i = 0; i < pairs; ++i) ip[i] = static_cast<int32_t>(keys[i] & ((int64_t(1) << 40) - 1));
  hdr[0] = static_cast<int32_t>(ng);
  hdr[1] = static_cast<int32_t>(pairs);
  hdr[2] = pb;
  hdr[3] = max_parts;
  hdr[4] = static_cast<int32_t>(B);
  hdr[5] = hdr[6] = hdr[7] = 0;
  *plan_ints = static_cast<int32_t>(kHeader + kGroupInts * ng + kMemberInts * B + pairs);
  return PA_OK;
}

}  // extern "C"
