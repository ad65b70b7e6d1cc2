// Host split-KV tile planner for dense MLA decode.
//
// Follows the tile-scheduler description on the FlashMLA new-kernel deep-dive
// page (nxmr.cn, section "Tile Scheduler"): count every request's 64-token KV
// blocks, cap each part at payload = ceil(total / parts) + fixed overhead, and
// walk the requests in order, filling parts greedily and cutting a request
// at a block boundary when it does not fit; the per-request piece counts let
// the combine step find each request's partial results.  A pass of our own
// then evens out the pieces of each request that parts hold alone
// (even_runs).  The pages run the walk as a single-warp GPU kernel; here it
// is plain host code, O(batch + parts).
#include "mla_internal.h"

#include <algorithm>
#include <vector>

namespace mla {

// After the walk (not part of the page's rule): the walk cuts a long request
// into pieces of payload - F blocks and a shorter last one.  Where consecutive
// parts each hold a piece of the same request and nothing else, their blocks
// are spread evenly over them (earlier pieces one block longer when the count
// does not divide), so the longest piece is as short as the part count
// allows; only block boundaries inside the run move, so the parts, piece
// indices and split counts stay the walk's.  Measured in graph-replayed
// decode steps on MI355X (A/B on one GPU): 18.7 -> 18.1 us on 16 requests of
// 1-4K tokens at h_q = 16, whose 3 + ... + 3 + 1 block pieces become
// 3 + ... + 2 + 2; 103.9 -> 102.3 us (split-KV kernel 85.3 -> 83.0) on 64
// requests of 4K tokens at h_q = 128, where 17 + 17 + 17 + 13 becomes 4 x 16.
static void even_runs(int32_t* sched, int np) {
  for (int p = 0; p < np;) {
    const int32_t* row = sched + (size_t)p * MLA_SCHED_INTS;
    const int r = row[0];
    int q = p;   // the run: parts p .. q - 1 hold request r alone
    while (q < np && sched[(size_t)q * MLA_SCHED_INTS] == r && sched[(size_t)q * MLA_SCHED_INTS + 1] == r) ++q;
    if (q - p >= 2) {
      const int start = row[2], end = sched[(size_t)(q - 1) * MLA_SCHED_INTS + 3];
      const int k = q - p, base = (end - start) / k, extra = (end - start) % k;
      int at = start;
      for (int i = 0; i < k; ++i) {
        int32_t* ri = sched + (size_t)(p + i) * MLA_SCHED_INTS;
        ri[2] = at;
        at += base + (i < extra ? 1 : 0);
        ri[3] = at;
      }
    }
    p = q > p ? q : p + 1;
  }
}

int plan(const int32_t* seqlens, int batch, int num_parts, int fixed_overhead, int force_splits,
         int32_t* sched, int max_parts, int32_t* num_splits, int* parts_out) {
  if (!seqlens || !sched || !num_splits || !parts_out)
    return set_error(MLA_ERR_INVALID, "mla_plan: null pointer argument");
  if (batch <= 0 || num_parts <= 0 || fixed_overhead < 0 || force_splits < 0)
    return set_error(MLA_ERR_INVALID, "mla_plan: batch=%d num_parts=%d fixed_overhead=%d force_splits=%d",
                     batch, num_parts, fixed_overhead, force_splits);
  std::vector<int> n(batch);
  for (int b = 0; b < batch; ++b) {
    if (seqlens[b] < 0) return set_error(MLA_ERR_INVALID, "mla_plan: cache_seqlens[%d] = %d < 0", b, seqlens[b]);
    n[b] = pages_of(seqlens[b]);
  }
  std::vector<int> pieces(batch, 0);
  int np = 0;
  auto emit = [&](int br, int er, int bb, int eb, int bp) -> bool {
    if (np >= max_parts) return false;
    int32_t* row = sched + (size_t)np * MLA_SCHED_INTS;
    row[0] = br; row[1] = er; row[2] = bb; row[3] = eb; row[4] = bp;
    row[5] = row[6] = row[7] = 0;
    ++np;
    return true;
  };
  if (force_splits > 0) {
    for (int r = 0; r < batch; ++r) {
      int cnt = std::max(1, std::min(force_splits, n[r]));
      int q = n[r] / cnt, extra = n[r] % cnt, start = 0;
      for (int i = 0; i < cnt; ++i) {
        int size = q + (i < extra ? 1 : 0);
        if (!emit(r, r, start, start + size, i))
          return set_error(MLA_ERR_CAPACITY, "mla_plan: more than max_parts=%d parts", max_parts);
        start += size;
      }
      pieces[r] = cnt;
    }
  } else {
    const long long F = fixed_overhead;
    long long total = 0;
    for (int b = 0; b < batch; ++b) total += n[b] + F;
    const long long payload = (total + num_parts - 1) / num_parts + F;
    int req = 0, blk = 0;
    for (int p = 0; p < num_parts && req < batch; ++p) {
      const bool last_part = (p == num_parts - 1);
      long long cap = payload;
      const int br = req, bb = blk, bp = pieces[req];
      int er = -1, eb = -1;
      while (req < batch) {
        const long long rem = n[req] - blk;
        if (last_part || rem + F <= cap) {   // the rest of this request fits
          cap -= rem + F;
          pieces[req] += 1;
          er = req; eb = n[req];
          ++req; blk = 0;
          continue;
        }
        const long long take = cap - F;
        if (take > 0) {                      // cut the request at a block boundary
          blk += (int)take;
          pieces[req] += 1;
          er = req; eb = blk;
        }
        break;
      }
      if (er < 0) continue;
      if (!emit(br, er, bb, eb, bp))
        return set_error(MLA_ERR_CAPACITY, "mla_plan: more than max_parts=%d parts", max_parts);
    }
  }
  if (force_splits == 0) even_runs(sched, np);
  num_splits[0] = 0;
  int max_pieces = 0;
  for (int b = 0; b < batch; ++b) {
    num_splits[b + 1] = num_splits[b] + pieces[b];
    max_pieces = std::max(max_pieces, pieces[b]);
  }
  for (int p = 0; p < np; ++p) sched[(size_t)p * MLA_SCHED_INTS + 5] = max_pieces;
  *parts_out = np;
  return MLA_OK;
}

// Column 6 of every row: 1 + the block id of the part's first page (page
// begin_block of begin_req) when that piece holds at least one page, else 0.
// The split-KV kernels then start that page's copy as soon as they have read
// the row, without waiting for the request's block-table entry.
int attach_pages(int32_t* sched, int num_parts, const int32_t* seqlens, int batch, const int32_t* block_table,
                 int max_blocks, int num_blocks) {
  if (!sched || !seqlens || !block_table)
    return set_error(MLA_ERR_INVALID, "mla_plan_attach_pages: null pointer argument");
  if (num_parts <= 0 || batch <= 0 || max_blocks <= 0 || num_blocks <= 0)
    return set_error(MLA_ERR_INVALID, "mla_plan_attach_pages: num_parts=%d batch=%d max_blocks=%d num_blocks=%d",
                     num_parts, batch, max_blocks, num_blocks);
  for (int q = 0; q < num_parts; ++q) {
    int32_t* row = sched + (size_t)q * MLA_SCHED_INTS;
    const int br = row[0], er = row[1], bb = row[2], eb = row[3];
    row[6] = 0;
    if (br > er) continue;   // a part with no work
    if (br < 0 || er >= batch || bb < 0 || eb < 0)
      return set_error(MLA_ERR_INVALID, "mla_plan_attach_pages: row %d names requests %d..%d of %d", q, br, er, batch);
    const int end = (br == er) ? eb : pages_of(seqlens[br]);   // end of the part's first piece
    if (bb >= end) continue;                                   // that piece holds no page
    if (bb >= max_blocks)
      return set_error(MLA_ERR_INVALID, "mla_plan_attach_pages: row %d starts at page %d >= max_blocks=%d", q, bb,
                       max_blocks);
    const int id = block_table[(size_t)br * max_blocks + bb];
    if (id < 0 || id >= num_blocks)
      return set_error(MLA_ERR_INVALID, "mla_plan_attach_pages: block_table[%d][%d] = %d outside [0, %d)", br, bb, id,
                       num_blocks);
    row[6] = id + 1;
  }
  return MLA_OK;
}

}  // namespace mla
