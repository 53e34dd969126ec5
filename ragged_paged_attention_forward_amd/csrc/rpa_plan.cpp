// Host-side ragged metadata builder.
//
// The pages' kernel keeps a block of queries on chip and streams in every key
// that block attends to, so each key is fetched once per query block that
// wants it; larger query blocks mean fewer re-reads ("Chasing speed of light on
// TPU v6e", section Attention, and footnote 6: the query block grows with the
// query/KV head ratio).  Here a prefill tile packs `prefill_rows` rows of
// (token, grouped query head) that share one KV head, and its key range is
// exactly the union of what those rows can see: causal, clipped by the window.
//
// Decode sequences (one or a few query tokens) are memory-bound at any batch
// ("TPU Deep Dive", chapter 4: decode attention intensity is about G; chapter
// 7: decode is memory-bound), so their key ranges are cut into splits that
// run in parallel and are merged by log-sum-exp afterwards; key ranges follow
// the true lengths, never a padded block ("Pallas Kernel: vLLM on TPU ...", S7:
// oversized KV blocks left most of a decode block as masked padding).
#include "rpa_plan.h"

#include <algorithm>
#include <cstdio>

namespace rpa {

namespace {

std::string fmt(const char* f, long long a, long long b = 0, long long c = 0) {
  char buf[256];
  std::snprintf(buf, sizeof buf, f, a, b, c);
  return buf;
}

int32_t range_begin(int64_t pos0, int32_t window) {
  if (window <= 0) return 0;
  int64_t lo = pos0 - window + 1;
  return lo > 0 ? static_cast<int32_t>(lo) : 0;
}

// Workgroup b of a launch runs on chiplet (XCD) b mod X, and each chiplet has
// its own L2.  Neighbouring items of the sorted list (consecutive query tiles
// of one sequence and KV head) read mostly the same keys.  So within each
// round of `round` launch positions (one workgroup per compute unit), the
// longest-first list is dealt to the chiplets in runs of `run` consecutive
// items: the tiles of a run execute side by side on one chiplet and share
// their K/V through its L2.  The runs go to chiplets 0, 1, .., X-1, then
// X-1, .., 0, and so on, so that every chiplet gets long and short items
// alike and the chiplets' total work stays even; a chiplet whose positions
// are used up passes the run on to the next one.
void interleave_for_chiplets(std::vector<rpa_work_item>* items, int round, int X, int run) {
  const int64_t n = static_cast<int64_t>(items->size());
  if (X <= 1 || round < X || n <= X || run < 1) return;
  std::vector<rpa_work_item> out(items->size());
  std::vector<int64_t> next(X);
  for (int64_t r0 = 0; r0 < n; r0 += round) {
    const int64_t m = std::min<int64_t>(round, n - r0);
    for (int x = 0; x < X; ++x) next[x] = x;   // next free position of chiplet x
    int64_t c = 0;                             // run counter
    int in_run = 0;
    for (int64_t k = 0; k < m; ++k) {
      const int64_t lap = c / X;
      int x = static_cast<int>(lap % 2 == 0 ? c % X : X - 1 - c % X);
      while (next[x] >= m) x = (x + 1) % X;    // free positions remain: m - k > 0
      out[r0 + next[x]] = (*items)[r0 + k];
      next[x] += X;
      if (++in_run == run) {
        in_run = 0;
        ++c;
      }
    }
  }
  items->swap(out);
}

}  // namespace

int validate_metadata(const PlanParams& p, const int32_t* cu, const int32_t* kv,
                      int32_t num_seqs, int32_t window, std::string* err) {
  if (num_seqs < 0 || num_seqs > p.max_num_seqs) {
    *err = fmt("num_seqs %lld outside [0, %lld]", num_seqs, p.max_num_seqs);
    return RPA_ERR_INVALID_ARG;
  }
  if (window < 0) {
    *err = fmt("window %lld is negative", window);
    return RPA_ERR_INVALID_ARG;
  }
  if (cu == nullptr || (num_seqs > 0 && kv == nullptr)) {
    *err = "cu_q_lens / kv_lens is NULL";
    return RPA_ERR_INVALID_ARG;
  }
  if (cu[0] != 0) {
    *err = fmt("cu_q_lens[0] = %lld, must be 0", cu[0]);
    return RPA_ERR_INVALID_ARG;
  }
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t q_len = static_cast<int64_t>(cu[s + 1]) - cu[s];
    if (q_len < 0) {
      *err = fmt("cu_q_lens decreases at sequence %lld", s);
      return RPA_ERR_INVALID_ARG;
    }
    if (kv[s] < 0) {
      *err = fmt("kv_lens[%lld] = %lld is negative", s, kv[s]);
      return RPA_ERR_INVALID_ARG;
    }
    if (q_len > kv[s]) {
      *err = fmt("sequence %lld: q_len %lld exceeds kv_len %lld", s, q_len, kv[s]);
      return RPA_ERR_INVALID_ARG;
    }
    const int64_t pages = (static_cast<int64_t>(kv[s]) + p.page_size - 1) / p.page_size;
    if (pages > p.max_pages_per_seq) {
      *err = fmt("sequence %lld needs %lld pages, max_pages_per_seq is %lld", s, pages,
                 p.max_pages_per_seq);
      return RPA_ERR_INVALID_ARG;
    }
  }
  if (cu[num_seqs] > p.max_q_tokens) {
    *err = fmt("%lld query tokens exceed max_q_tokens %lld", cu[num_seqs], p.max_q_tokens);
    return RPA_ERR_INVALID_ARG;
  }
  return RPA_OK;
}

// Long prefill items (the last query tiles of a long chunk) can outlast the
// rest of the launch by far, with most compute units idle.  Such an item is
// cut along its key range into splits that each write a partial result
// (normalised O and log-sum-exp per row); the merge kernel that follows the
// prefill launch combines them (several workgroups per group).  Automatic mode splits only when the longest item
// exceeds 1.5x the average work of a compute unit, into pieces of about that
// average, at least 512 keys on multiples of 256 for items with full tiles
// (smaller pieces measured slower: every split writes and re-reads its rows'
// fp32 partials).  Items with few query rows (single tokens of many grouped
// heads, too many rows for a decode item) have small partials and are memory
// bound: their average is taken per workgroup slot (compute units x prefill
// workgroups one compute unit holds), their floor shrinks with their rows
// (down to 128 keys) and pieces round to 128 keys (measured on 128 single
// tokens x 32 heads at d = 128: 24.5 us with 384-key pieces against 34.4 us
// with 768).  Boundaries sit on multiples of
// 64 keys so that no key tile is shared by two splits.
static void split_long_prefill_items(const PlanParams& p, Plan* out) {
  out->prefill_split_keys = 0;
  if (out->prefill.empty() || p.prefill_split_keys < 0) return;
  int64_t total = 0, longest = 0, max_rows = 0;
  const int group = p.num_q_heads / p.num_kv_heads;
  for (const auto& it : out->prefill) {
    const int64_t keys = it.kv_end - it.kv_begin;
    total += keys;
    longest = std::max(longest, keys);
    max_rows = std::max<int64_t>(max_rows, int64_t(it.q_count) * group);
  }
  const bool full_rows = 2 * max_rows > p.prefill_rows;
  int64_t piece = p.prefill_split_keys;
  if (piece == 0) {
    const int slots = p.num_cus * (full_rows ? 1 : std::max(1, p.prefill_wgs_per_cu));
    const int64_t avg = total / std::max(1, slots);
    if (2 * longest <= 3 * avg) return;
    piece = avg;
  }
  if (full_rows) {
    piece = std::max<int64_t>(512, (piece + 255) / 256 * 256);
  } else {
    const int64_t floor = std::max<int64_t>(128, 512 * max_rows / std::max(1, p.prefill_rows) / 128 * 128);
    piece = std::max<int64_t>(floor, (piece + 127) / 128 * 128);
  }
  if (2 * longest <= 3 * piece) return;
  out->prefill_split_keys = static_cast<int>(piece);
  const int slots = p.prefill_rows / 16;   // 16-row partial slots per split
  std::vector<rpa_work_item> items;
  items.reserve(out->prefill.size());
  for (const auto& it : out->prefill) {
    const int64_t keys = it.kv_end - it.kv_begin;
    const int64_t n = (2 * keys <= 3 * piece) ? 1 : (keys + piece / 2) / piece;   // round(keys / piece)
    if (n <= 1) {
      items.push_back(it);
      continue;
    }
    rpa_work_item base = it;
    base.split_group = static_cast<int32_t>(out->groups.size());
    base.num_splits = static_cast<int32_t>(n);
    base.partial_base = out->num_partials;
    out->num_partials += static_cast<int>(n) * slots;
    out->groups.push_back(base);
    int64_t lo = it.kv_begin;
    for (int64_t i = 0; i < n; ++i) {
      int64_t hi = it.kv_end;
      if (i + 1 < n) hi = (it.kv_begin + (keys * (i + 1)) / n + 63) / 64 * 64;
      rpa_work_item s = base;
      s.split_index = static_cast<int32_t>(i);
      s.self_append = i == 0 ? base.self_append : 0;
      s.kv_begin = static_cast<int32_t>(lo);
      s.kv_end = static_cast<int32_t>(hi);
      items.push_back(s);
      lo = hi;
    }
  }
  out->prefill.swap(items);
}

void build_plan(const PlanParams& p, const int32_t* cu, const int32_t* kv, int32_t num_seqs,
                int32_t window, Plan* out) {
  out->prefill.clear();
  out->decode.clear();
  out->decode2.clear();
  out->groups.clear();
  out->num_partials = 0;
  out->stage.clear();
  out->stage_table.clear();
  out->stage_pages = 0;
  out->visible_pairs = 0;
  out->total_q = num_seqs > 0 ? cu[num_seqs] : 0;

  const int group = p.num_q_heads / p.num_kv_heads;
  const int tile_tokens = std::max(1, p.prefill_rows / group);
  const int dec_tokens = decode_rows_limit(p) / group;  // 0 when G exceeds a decode item

  struct DecodeSeq {
    int32_t seq, q_start, q_count, pos0, kv_begin, kv_end;
    bool whole;        // the item holds every token of its sequence
    int32_t new_pos0;  // position of the sequence's first new token
  };
  std::vector<DecodeSeq> dec;

  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t q_len = cu[s + 1] - cu[s];
    const int32_t kv_len = kv[s];
    if (q_len == 0) continue;
    const int32_t pos_first = kv_len - q_len;
    for (int32_t r = 0; r < q_len; ++r) out->visible_pairs += visible_keys(pos_first + r, window);

    const bool fits_decode = dec_tokens > 0 && q_len <= dec_tokens;
    const bool use_decode = p.path_mode != 1 && fits_decode;
    if (use_decode) {
      dec.push_back({s, cu[s], q_len, pos_first, range_begin(pos_first, window), kv_len, true, pos_first});
      continue;
    }
    if (p.path_mode == 3 && dec_tokens > 0) {
      // every token through the decode kernel: consecutive chunks of
      // dec_tokens tokens, each with the key range its rows see
      for (int32_t t = 0; t < q_len; t += dec_tokens) {
        const int32_t count = std::min(dec_tokens, q_len - t);
        const int32_t pos0 = pos_first + t;
        dec.push_back({s, cu[s] + t, count, pos0, range_begin(pos0, window), pos0 + count, count == q_len,
                       pos_first});
      }
      continue;
    }
    for (int32_t g = 0; g < p.num_kv_heads; ++g) {
      for (int32_t t = 0; t < q_len; t += tile_tokens) {
        const int32_t count = std::min(tile_tokens, q_len - t);
        rpa_work_item it{};
        it.seq = s;
        it.kv_head = g;
        it.q_start = cu[s] + t;
        it.q_count = count;
        it.q_pos0 = pos_first + t;
        it.kv_begin = range_begin(it.q_pos0, window);
        it.kv_end = it.q_pos0 + count;  // last position + 1
        it.split_group = -1;
        it.split_index = 0;
        it.num_splits = 1;
        it.partial_base = 0;
        it.kind = 0;
        // bf16 cache: the tile's first split writes its tokens' new rows in an appending call
        it.self_append = p.kv8 ? 0 : 1;
        it.new_pos0 = pos_first;
        out->prefill.push_back(it);
      }
    }
  }

  // Every page that the prefill items of a sequence read (from the page of
  // their first key to the sequence's last page) gets a page of the bf16
  // staging pool (pool pages in sequence order), and the pool's page table
  // maps the sequence's pages to them.  A sequence's items are consecutive
  // here (before splitting and sorting).
  if (p.stage_prefill && !out->prefill.empty()) {
    out->stage_table.assign(static_cast<size_t>(num_seqs) * p.max_pages_per_seq, 0);
    for (size_t i = 0; i < out->prefill.size();) {
      const int32_t seq = out->prefill[i].seq;
      int32_t first_key = out->prefill[i].kv_begin;
      for (; i < out->prefill.size() && out->prefill[i].seq == seq; ++i)
        first_key = std::min(first_key, out->prefill[i].kv_begin);
      const int32_t n = (kv[seq] + p.page_size - 1) / p.page_size;
      for (int32_t lp = first_key / p.page_size; lp < n; ++lp) {
        out->stage.push_back(seq);
        out->stage.push_back(lp);
        out->stage.push_back(out->stage_pages);
        out->stage_table[static_cast<size_t>(seq) * p.max_pages_per_seq + lp] = out->stage_pages;
        ++out->stage_pages;
      }
    }
  }

  split_long_prefill_items(p, out);
  out->prefill_groups = static_cast<int32_t>(out->groups.size());

  // Longest first: the most expensive tiles start first so the tail is short.
  std::stable_sort(out->prefill.begin(), out->prefill.end(),
                   [](const rpa_work_item& a, const rpa_work_item& b) {
                     const int64_t ca = int64_t(a.kv_end - a.kv_begin) * a.q_count;
                     const int64_t cb = int64_t(b.kv_end - b.kv_begin) * b.q_count;
                     return ca > cb;
                   });
  interleave_for_chiplets(&out->prefill, p.num_cus, p.xcd_groups, p.xcd_run);

  // Decode split size: enough splits to give every compute unit a few
  // workgroups, in whole multiples of what one workgroup takes per step.
  const int64_t wg_keys = int64_t(p.decode_wave_keys) * p.decode_waves;
  int64_t split = p.decode_split_keys;
  if (split <= 0) {
    int64_t total = 0;
    for (const auto& d : dec) total += int64_t(d.kv_end - d.kv_begin) * p.num_kv_heads;
    const int64_t target = int64_t(2) * p.num_cus;
    split = (total + target - 1) / std::max<int64_t>(target, 1);
    split = (split + wg_keys - 1) / wg_keys * wg_keys;
    if (split < wg_keys) split = wg_keys;
  } else {
    split = (split + p.decode_wave_keys - 1) / p.decode_wave_keys * p.decode_wave_keys;
  }
  out->decode_split_keys = static_cast<int>(split);

  // Split boundaries: n = ceil(keys / split) pieces of about equal length, on
  // multiples of the keys one wave takes per step (so that no wave chunk is
  // read by two pieces), each at most `split` keys; where rounding would
  // break that bound, fixed pieces of `split` keys and a remainder.  Equal
  // pieces keep the split groups' pieces shorter than the longest unsplit
  // items, so that their merge overlaps the streaming of the others.
  std::vector<int64_t> bounds;
  auto split_bounds = [&](int64_t kv_begin, int64_t kv_end, int32_t n) {
    const int64_t keys = kv_end - kv_begin;
    const int64_t w = std::max(1, p.decode_wave_keys);
    bounds.assign(n + 1, kv_begin);
    bounds[n] = kv_end;
    bool ok = true;
    for (int32_t i = 1; i < n; ++i) {
      int64_t b = kv_begin + (keys * i + n / 2) / n;
      b = (b + w / 2) / w * w;
      bounds[i] = std::min(std::max(b, kv_begin), kv_end);
    }
    for (int32_t i = 0; i < n; ++i)
      ok = ok && bounds[i + 1] > bounds[i] && bounds[i + 1] - bounds[i] <= split;
    if (!ok)
      for (int32_t i = 1; i < n; ++i) bounds[i] = kv_begin + int64_t(i) * split;
  };

  for (const auto& d : dec) {
    const int64_t keys = d.kv_end - d.kv_begin;
    const int32_t n = static_cast<int32_t>(std::max<int64_t>(1, (keys + split - 1) / split));
    // items of more than 16 rows go to the two-block decode kernel (kind 2),
    // whose splits take two 16-row partial slots each
    const bool two = d.q_count * group > 16;
    std::vector<rpa_work_item>& dst = two ? out->decode2 : out->decode;
    for (int32_t g = 0; g < p.num_kv_heads; ++g) {
      rpa_work_item base{};
      base.seq = d.seq;
      base.kv_head = g;
      base.q_start = d.q_start;
      base.q_count = d.q_count;
      base.q_pos0 = d.pos0;
      base.kind = two ? 2 : 1;
      base.self_append = d.whole ? 1 : 0;
      base.new_pos0 = d.new_pos0;
      base.num_splits = n;
      if (n == 1) {
        base.kv_begin = d.kv_begin;
        base.kv_end = d.kv_end;
        base.split_group = -1;
        base.split_index = 0;
        base.partial_base = 0;
        dst.push_back(base);
        continue;
      }
      base.split_group = static_cast<int32_t>(out->groups.size());
      base.partial_base = out->num_partials;
      out->num_partials += n * (two ? 2 : 1);
      split_bounds(d.kv_begin, d.kv_end, n);
      for (int32_t i = 0; i < n; ++i) {
        rpa_work_item it = base;
        it.split_index = i;
        it.kv_begin = static_cast<int32_t>(bounds[i]);
        it.kv_end = static_cast<int32_t>(bounds[i + 1]);
        if (i == 0) {
          rpa_work_item grp = it;
          grp.kv_begin = d.kv_begin;
          grp.kv_end = d.kv_end;
          out->groups.push_back(grp);
        }
        dst.push_back(it);
      }
    }
  }
  auto longest_first = [](const rpa_work_item& a, const rpa_work_item& b) {
    return (a.kv_end - a.kv_begin) > (b.kv_end - b.kv_begin);
  };
  std::stable_sort(out->decode.begin(), out->decode.end(), longest_first);
  std::stable_sort(out->decode2.begin(), out->decode2.end(), longest_first);
  out->append_items = 0;
  out->prefill_writer_items = 0;
  for (const auto* list : {&out->prefill, &out->decode, &out->decode2})
    for (const auto& it : *list) out->append_items += (it.split_index == 0 && it.self_append == 0) ? 1 : 0;
  out->new_align = 1 << 30;
  for (const auto& it : out->prefill) {
    out->prefill_writer_items += it.self_append;
    if (it.new_pos0 > 0) out->new_align = std::min(out->new_align, it.new_pos0 & -it.new_pos0);
  }
}

}  // namespace rpa
