// Invariants of the fp8 staging list built by the host planner, on random
// ragged batches (run by tests/test_planner.py): every page that a prefill
// item reads (by the kernel's key clamp, including the first tile of a range
// that starts inside a tile) has a staged pool page that maps back to that
// (sequence, page);
// pool pages are numbered 0.. in list order; no staging without prefill
// items.  And the fields an appending call uses: every item's new_pos0 is
// its sequence's kv_len - q_len; with a bf16 cache each (token, KV head) of
// a sequence served by prefill items is written by exactly one of them
// (split 0 of the query tile holding it, self_append set), with an fp8
// cache by none (the copy kernel quantizes those rows).
// Exit status 0 when every check holds.
#include <algorithm>
#include <cstdio>
#include <random>
#include <string>
#include <vector>

#include "rpa_plan.h"

int main() {
  std::mt19937 rng(1);
  int bad = 0, planned = 0;
  for (int trial = 0; trial < 400; ++trial) {
    rpa::PlanParams p;
    const int group = 1 << (rng() % 6);
    p.num_kv_heads = 1 + rng() % 3;
    p.num_q_heads = group * p.num_kv_heads;
    p.head_dim = 256;
    p.page_size = std::vector<int>{16, 32, 64, 128}[rng() % 4];
    const int num_seqs = 1 + rng() % 20;
    p.max_num_seqs = num_seqs;
    p.prefill_rows = 256;
    p.stage_prefill = true;
    p.kv8 = rng() % 2 == 0;
    p.path_mode = rng() % 4;
    std::vector<int32_t> cu(num_seqs + 1, 0), kv(num_seqs);
    int max_pages = 1;
    for (int s = 0; s < num_seqs; ++s) {
      const int q = (rng() % 3 == 0) ? 1 + rng() % 300 : rng() % 2;
      const int k = q + rng() % 700;
      cu[s + 1] = cu[s] + q;
      kv[s] = k;
      max_pages = std::max(max_pages, (k + p.page_size - 1) / p.page_size);
    }
    p.max_pages_per_seq = max_pages;
    p.max_q_tokens = cu[num_seqs];
    const int window = (rng() % 2) * (1 + rng() % 200);
    std::string err;
    if (rpa::validate_metadata(p, cu.data(), kv.data(), num_seqs, window, &err) != RPA_OK) {
      std::printf("metadata rejected: %s\n", err.c_str());
      ++bad;
      continue;
    }
    rpa::Plan plan;
    rpa::build_plan(p, cu.data(), kv.data(), num_seqs, window, &plan);
    ++planned;
    // appending-call fields
    std::vector<int> writes(static_cast<size_t>(cu[num_seqs]) * p.num_kv_heads, 0);
    std::vector<char> prefill_seq(num_seqs, 0);
    for (const auto* list : {&plan.prefill, &plan.decode, &plan.decode2})
      for (const auto& it : *list) bad += it.new_pos0 != kv[it.seq] - (cu[it.seq + 1] - cu[it.seq]);
    for (const auto& it : plan.prefill) {
      prefill_seq[it.seq] = 1;
      const int want = (!p.kv8 && it.split_index == 0) ? 1 : 0;
      bad += it.self_append != want;
      if (it.self_append)
        for (int t = it.q_start; t < it.q_start + it.q_count; ++t)
          ++writes[static_cast<size_t>(t) * p.num_kv_heads + it.kv_head];
    }
    for (int s = 0; s < num_seqs; ++s)
      if (prefill_seq[s])
        for (int t = cu[s]; t < cu[s + 1]; ++t)
          for (int g = 0; g < p.num_kv_heads; ++g)
            bad += writes[static_cast<size_t>(t) * p.num_kv_heads + g] != (p.kv8 ? 0 : 1);
    // new_align: a power of two dividing every prefill sequence's first new
    // position, and the largest one (up to 2^30) that does
    {
      int writers = 0;
      for (const auto& it : plan.prefill) writers += it.self_append;
      bad += plan.prefill_writer_items != writers;
      const int a = plan.new_align;
      bad += a <= 0 || (a & (a - 1)) != 0 || a > (1 << 30);
      bool all_twice = a < (1 << 30);
      for (int s = 0; s < num_seqs; ++s)
        if (prefill_seq[s]) {
          const int n0 = kv[s] - (cu[s + 1] - cu[s]);
          bad += a > 0 && n0 % a != 0;
          all_twice = all_twice && n0 % (2 * a) == 0;
        }
      bad += all_twice;
    }
    if (plan.prefill.empty()) {
      bad += plan.stage_pages != 0;
      continue;
    }
    bad += static_cast<int>(plan.stage.size()) != 3 * plan.stage_pages;
    bad += plan.stage_table.size() != static_cast<size_t>(num_seqs) * max_pages;
    for (int b = 0; b < plan.stage_pages; ++b) {
      const int s = plan.stage[3 * b], lp = plan.stage[3 * b + 1], slot = plan.stage[3 * b + 2];
      const bool ok = s >= 0 && s < num_seqs && lp >= 0 && lp < (kv[s] + p.page_size - 1) / p.page_size &&
                      slot == b && plan.stage_table[static_cast<size_t>(s) * max_pages + lp] == slot;
      bad += !ok;
    }
    // The pages the prefill kernel reads for an item: its key tiles of BN
    // keys start at floor(kv_begin / BN) * BN, and every row of a tile reads
    // the key clamped into [max(tile start, kv_begin), min(tile end, kv_end))
    // -- so the first tile's rows below kv_begin read no page before
    // kv_begin's.  Each such page must be staged and map back to itself.
    for (const auto& it : plan.prefill) {
      const int bn = 32;   // key tile of the head size 256 kernel
      for (int k0 = it.kv_begin / bn * bn; k0 < it.kv_end; k0 += bn) {
        const int lo = std::max(k0, it.kv_begin), hi = std::min(k0 + bn, it.kv_end);
        for (int r = 0; r < bn; ++r) {
          const int key = std::min(std::max(k0 + r, lo), hi - 1);
          const int lp = key / p.page_size;
          const int slot = plan.stage_table[static_cast<size_t>(it.seq) * max_pages + lp];
          const bool ok = slot >= 0 && slot < plan.stage_pages && plan.stage[3 * slot] == it.seq &&
                          plan.stage[3 * slot + 1] == lp && lp >= it.kv_begin / p.page_size;
          bad += !ok;
        }
      }
    }
  }
  std::printf("plans %d, failed checks %d\n", planned, bad);
  return bad == 0 ? 0 : 1;
}
